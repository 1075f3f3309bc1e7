// Backward of block-sparse attention (gfx950, bf16 Q/K/V/O/dO).
//
// The pages name the backward as the missing half of the method and say it
// walks the block metadata transposed (flash-attention pull request 2224,
// review thread).  This is the gradient of the forward over the listed
// blocks, with the forward's LSE:
//   P = exp(scale*S - LSE), dV = P^T dO, dP = dO V^T, D = rowsum(dO * O),
//   dS = P * (dP - D), dQ = scale * dS K, dK = scale * dS^T Q.
// Three launches on the caller's stream:
//   1. bwd_rowdot_kernel: D per row (fp32 workspace).
//   2. bwd_dq_kernel: one workgroup per 128 (or 64) rows of a Q block, walking
//      the forward's lists in 64-key sub-tiles.  S^T and dP^T come from K and
//      V rows in LDS against Q and dO in registers; dQ^T accumulates K^T (the
//      K tile read transposed) times dS^T.  A lane owns one query row, as in
//      the forward, and dS feeds the last product straight from registers.
//   3. bwd_dkdv_kernel: one workgroup per 128 (or 64) keys of a KV block,
//      walking the KV-major lists (the Q blocks that list the KV block) of
//      every Q head of its KV head, in 64-row sub-tiles.  The roles swap: a
//      lane owns one key, K and V sit in registers, Q and dO tiles in LDS.
//      Summing the group's heads in one workgroup needs no atomics.
// Tiles move from HBM straight into LDS (global_load_lds) in a swizzled
// row-major layout that both the row reads and the transposing reads
// (ds_read_b64_tr_b16) take without bank conflicts; two LDS stages up to
// d = 128 (the next sub-tile streams in while the current one computes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "bsa_fwd_common.h"

// Row-dot workspace of the allocation-free entry point (bsa_bwd_noalloc):
// one copy per GPU, held until the process ends.  Host code never passes
// this name to a kernel (on the host it is a stand-in, not a device
// address); it uses the address bwd_noalloc_scratch looks up per device.
static __device__ __align__(256) float scratch[bsa::kBwdNoallocMaxRows];

namespace bsa {
namespace {

using namespace dev;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

// A dQ workgroup of NW waves owns 32*NW rows, a dK/dV workgroup of NQ waves
// 32*NQ keys: 4 when the block size is a multiple of 128, else 2.  The other
// side streams in sub-tiles of kBwdT positions.
constexpr int kBwdT = 64;

__device__ __forceinline__ uint32_t word4(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The positions [lo, hi] of a 64-position sub-tile that the element rule of
// a mask-list block keeps for this lane (the inner loops test them as bits,
// key_bits, instead of branching per element).  Keys (dQ: the lane owns
// sequence row `row`, the sub-tile holds keys k0 ..) or rows (dK/dV: the
// lane owns key `key`, the sub-tile holds rows r0 ..) of KV block j.
__device__ __forceinline__ void keys_kept(const BwdParams& p, const int32_t* kvv, int row, int k0,
                                          int j, int& lo, int& hi) {
  lo = 0;
  hi = kBwdT - 1;
  switch (p.mask_mod) {
    case kMaskCausal: hi = row - k0; break;
    case kMaskKvValid: hi = kvv[j] + j * p.block_kv - k0 - 1; break;
    case kMaskLocal:
      if (p.win_left >= 0) lo = row - p.win_left - k0;
      if (p.win_right >= 0) hi = row + p.win_right - k0;
      break;
    default: break;
  }
}

__device__ __forceinline__ void rows_kept(const BwdParams& p, const int32_t* kvv, int key, int r0,
                                          int j, int& lo, int& hi) {
  lo = 0;
  hi = kBwdT - 1;
  switch (p.mask_mod) {
    case kMaskCausal: lo = key - r0; break;
    case kMaskKvValid:
      if (key - j * p.block_kv >= kvv[j]) hi = -1;
      break;
    case kMaskLocal:
      if (p.win_right >= 0) lo = key - p.win_right - r0;
      if (p.win_left >= 0) hi = key + p.win_left - r0;
      break;
    default: break;
  }
}

// Backward tiles in LDS: 64 positions (keys, or query rows) x D bf16, rows
// unpadded: chunk c (16 bytes) of row r at slot r*DC + (c ^ swz(r)).  A tile
// is read as rows (ds_read_b128: the 16 lanes of a quarter-wave read one
// chunk of 16 consecutive rows) and transposed (ds_read_b64_tr_b16: half a
// wave reads 4 consecutive rows x 4 consecutive chunks).  swz maps both
// patterns onto 16 different 16-byte bank groups (the transposed reads at
// d = 192 pair up two to a group).  swz depends on r mod 16 only.
template <int D>
struct BTile {
  static constexpr int DC = D / 8;
  static constexpr int BYTES = kBwdT * DC * 16;
  __device__ __forceinline__ static int swz(int r) {
    return D == 64 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 3)
         : D == 96 ? (r >> 2) & 3
         : D == 192 ? (r >> 1) & 7
                    : 4 * (r & 3) + ((r >> 2) & 3);
  }
};

// One 16-byte global_load_lds per lane: the lane's 16 bytes at base + off go
// to LDS address lds_addr + 16 * lane.  The base is a scalar (SGPR) operand
// and the LDS address goes in M0.  The compiler's hazard checks do not see
// inside the asm, so its s_nop 4 provides the wait states the load needs
// after the instructions that set its operands (five after a VALU write of
// an SGPR it reads, e.g. a base restored with v_readlane).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "{m0}"(lds_addr)
               : "memory");
}

__device__ __forceinline__ uint2 read_tr(const unsigned char* lds, int byte_off) {
  lds_char* base = (lds_char*)(lds);  // generic -> LDS address space
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + byte_off));
  return __builtin_bit_cast(uint2, v);
}

// Rows 0 .. n-1 (1 <= n <= 64) of a [*, D] bf16 tensor (row stride ss
// elements, first row at base) into a BTile at LDS address lds, by the
// workgroup's first NS waves (wave ws of them).  Rows past n repeat row n-1:
// every product that reads them multiplies by a zero P or dS.  64*ss*2 must
// fit 31 bits (checked by the caller).
template <int D, int NS>
__device__ __forceinline__ void stage_tile(const __bf16* base, int64_t ss, int n, uint32_t lds,
                                           int ws, int lane) {
  constexpr int DC = D / 8, NI = DC;  // 1 KiB DMA blocks per tile (64 slots each)
  // the base is wave-uniform; say so, since it is an SGPR operand
  const uint64_t u = (uint64_t)(size_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  const void* ub = (const void*)(size_t)(((uint64_t)hi << 32) | lo);
  const int rs = (int)(ss * 2);
  // The lane's offsets are recomputed at every call (a few VALU) instead of
  // being hoisted as loop invariants: kept live across the kernel they
  // spilled, and each reload from scratch waits for every vector-memory op
  // in flight, these DMAs included, which serialized them.
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int m = 0; m < (NI + NS - 1) / NS; ++m) {
    const int ii = m * NS + ws;
    if (ii >= NI) break;
    const int slot = ii * 64 + ln;
    const int r = slot / DC, c = (slot % DC) ^ BTile<D>::swz(r);
    dma16(ub, (uint32_t)(min(r, n - 1) * rs + c * 16), lds + ii * 1024);
  }
}

// Largest b < B with cu[b] <= x (cu: B+1 nondecreasing prefix sums), i.e.
// the sequence of packed block x.  Wave-uniform.
__device__ __forceinline__ int seq_of(const int32_t* cu, int B, int x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// One sequence's view for a workgroup: token starts of its Q rows and keys,
// its lengths and block counts, the index of its valid counts.  Batched:
// sequence b of the batch (starts 0, lengths Sq and Sk).  Packed varlen:
// sequence b of the pack, found from the workgroup's global block id.
struct SeqView {
  int b;
  int tq0, tk0;  // token starts (varlen) or 0
  int Sq, Sk, M, N;
  int64_t slot0;  // varlen: list-slot offset of the sequence
  const int32_t* kvv;
};

template <bool VL>
__device__ __forceinline__ SeqView seq_view(const BwdParams& p, int b) {
  SeqView v;
  v.b = b;
  if constexpr (VL) {
    v.tq0 = p.cu_q[b];
    v.tk0 = p.cu_k[b];
    v.Sq = p.cu_q[b + 1] - v.tq0;
    v.Sk = p.cu_k[b + 1] - v.tk0;
    v.M = p.cu_m[b + 1] - p.cu_m[b];
    v.N = p.cu_n[b + 1] - p.cu_n[b];
    v.slot0 = p.boff[b];
    v.kvv = p.kv_valid ? p.kv_valid + (int64_t)b * p.kvv_ld : nullptr;
  } else {
    v.tq0 = 0;
    v.tk0 = 0;
    v.Sq = p.Sq;
    v.Sk = p.Sk;
    v.M = p.M;
    v.N = p.N;
    v.slot0 = 0;
    v.kvv = p.kv_valid;
  }
  return v;
}

// The sub-tiles of one walk, in order: for each list (mask, then full), for
// each listed block id, the block's positions [id*blen, min((id+1)*blen, S))
// in pieces of 64.  All state is wave-uniform.
// (Two named fields per list, not arrays: an array indexed by the run-time
// list number would live in scratch memory.)
struct SubWalk {
  const int32_t* idx0;
  const int32_t* idx1;
  int64_t istep0, istep1;
  int cnt0, cnt1;
  int nmax, blen, S;
  int list, e, id, pos, end;
  __device__ __forceinline__ bool start_block() {
    while (list < 2) {
      const int cnt = list == 0 ? cnt0 : cnt1;
      const int32_t* idx = list == 0 ? idx0 : idx1;
      const int64_t istep = list == 0 ? istep0 : istep1;
      while (e < cnt) {
        const int v = idx[(int64_t)e * istep];
        if (v >= 0 && v < nmax) {
          id = v;
          pos = v * blen;
          end = min((v + 1) * blen, S);
          return true;
        }
        ++e;
      }
      ++list;
      e = 0;
    }
    return false;
  }
  // first call: list = 0, e = 0 set by the caller, then first(); later next()
  __device__ __forceinline__ bool first() { return start_block(); }
  __device__ __forceinline__ bool next() {
    pos += kBwdT;
    if (pos < end) return true;
    ++e;
    return start_block();
  }
};

// B-operand fragments of one row (query row for dQ, key for dK/dV):
// frag[ks] = X[row][16*ks + 8*h32 .. +7], zero when the row is invalid.
template <int D>
__device__ __forceinline__ void row_frags(const __bf16* rowp, bool valid, int h32,
                                          uint4 (&frag)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    frag[ks] = valid ? *reinterpret_cast<const uint4*>(rowp + ks * 16 + h32 * 8)
                     : make_uint4(0, 0, 0, 0);
}

// A lane's transposing reads of a tile (the forward's V^T reads): two reads
// of 4 positions each give the A operand [32 head dims x 16 positions] of
// head-dim block db and position block ps.
template <int D>
struct TrGeo {
  int base[2], sw[2], c0, half8;
  __device__ __forceinline__ explicit TrGeo(int lane) {
    const int h32 = lane >> 5, vs = lane & 15, vg = lane >> 4;
    const int pos = 8 * h32 + (vs >> 2);
    const int vd = 16 * (vg & 1) + 4 * (((vs & 1) << 1) | ((vs >> 1) & 1));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      base[t] = (pos + 4 * t) * (D / 8) * 16;
      sw[t] = BTile<D>::swz(pos + 4 * t);  // swz(pos + 16 ps) = swz(pos)
    }
    c0 = vd >> 3;
    half8 = 8 * ((vd >> 2) & 1);
  }
  __device__ __forceinline__ uint4 op(const unsigned char* t, int ps, int db) const {
    const int po = ps * 16 * (D / 8) * 16;
    const uint2 x = read_tr(t, base[0] + po + ((c0 + 4 * db) ^ sw[0]) * 16 + half8);
    const uint2 y = read_tr(t, base[1] + po + ((c0 + 4 * db) ^ sw[1]) * 16 + half8);
    return make_uint4(x.x, x.y, y.x, y.y);
  }
};

// acc[db] += X^T (the tile read transposed: head dims x positions) times the
// operand of pk (positions x this lane's column), over the 64 positions.
// PRE: every operand read issued before the first product.
template <int D, bool PRE = false>
__device__ __forceinline__ void tr_product(const unsigned char* t, const TrGeo<D>& g,
                                           const uint32_t (&pk0)[8], const uint32_t (&pk1)[8],
                                           f32x16_t (&acc)[D / 32]) {
  if constexpr (PRE) {
    uint4 a[4][D / 32];
#pragma unroll
    for (int ps = 0; ps < 4; ++ps)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) a[ps][db] = g.op(t, ps, db);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const uint4 bop = p_operand(pk0, pk1, ps);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(a[ps][db], bop, acc[db]);
    }
  } else {
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const uint4 bop = p_operand(pk0, pk1, ps);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(g.op(t, ps, db), bop, acc[db]);
    }
  }
}

// tr_product with the reads of one position step (every head-dim block) at a
// time issued ahead of its MFMAs.
template <int D>
__device__ __forceinline__ void tr_product_steps(const unsigned char* t, const TrGeo<D>& g,
                                                 const uint32_t (&pk0)[8],
                                                 const uint32_t (&pk1)[8],
                                                 f32x16_t (&acc)[D / 32]) {
#pragma unroll
  for (int ps = 0; ps < 4; ++ps) {
    uint4 a[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) a[db] = g.op(t, ps, db);
    __builtin_amdgcn_sched_barrier(0);
    const uint4 bop = p_operand(pk0, pk1, ps);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(a[db], bop, acc[db]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc (rows of head_dim per lane, the forward's output layout) * mul -> bf16 row.
template <int DB>
__device__ __forceinline__ void store_row(__bf16* dst, int h32, const f32x16_t (&acc)[DB],
                                          float mul) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int r0 = 8 * half;
      *reinterpret_cast<uint4*>(dst + db * 32 + 16 * half + 8 * h32) =
          make_uint4(pack_bf16x2(acc[db][r0] * mul, acc[db][r0 + 1] * mul),
                     pack_bf16x2(acc[db][r0 + 2] * mul, acc[db][r0 + 3] * mul),
                     pack_bf16x2(acc[db][r0 + 4] * mul, acc[db][r0 + 5] * mul),
                     pack_bf16x2(acc[db][r0 + 6] * mul, acc[db][r0 + 7] * mul));
    }
}

// D[b,h,r] = sum_d dO * O (fp32).  16 lanes per row, each summing 16-byte
// chunks c = l16, l16 + 16, ... of both rows, so a row's loads coalesce;
// the lanes' sums are added with shuffles.  The summation order is fixed.
constexpr int kRowdotLanes = 16;

template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const BwdParams p) {
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / kRowdotLanes;
  const int l16 = threadIdx.x % kRowdotLanes;
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  const bool live = t < rows;
  const int64_t tt = live ? t : 0;
  const int r = (int)(tt % p.Sq);
  const int64_t bh = tt / p.Sq;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const __bf16* o = reinterpret_cast<const __bf16*>(p.o) + b * p.o_sb + (int64_t)r * p.o_ss + h * p.o_sh;
  const __bf16* g = reinterpret_cast<const __bf16*>(p.dout) + b * p.do_sb + (int64_t)r * p.do_ss + h * p.do_sh;
  float acc = 0.f;
  if (live) {
#pragma unroll
    for (int c = l16; c < D / 8; c += kRowdotLanes) {
      const uint4 a = *reinterpret_cast<const uint4*>(o + c * 8);
      const uint4 e = *reinterpret_cast<const uint4*>(g + c * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = word4(a, i), y = word4(e, i);
        acc = fmaf(__uint_as_float(x << 16), __uint_as_float(y << 16), acc);
        acc = fmaf(__uint_as_float(x & 0xffff0000u), __uint_as_float(y & 0xffff0000u), acc);
      }
    }
  }
#pragma unroll
  for (int m = kRowdotLanes / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
  if (live && l16 == 0) p.drow[t] = acc;
}

// log2-domain LSE for exp2(s*c - lse2); a row with no key (LSE = -inf) gives
// +inf, so every p of it is 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse == neg_inf() ? __builtin_inff() : lse * 1.4426950408889634f;  // log2(e)
}

// s_waitcnt vmcnt(0): this wave's vector-memory ops, DMA included, are done.
__device__ __forceinline__ void wait_vmem0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// PX: the proxy route (BwdParams, px_*): in a sub-tile of summary keys only
// the summaries the Q block takes count, each with its block's log2 c_n
// added to its exponent (one weight per sub-tile, taken off the LSE); kept
// keys are tested as bits in every sub-tile of this instance.
template <int D, int NW, bool VL, bool PX = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))  // two waves per SIMD up to d = 128
void bwd_dq_kernel(const BwdParams p) {
  constexpr int TW = NW * 32;
  constexpr int DS = D / 16, DB = D / 32;
  // LDS stages of (K, V) tiles: two for 4-wave workgroups up to d = 128; one
  // for 2-wave ones, whose two stages (64 KiB at d = 128) would leave room
  // for one wave per SIMD (one stage: two, and d128 64-row sweeps -4 %)
  constexpr int ST = D <= 128 && NW == 4 ? 2 : 1;
  using T = BTile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[ST * 2 * T::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h32 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qsub = cdiv(p.block_q, TW);
  int t = blockIdx.x;
  const int s = t % qsub;
  t /= qsub;
  // mrow: the list row (batched: Q block i; varlen: global Q block id)
  const int mrow = t % p.M;
  t /= p.M;
  const int h = VL ? t : t % p.H, hk = h / p.hrep;
  const SeqView sv0 = seq_view<VL>(p, VL ? seq_of(p.cu_m, p.B, mrow) : t / p.H);
  const int b = sv0.b;
  const int i = VL ? mrow - p.cu_m[b] : mrow;
  const int r0 = i * p.block_q + s * TW;
  const int rend = min((i + 1) * p.block_q, sv0.Sq);
  if (r0 >= rend) return;
  const int row = r0 + 32 * w + l32;  // sequence-local
  const bool rvalid = row < rend;

  // VL: batch strides are 0 and the token start moves the base
  const int64_t qtok = (int64_t)sv0.tq0 + row;
  const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sb + qtok * p.q_ss + h * p.q_sh;
  const __bf16* grow = reinterpret_cast<const __bf16*>(p.dout) + b * p.do_sb + qtok * p.do_ss + h * p.do_sh;
  uint4 qf[DS], gf[DS];
  row_frags<D>(qrow, rvalid, h32, qf);
  row_frags<D>(grow, rvalid, h32, gf);
  // LSE and row dots: [B,H,Sq], or [H,total_q] for varlen (Sq = total_q)
  const int64_t lrow = VL ? (int64_t)h * p.Sq + qtok : ((int64_t)b * p.H + h) * p.Sq + row;
  const float lse2 = rvalid ? lse2_of(p.lse[lrow]) : __builtin_inff();
  const float drow = rvalid ? p.drow[lrow] : 0.f;
  const __bf16* kb0 = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb +
                      (int64_t)sv0.tk0 * p.k_ss + hk * p.k_sh;
  const __bf16* vb0 = reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb +
                      (int64_t)sv0.tk0 * p.v_ss + hk * p.v_sh;

  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  const int arow = swap_b23(l32), asw = T::swz(arow);
  const TrGeo<D> tg(lane);

  SubWalk W{};
  for (int list = 0; list < 2; ++list) {
    const int32_t* cntp = list == 0 ? p.mcnt : p.fcnt;
    const int64_t* cs = list == 0 ? p.mc_s : p.fc_s;
    const int64_t* is = list == 0 ? p.mi_s : p.fi_s;
    const int c = cntp ? min(max(cntp[VL ? h * cs[1] + mrow * cs[2]
                                        : b * cs[0] + h * cs[1] + i * cs[2]], 0), sv0.N)
                       : 0;
    const int32_t* ip =
        cntp ? (list == 0 ? p.midx : p.fidx) +
                   (VL ? h * is[1] + (sv0.slot0 + (int64_t)i * sv0.N) * is[3]
                       : b * is[0] + h * is[1] + i * is[2])
             : nullptr;
    if (list == 0) {
      W.cnt0 = c; W.idx0 = ip; W.istep0 = is[3];
    } else {
      W.cnt1 = c; W.idx1 = ip; W.istep1 = is[3];
    }
  }
  W.nmax = sv0.N;
  W.blen = p.block_kv;
  W.S = sv0.Sk;
  const uint32_t lds0 = (uint32_t)(size_t)((lds_char*)smem);
  // K and V rows of the walk's current sub-tile into a stage
  auto issue = [&](int stage) {
    const int nk = min(kBwdT, W.end - W.pos);
    const uint32_t kl = lds0 + stage * 2 * T::BYTES;
    stage_tile<D, NW>(kb0 + (int64_t)W.pos * p.k_ss, p.k_ss, nk, kl, w, lane);
    stage_tile<D, NW>(vb0 + (int64_t)W.pos * p.v_ss, p.v_ss, nk, kl + T::BYTES, w, lane);
  };
  bool have = W.first();
  if (have) issue(0);
  wait_vmem0();
  __syncthreads();
  int st = 0;
  while (have) {
    const int list = W.list, j = W.id, k0 = W.pos, nk = min(kBwdT, W.end - W.pos);
    const bool more = W.next();
    if (ST == 2 && more) issue(st ^ 1);  // streams in while this sub-tile computes
    {
      const unsigned char* kt = smem + st * 2 * T::BYTES;
      const unsigned char* vt = kt + T::BYTES;
      // kept keys of this sub-tile for this lane's row
      int klo = 0, khi = kBwdT - 1;
      if (list == 0) keys_kept(p, sv0.kvv, row, k0, j, klo, khi);
      khi = min(khi, nk - 1);
      // the lane's kept keys as bits (kb0 / kb1: keys of each half, bit
      // 16*(reg >> 3) + (reg & 7) for accumulator reg; one bit test per
      // element is cheaper than the two compares of a range): from the key
      // range, or on the proxy route in a chunk of summaries from the Q
      // block's bit set, whose log-weight comes off the row's LSE
      uint32_t kb0, kb1;
      float l2e = lse2;
      if constexpr (!PX) {
        const uint64_t lm = key_bits(klo, khi) >> (8 * h32);
        kb0 = (uint32_t)lm;
        kb1 = (uint32_t)(lm >> 32);
      } else {
        uint64_t kb;
        if (j < p.px_n) {
          khi = min(khi, p.px_sk - k0 - 1);
          kb = khi >= 63 ? ~0ull : khi < 0 ? 0ull : (1ull << (khi + 1)) - 1;
        } else {
          const int n0 = k0 - p.px_k0;  // summary position of the sub-tile's key 0
          const uint64_t* wp = p.px_keep + ((int64_t)(b * p.H + h) * p.M + i) * p.px_w;
          const int wi = n0 >> 6, sh = n0 & 63;
          const uint64_t lo = wi < p.px_w ? wp[wi] : 0ull;
          const uint64_t hi = (sh != 0 && wi + 1 < p.px_w) ? wp[wi + 1] : 0ull;
          kb = (lo >> sh) | (sh != 0 ? hi << (64 - sh) : 0ull);
          if (khi < 63) kb &= khi < 0 ? 0ull : (1ull << (khi + 1)) - 1;
          l2e = lse2 - (j == p.px_gl ? p.px_lwl : p.px_lw);
        }
        const uint64_t lm = kb >> (8 * h32);
        kb0 = (uint32_t)lm;
        kb1 = (uint32_t)(lm >> 32);
      }
      // per half (keys 32*hf ..): S^T and dP^T, then dS packed for the last
      // product; one half at a time keeps the registers of the other free
      uint32_t pk[2][8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x16_t sa, da;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sa[r] = 0.f;
          da[r] = 0.f;
        }
        const unsigned char* kr = kt + (arow + 32 * hf) * (D / 8) * 16;
        const unsigned char* vr = vt + (arow + 32 * hf) * (D / 8) * 16;
        if constexpr (D > 128) {
          // one wave per SIMD: the reads of 4 k-steps at a time ahead of their
          // MFMAs
#pragma unroll
          for (int k0 = 0; k0 < DS; k0 += 4) {
            uint4 ka[4], va[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int c = ((2 * (k0 + u) + h32) ^ asw) * 16;
              ka[u] = *reinterpret_cast<const uint4*>(kr + c);
              va[u] = *reinterpret_cast<const uint4*>(vr + c);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              sa = mfma32(ka[u], qf[k0 + u], sa);  // S^T
              da = mfma32(va[u], gf[k0 + u], da);  // dP^T
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < DS; ++ks) {
            const int c = ((2 * ks + h32) ^ asw) * 16;
            sa = mfma32(*reinterpret_cast<const uint4*>(kr + c), qf[ks], sa);  // S^T
            da = mfma32(*reinterpret_cast<const uint4*>(vr + c), gf[ks], da);  // dP^T
          }
        }
        const uint32_t kbh = hf == 0 ? kb0 : kb1;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          float v[2];
#pragma unroll
          for (int y = 0; y < 2; ++y) {
            const int reg = 2 * x + y;
            const bool keep = ((kbh >> (16 * (reg >> 3) + (reg & 7))) & 1u) != 0;
            const float pr = keep ? __builtin_amdgcn_exp2f(fmaf(sa[reg], p.c, -l2e)) : 0.f;
            v[y] = pr * (da[reg] - drow);
          }
          pk[hf][x] = pack_bf16x2(v[0], v[1]);
        }
      }
      if constexpr (D > 128)
        tr_product_steps<D>(kt, tg, pk[0], pk[1], acc);  // dQ^T += K^T dS^T
      else
        tr_product<D>(kt, tg, pk[0], pk[1], acc);
    }
    if (ST == 1) {
      __syncthreads();  // every wave is done with the stage
      if (more) issue(0);
    }
    wait_vmem0();
    __syncthreads();  // the next sub-tile has landed
    st = ST == 2 ? st ^ 1 : 0;
    have = more;
  }
  if (rvalid) {
    __bf16* dst = reinterpret_cast<__bf16*>(p.dq) + b * p.dq_sb + qtok * p.dq_ss + h * p.dq_sh;
    store_row<DB>(dst, h32, acc, p.scale);
  }
}

// NQ waves own 32 keys each (NQ*32 keys per workgroup); each computes P,
// dV, dP, dS and dK for its keys.  (Two groups of waves, one for dV and one
// for dK, each holding one accumulator at two waves per SIMD, measured
// slower at d = 128: 1.03 against 0.56 ms on the d128 sweep, the registers
// of the shared path spilled.)  The waves stage the Q and dO tiles and the
// rows' LSE and row dots.
// MODE: 0 computes dV and dK; 1 dV only; 2 dK only.  At d = 256 the two
// accumulators, K and V fragments and the products' operands need more than
// the 512 registers of a wave, so dV and dK run as two launches (S computed
// in both) instead of one that spills.
// PX: the proxy route (BwdParams, px_*): a workgroup of summary keys keeps,
// per Q block, the rows of the Q blocks whose bit set holds its lane's
// summary, takes its chunk's log2 c_n off the rows' staged LSE (adding it to
// the exponent) and writes the summaries' gradients (dV over c_n);
// workgroups of keys stop at px_sk.
template <int D, int NQ, bool VL, int MODE, bool PX = false>
__global__ __launch_bounds__(NQ * 64)
__attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1)))
void bwd_dkdv_kernel(const BwdParams p) {
  constexpr bool DO_DV = MODE != 2, DO_DK = MODE != 1;
  // Up to d = 128 each product's LDS operand reads are all issued before its
  // first MFMA (a scheduling barrier keeps them there): left to itself the
  // compiler put each read just ahead of its MFMA with a wait between, and
  // with one wave per SIMD nothing hid that latency (d128 sweep backward
  // 0.465 -> 0.424 ms).  Beyond d = 128 all of them would spill, and the
  // reads go 4 k-steps (S, dP) or one position step (dV, dK) ahead (d192 /
  // d256 sweep backward -8 / -6.5 %).
  constexpr bool PRE = D <= 128;
  constexpr int TW = NQ * 32;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int ST = D <= 128 ? 2 : 1;  // LDS stages of (Q, dO) tiles
  using T = BTile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[ST * 2 * T::BYTES];
  __shared__ __attribute__((aligned(16))) float lse2s[ST][kBwdT];
  __shared__ __attribute__((aligned(16))) float drows[ST][kBwdT];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h32 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w % NQ;
  const int ksub = cdiv(p.block_kv, TW);
  int t = blockIdx.x;
  const int s = t % ksub;
  t /= ksub;
  if (p.kv_order) t = p.kv_order[t];  // longest lists first
  // nrow: the KV-major list row (batched: KV block j; varlen: global KV block id)
  const int nrow = t % p.N;
  t /= p.N;
  const int Hkv = p.H / p.hrep;
  const int hk = VL ? t : t % Hkv;
  const SeqView sv0 = seq_view<VL>(p, VL ? seq_of(p.cu_n, p.B, nrow) : t / Hkv);
  const int b = sv0.b;
  const int j = VL ? nrow - p.cu_n[b] : nrow;
  const int k0 = j * p.block_kv + s * TW;
  int kend = min((j + 1) * p.block_kv, sv0.Sk);
  bool summ = false;  // proxy route: a workgroup of summary keys
  if constexpr (PX) {
    if (j < p.px_n)
      kend = min(kend, p.px_sk);
    else
      summ = true;
  }
  if (k0 >= kend) return;
  const int key = k0 + 32 * wq + l32;  // sequence-local
  bool kvalid = key < kend;
  int pu = 0, pn = 0;  // summary position of this lane's key, and its block
  float lwk = 0.f;     // the workgroup's log2 c_n, taken off the staged LSE
  if constexpr (PX) {
    if (summ) {
      pu = key - p.px_k0;
      const bool last = j == p.px_gl;  // a chunk of its own: position = its first key
      pn = last ? p.px_n - 1 : pu;
      kvalid = kvalid && (last ? key == j * p.block_kv : pu < p.px_nreg);
      lwk = last ? p.px_lwl : p.px_lw;
    }
  }

  const int64_t ktok = (int64_t)sv0.tk0 + key;
  const __bf16* krow = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + ktok * p.k_ss + hk * p.k_sh;
  const __bf16* vrow = reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + ktok * p.v_ss + hk * p.v_sh;
  uint4 kf[DS], vf[DS];
  row_frags<D>(krow, kvalid, h32, kf);
  if (DO_DK) row_frags<D>(vrow, kvalid, h32, vf);

  // where this lane's dK and dV rows go (set before the walk, so the walk
  // keeps two addresses live rather than the tensors' bases and strides)
  __bf16* kdst = reinterpret_cast<__bf16*>(p.dk) + b * p.dk_sb + ktok * p.dk_ss + hk * p.dk_sh;
  __bf16* vdst = reinterpret_cast<__bf16*>(p.dv) + b * p.dv_sb + ktok * p.dv_ss + hk * p.dv_sh;
  float vmul = 1.f;
  if constexpr (PX) {
    if (summ) {  // the summaries' gradients: d(mean key), d(summed value) = dV / c_n
      kdst = reinterpret_cast<__bf16*>(p.px_dks) + b * p.px_dks_sb + (int64_t)pn * p.px_dks_sn +
             hk * p.px_dks_sh;
      vdst = reinterpret_cast<__bf16*>(p.px_dvs) + b * p.px_dvs_sb + (int64_t)pn * p.px_dvs_sn +
             hk * p.px_dvs_sh;
      vmul = 1.f / (float)(j == p.px_gl ? p.px_cl : p.block_kv);
    }
  }

  f32x16_t dv[DB], dk[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[db][r] = 0.f;
      dk[db][r] = 0.f;
    }
  const int arow = swap_b23(l32), asw = T::swz(arow);
  const TrGeo<D> tg(lane);
  const uint32_t lds0 = (uint32_t)(size_t)((lds_char*)smem);

  int st = 0;
  for (int h = hk * p.hrep; h < (hk + 1) * p.hrep; ++h) {
    const __bf16* qb0 = reinterpret_cast<const __bf16*>(p.q) + b * p.q_sb +
                        (int64_t)sv0.tq0 * p.q_ss + h * p.q_sh;
    const __bf16* gb0 = reinterpret_cast<const __bf16*>(p.dout) + b * p.do_sb +
                        (int64_t)sv0.tq0 * p.do_ss + h * p.do_sh;
    // row r of the sequence at lbase + r in the LSE and row dots
    const int64_t lbase = VL ? (int64_t)h * p.Sq + sv0.tq0 : ((int64_t)b * p.H + h) * p.Sq;
    SubWalk W{};
    for (int list = 0; list < 2; ++list) {
      const int32_t* cntp = list == 0 ? p.tmcnt : p.tfcnt;
      const int64_t* cs = list == 0 ? p.tmc_s : p.tfc_s;
      const int64_t* is = list == 0 ? p.tmi_s : p.tfi_s;
      const int c = cntp ? min(max(cntp[VL ? h * cs[1] + nrow * cs[2]
                                          : b * cs[0] + h * cs[1] + j * cs[2]], 0), sv0.M)
                         : 0;
      const int32_t* ip =
          cntp ? (list == 0 ? p.tmidx : p.tfidx) +
                     (VL ? h * is[1] + (sv0.slot0 + (int64_t)j * sv0.M) * is[3]
                         : b * is[0] + h * is[1] + j * is[2])
               : nullptr;
      if (list == 0) {
        W.cnt0 = c; W.idx0 = ip; W.istep0 = is[3];
      } else {
        W.cnt1 = c; W.idx1 = ip; W.istep1 = is[3];
      }
    }
    W.nmax = sv0.M;
    W.blen = p.block_q;
    W.S = sv0.Sq;
    float l2n = 0.f, drn = 0.f;  // wave 0: its lane's row of the staged sub-tile
    // proxy route: whether the staged (kwn) and the current (kwc) sub-tile's
    // Q block takes this lane's summary; the lane's word of Q block 0 (the
    // next Q block's is px_w words on)
    uint32_t kwn = 1, kwc = 1;
    const uint64_t* kwrow = nullptr;
    if constexpr (PX) {
      if (summ && kvalid)
        kwrow = p.px_keep + ((int64_t)(b * p.H + h) * p.M) * p.px_w + (pu >> 6);
    }
    // Q and dO rows (and the rows' LSE and row dots) of the walk's current
    // sub-tile into a stage
    auto issue = [&](int stage) {
      const int nr = min(kBwdT, W.end - W.pos), r0 = W.pos;
      const uint32_t ql = lds0 + stage * 2 * T::BYTES;
      stage_tile<D, NQ>(qb0 + (int64_t)r0 * p.q_ss, p.q_ss, nr, ql, w, lane);
      stage_tile<D, NQ>(gb0 + (int64_t)r0 * p.do_ss, p.do_ss, nr, ql + T::BYTES, w, lane);
      if (w == 0) {
        l2n = lane < nr ? lse2_of(p.lse[lbase + r0 + lane]) - lwk : __builtin_inff();
        drn = lane < nr ? p.drow[lbase + r0 + lane] : 0.f;
      }
      if constexpr (PX) {
        if (summ)
          kwn = kwrow ? (uint32_t)(kwrow[(int64_t)W.id * p.px_w] >> (pu & 63)) & 1u : 0u;
      }
    };
    auto put_rows = [&](int stage) {
      if (w == 0) {
        lse2s[stage][lane] = l2n;
        drows[stage][lane] = drn;
      }
    };
    // The stage about to be filled was last read before the previous
    // sub-tile's closing barrier.
    bool have = W.first();
    if (have) {
      issue(st);
      put_rows(st);
    }
    kwc = kwn;
    wait_vmem0();
    __syncthreads();
    while (have) {
      const int list = W.list, r0 = W.pos, nr = min(kBwdT, W.end - W.pos);
      const bool more = W.next();
      if (ST == 2 && more) issue(st ^ 1);  // streams in while this sub-tile computes
      {
        const unsigned char* qt = smem + st * 2 * T::BYTES;
        const unsigned char* gt = qt + T::BYTES;
        // kept rows of this sub-tile for this lane's key
        int rlo = 0, rhi = kBwdT - 1;
        if (list == 0) rows_kept(p, sv0.kvv, key, r0, j, rlo, rhi);
        rhi = kvalid && kwc ? min(rhi, nr - 1) : -1;
        // as bits of the lane's rows (rb0 / rb1: rows of each half, bit
        // 16*(reg >> 3) + (reg & 7) for accumulator reg)
        const uint64_t rlm = key_bits(rlo, rhi) >> (8 * h32);
        const uint32_t rb0 = (uint32_t)rlm, rb1 = (uint32_t)(rlm >> 32);
        // per half (rows 32*hf ..): S and dP, then P and dS packed for the
        // last products; one half at a time keeps the registers of the other
        // free
        uint32_t pk[2][8], pks[2][8];  // P, dS
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          f32x16_t sa, da;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sa[r] = 0.f;
            da[r] = 0.f;
          }
          const unsigned char* qr = qt + (arow + 32 * hf) * (D / 8) * 16;
          const unsigned char* gr = gt + (arow + 32 * hf) * (D / 8) * 16;
          // this lane's rows of the half, 32 hf + 16 r8 + 8 h32 + 0..7 (r8 = 0,
          // 1): their LSE and row dots read as vectors ahead of the products
          // (element by element, each read's latency was exposed)
          float4 l4[4], d4[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int r = 32 * hf + 16 * (q4 >> 1) + 8 * h32 + 4 * (q4 & 1);
            l4[q4] = *reinterpret_cast<const float4*>(&lse2s[st][r]);
            d4[q4] = *reinterpret_cast<const float4*>(&drows[st][r]);
          }
          if constexpr (PRE) {
            // every operand read issued before the first product
            uint4 qa[DS], ga[DS];
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) {
              const int c = ((2 * ks + h32) ^ asw) * 16;
              qa[ks] = *reinterpret_cast<const uint4*>(qr + c);
              if (DO_DK) ga[ks] = *reinterpret_cast<const uint4*>(gr + c);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < DS; ++ks) {
              sa = mfma32(qa[ks], kf[ks], sa);               // S
              if (DO_DK) da = mfma32(ga[ks], vf[ks], da);  // dP
            }
          } else {
            // d > 128: the reads of 4 k-steps at a time ahead of their MFMAs
#pragma unroll
            for (int k0 = 0; k0 < DS; k0 += 4) {
              uint4 qa[4], ga[4];
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const int c = ((2 * (k0 + u) + h32) ^ asw) * 16;
                qa[u] = *reinterpret_cast<const uint4*>(qr + c);
                if (DO_DK) ga[u] = *reinterpret_cast<const uint4*>(gr + c);
              }
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                sa = mfma32(qa[u], kf[k0 + u], sa);               // S
                if (DO_DK) da = mfma32(ga[u], vf[k0 + u], da);  // dP
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            float v[2], w2[2];
#pragma unroll
            for (int y = 0; y < 2; ++y) {
              const int reg = 2 * x + y;
              const uint32_t rbh = hf == 0 ? rb0 : rb1;
              const bool keep = ((rbh >> (16 * (reg >> 3) + (reg & 7))) & 1u) != 0;
              const int q4 = 2 * (reg >> 3) + ((reg & 7) >> 2), e4 = reg & 3;
              const float l2 = e4 == 0 ? l4[q4].x : e4 == 1 ? l4[q4].y : e4 == 2 ? l4[q4].z : l4[q4].w;
              const float dr = e4 == 0 ? d4[q4].x : e4 == 1 ? d4[q4].y : e4 == 2 ? d4[q4].z : d4[q4].w;
              const float pr = keep ? __builtin_amdgcn_exp2f(fmaf(sa[reg], p.c, -l2)) : 0.f;
              v[y] = pr;
              w2[y] = DO_DK ? pr * (da[reg] - dr) : 0.f;
            }
            if (DO_DV) pk[hf][x] = pack_bf16x2(v[0], v[1]);
            if (DO_DK) pks[hf][x] = pack_bf16x2(w2[0], w2[1]);
          }
        }
        if constexpr (PRE) {
          if (DO_DV) tr_product<D, true>(gt, tg, pk[0], pk[1], dv);    // dV^T += dO^T P
          if (DO_DK) tr_product<D, true>(qt, tg, pks[0], pks[1], dk);  // dK^T += Q^T dS
        } else {
          if (DO_DV) tr_product_steps<D>(gt, tg, pk[0], pk[1], dv);
          if (DO_DK) tr_product_steps<D>(qt, tg, pks[0], pks[1], dk);
        }
      }
      if (ST == 2 && more) put_rows(st ^ 1);
      if (ST == 1) {
        __syncthreads();  // every wave is done with the stage
        if (more) {
          issue(0);
          put_rows(0);
        }
      }
      wait_vmem0();
      __syncthreads();  // the next sub-tile has landed
      st = ST == 2 ? st ^ 1 : 0;
      kwc = kwn;
      have = more;
    }
  }

  if (kvalid) {
    if (DO_DK) store_row<DB>(kdst, h32, dk, p.scale);
    if (DO_DV) store_row<DB>(vdst, h32, dv, vmul);
  }
}

// The dK/dV workgroups' work varies with their KV-major list lengths (the
// number of Q blocks that list the KV block, over the KV head's Q heads);
// started in index order, a long one can start last and set the kernel's
// end.  One workgroup counting-sorts the n rows by decreasing length into
// `order` (buckets of one length each up to 1023, longer ones together;
// order inside a bucket is arbitrary and does not change any result).
constexpr int kOrderBuckets = 1024;

template <bool VL>
__global__ __launch_bounds__(kOrderBuckets) void bwd_kv_order_kernel(const BwdParams p, int n) {
  __shared__ int hist[kOrderBuckets];
  const int tid = threadIdx.x;
  const int Hkv = p.H / p.hrep;
  auto bucket = [&](int t) {  // kOrderBuckets - 1 - min(length, kOrderBuckets - 1)
    const int nrow = t % p.N, rest = t / p.N;
    const int hk = VL ? rest : rest % Hkv, b = VL ? 0 : rest / Hkv;
    int len = 0;
    for (int h = hk * p.hrep; h < (hk + 1) * p.hrep; ++h) {
      if (p.tmcnt)
        len += max(p.tmcnt[VL ? h * p.tmc_s[1] + nrow * p.tmc_s[2]
                              : b * p.tmc_s[0] + h * p.tmc_s[1] + nrow * p.tmc_s[2]], 0);
      if (p.tfcnt)
        len += max(p.tfcnt[VL ? h * p.tfc_s[1] + nrow * p.tfc_s[2]
                              : b * p.tfc_s[0] + h * p.tfc_s[1] + nrow * p.tfc_s[2]], 0);
    }
    return kOrderBuckets - 1 - min(len, kOrderBuckets - 1);
  };
  hist[tid] = 0;
  __syncthreads();
  for (int t = tid; t < n; t += kOrderBuckets) atomicAdd(&hist[bucket(t)], 1);
  __syncthreads();
  // exclusive prefix sum over the buckets (one per thread)
  const int mine = hist[tid];
  int incl = mine;
  for (int o = 1; o < kOrderBuckets; o <<= 1) {
    __syncthreads();
    const int add = tid >= o ? hist[tid - o] : 0;
    __syncthreads();
    incl += add;
    hist[tid] = incl;
  }
  __syncthreads();
  hist[tid] = incl - mine;
  __syncthreads();
  for (int t = tid; t < n; t += kOrderBuckets) p.kv_order[atomicAdd(&hist[bucket(t)], 1)] = t;
}

template <int D, bool VL, bool PX = false>
hipError_t launch_bwd_dv(const BwdParams& p, hipStream_t st) {
  // varlen: the row dots run over [H, total_q] as one sequence of Sq rows
  const int64_t rows = (VL ? 1 : (int64_t)p.B) * p.H * p.Sq;
  if (rows > 0) {
    BwdParams pr = p;
    if (VL) pr.B = 1;
    const int64_t per = 256 / kRowdotLanes;
    hipLaunchKernelGGL(bwd_rowdot_kernel<D>, dim3((unsigned)((rows + per - 1) / per)), dim3(256),
                       0, st, pr);
  }
  // batched: B*H*M Q-block rows and B*H_kv*N KV-block rows; varlen: the
  // M and N totals over the sequences carry the batch
  const int64_t nb = VL ? 1 : p.B;
  const int nwq = p.block_q % 128 == 0 ? 4 : 2, nqk = p.block_kv % 128 == 0 ? 4 : 2;
  const int64_t gq = nb * p.H * p.M * ((p.block_q + 32 * nwq - 1) / (32 * nwq));
  const int64_t gk = nb * (p.H / p.hrep) * p.N * ((p.block_kv + 32 * nqk - 1) / (32 * nqk));
  const int kthreads = nqk * 64;
  if (gq > 0) {
    if (nwq == 4)
      hipLaunchKernelGGL((bwd_dq_kernel<D, 4, VL, PX>), dim3((unsigned)gq), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, 2, VL, PX>), dim3((unsigned)gq), dim3(128), 0, st, p);
  }
  if (gk > 0 && p.kv_order) {
    const int64_t items = nb * (p.H / p.hrep) * p.N;
    hipLaunchKernelGGL(bwd_kv_order_kernel<VL>, dim3(1), dim3(kOrderBuckets), 0, st, p,
                       (int)items);
  }
  auto dkdv = [&](auto mode) {
    constexpr int M = decltype(mode)::value;
    if (nqk == 4)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, 4, VL, M, PX>), dim3((unsigned)gk), dim3(kthreads),
                         0, st, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, 2, VL, M, PX>), dim3((unsigned)gk), dim3(kthreads),
                         0, st, p);
  };
  if (gk > 0) {
    if constexpr (D >= 256) {
      dkdv(std::integral_constant<int, 1>{});
      dkdv(std::integral_constant<int, 2>{});
    } else {
      dkdv(std::integral_constant<int, 0>{});
    }
  }
  return hipGetLastError();
}

// fp32 <-> bf16 staging of the fp32 backward (HBM-bound elementwise).  A
// thread moves 8 consecutive head_dim elements of one (b, s, h) row: two
// 16-byte fp32 accesses and one 16-byte bf16 access, consecutive threads on
// consecutive chunks of a row.  The bf16 side is contiguous [B,S,H,D]; the
// fp32 side has element strides {sb, ss, sh} and a unit head_dim stride.
// fp32 -> bf16 rounds to nearest even (as the fp32 forward does at load).
__global__ __launch_bounds__(256) void cast_f32_bf16_kernel(const float* __restrict__ src,
                                                             int64_t sb, int64_t ss, int64_t sh,
                                                             int32_t S, int32_t H, int32_t D,
                                                             int64_t chunks,
                                                             __bf16* __restrict__ dst) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int cpr = D / 8;
  const int64_t row = c / cpr;
  const int d0 = (int)(c % cpr) * 8;
  const int h = (int)(row % H);
  const int64_t bs = row / H;
  const int64_t s = bs % S, b = bs / S;
  const float* a = src + b * sb + s * ss + (int64_t)h * sh + d0;
  const float4 x = *reinterpret_cast<const float4*>(a);
  const float4 y = *reinterpret_cast<const float4*>(a + 4);
  *reinterpret_cast<uint4*>(dst + row * D + d0) =
      make_uint4(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w), pack_bf16x2(y.x, y.y),
                 pack_bf16x2(y.z, y.w));
}

__global__ __launch_bounds__(256) void cast_bf16_f32_kernel(const __bf16* __restrict__ src,
                                                             int64_t sb, int64_t ss, int64_t sh,
                                                             int32_t S, int32_t H, int32_t D,
                                                             int64_t chunks,
                                                             float* __restrict__ dst) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int cpr = D / 8;
  const int64_t row = c / cpr;
  const int d0 = (int)(c % cpr) * 8;
  const int h = (int)(row % H);
  const int64_t bs = row / H;
  const int64_t s = bs % S, b = bs / S;
  const uint4 v = *reinterpret_cast<const uint4*>(src + row * D + d0);
  auto lo = [](uint32_t u) { return __uint_as_float(u << 16); };
  auto hi = [](uint32_t u) { return __uint_as_float(u & 0xffff0000u); };
  float* a = dst + b * sb + s * ss + (int64_t)h * sh + d0;
  *reinterpret_cast<float4*>(a) = make_float4(lo(v.x), hi(v.x), lo(v.y), hi(v.y));
  *reinterpret_cast<float4*>(a + 4) = make_float4(lo(v.z), hi(v.z), lo(v.w), hi(v.w));
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t st) {
  if (p.px_keep) return launch_bwd_dv<D, false, true>(p, st);  // the proxy route (batched)
  return p.varlen ? launch_bwd_dv<D, true>(p, st) : launch_bwd_dv<D, false>(p, st);
}

}  // namespace

hipError_t bwd_noalloc_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<float*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {  // once per device, with that device current
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<float*>(a);
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_cast_f32_bf16(const float* src, const int64_t str[3], int32_t B, int32_t S,
                                int32_t H, int32_t D, uint16_t* dst, hipStream_t st) {
  const int64_t chunks = (int64_t)B * S * H * (D / 8);
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(cast_f32_bf16_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                     st, src, str[0], str[1], str[2], S, H, D, chunks,
                     reinterpret_cast<__bf16*>(dst));
  return hipGetLastError();
}

hipError_t launch_cast_bf16_f32(const uint16_t* src, const int64_t str[3], int32_t B, int32_t S,
                                int32_t H, int32_t D, float* dst, hipStream_t st) {
  const int64_t chunks = (int64_t)B * S * H * (D / 8);
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(cast_bf16_f32_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                     st, reinterpret_cast<const __bf16*>(src), str[0], str[1], str[2], S, H, D,
                     chunks, dst);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_bwd_d<64>(p, s);
    case 96: return launch_bwd_d<96>(p, s);
    case 128: return launch_bwd_d<128>(p, s);
    case 192: return launch_bwd_d<192>(p, s);
    case 256: return launch_bwd_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bsa
