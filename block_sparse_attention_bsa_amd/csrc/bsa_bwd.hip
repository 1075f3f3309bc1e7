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
//   2. bwd_dq_kernel: one workgroup per 128 (or 64) rows of a Q block, walking the
//      forward's lists in 64-key sub-tiles.  S and dP^T come from K and V
//      rows in LDS against Q and dO in registers; dQ accumulates dS times K
//      read transposed from LDS.  The layouts are those of the forward: a lane
//      owns one query row, P and dS feed the last product straight from
//      registers.
//   3. bwd_dkdv_kernel: one workgroup per 128 (or 64) keys of a KV block, walking the
//      KV-major lists (the Q blocks that list the KV block) of every Q head of
//      its KV head, in 64-row sub-tiles.  The roles swap: a lane owns one key,
//      K and V sit in registers, Q and dO rows (and their transposes) in LDS.
//      Summing the group's heads in one workgroup needs no atomics.
// Each sub-tile is loaded, converted and transposed through registers by all
// threads, then computed; one LDS stage.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "bsa_fwd_common.h"

// Row-dot workspace of the allocation-free entry point (bsa_bwd_noalloc):
// one copy per GPU, held until the process ends.  Host code never passes
// this name to a kernel (on the host it is a stand-in, not a device
// address); it uses the address bwd_noalloc_scratch looks up per device.
static __device__ __align__(256) float scratch[bsa::kBwdNoallocMaxRows];

namespace bsa {
namespace {

using namespace dev;

// A workgroup of NW waves owns 32*NW rows (dQ) or keys (dK, dV): NW = 4 when
// the block size is a multiple of 128, else 2.  The other side streams in
// sub-tiles of kBwdT positions.
constexpr int kBwdT = 64;

__device__ __forceinline__ uint32_t word4(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Element rule of a mask-list block (row and key are sequence positions;
// kib is the key's offset inside its KV block j; kvv the sequence's
// valid counts).
__device__ __forceinline__ bool keep_elem(const BwdParams& p, const int32_t* kvv, int row, int key,
                                          int j, int kib) {
  switch (p.mask_mod) {
    case kMaskCausal: return key <= row;
    case kMaskKvValid: return kib < kvv[j];
    case kMaskLocal:
      return (p.win_left < 0 || row - key <= p.win_left) &&
             (p.win_right < 0 || key - row <= p.win_right);
    default: return true;
  }
}

// Staging of rows 0 .. n-1 (n <= 64) of a [*, D] bf16 tensor (row stride ss)
// into LDS: row-major at rm (row pitch RM bytes) and/or transposed at tr
// (tr[d] is a row of 64 positions, pitch TR bytes); rows past n are zero.
// load() issues the global reads into registers, store() writes LDS, so the
// reads of the next sub-tile can be in flight while the current one is
// computed.  Every thread of the workgroup takes part; no barrier inside.
template <int D, int NT>
struct Stage {
  static constexpr int DC = D / 8;
  static constexpr int RM = D * 2 + 16;
  static constexpr int TR = kBwdT * 2 + 16;
  static constexpr int BL = (kBwdT / 4) * DC;  // blocks of 4 rows x 8 dims
  static constexpr int PER = (BL + NT - 1) / NT;
  uint4 r[PER][4];
  __device__ __forceinline__ void load(const __bf16* base, int64_t ss, int n, int tid) {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int bi = tid + c * NT;
      const int g = bi / DC, dc = bi % DC;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = 4 * g + rr;
        r[c][rr] = (bi < BL && row < n)
                       ? *reinterpret_cast<const uint4*>(base + (int64_t)row * ss + dc * 8)
                       : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(unsigned char* rm, unsigned char* tr, int tid) const {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int bi = tid + c * NT;
      if (bi >= BL) continue;
      const int g = bi / DC, dc = bi % DC;
      if (rm) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<uint4*>(rm + (4 * g + rr) * RM + dc * 16) = r[c][rr];
      }
      if (tr) {
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const uint32_t x0 = word4(r[c][0], dd >> 1), x1 = word4(r[c][1], dd >> 1);
          const uint32_t x2 = word4(r[c][2], dd >> 1), x3 = word4(r[c][3], dd >> 1);
          uint2 out;
          if ((dd & 1) == 0) {
            out.x = (x0 & 0xffffu) | (x1 << 16);
            out.y = (x2 & 0xffffu) | (x3 << 16);
          } else {
            out.x = (x0 >> 16) | (x1 & 0xffff0000u);
            out.y = (x2 >> 16) | (x3 & 0xffff0000u);
          }
          *reinterpret_cast<uint2*>(tr + (dc * 8 + dd) * TR + g * 8) = out;
        }
      }
    }
  }
};

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

// Product over head_dim of two 32x32 tiles: rows arow / arow+32 of the LDS
// tile (pitch RM) against this lane's fragments.
template <int D>
__device__ __forceinline__ void tile_dot(const unsigned char* lds, int arow, int h32,
                                         const uint4 (&frag)[D / 16], f32x16_t& s0,
                                         f32x16_t& s1) {
  constexpr int RM = D * 2 + 16;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = 0.f;
    s1[r] = 0.f;
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint4 a0 = *reinterpret_cast<const uint4*>(lds + arow * RM + ks * 32 + h32 * 16);
    const uint4 a1 = *reinterpret_cast<const uint4*>(lds + (arow + 32) * RM + ks * 32 + h32 * 16);
    s0 = mfma32(a0, frag[ks], s0);
    s1 = mfma32(a1, frag[ks], s1);
  }
}

// acc[db] += T^T(LDS, transposed tile: tr[d][64]) x operand(pk), over the 64
// positions of the sub-tile.
template <int DB>
__device__ __forceinline__ void tr_product(const unsigned char* tr, int arow, int h32,
                                           const uint32_t (&pk0)[8], const uint32_t (&pk1)[8],
                                           f32x16_t (&acc)[DB]) {
  constexpr int TR = kBwdT * 2 + 16;
#pragma unroll
  for (int ps = 0; ps < 4; ++ps) {
    const uint4 bop = p_operand(pk0, pk1, ps);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint4 a =
          *reinterpret_cast<const uint4*>(tr + (db * 32 + arow) * TR + ps * 32 + h32 * 16);
      acc[db] = mfma32(a, bop, acc[db]);
    }
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

// D[b,h,r] = sum_d dO * O (fp32), one thread per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const BwdParams p) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  if (t >= rows) return;
  const int r = (int)(t % p.Sq);
  const int64_t bh = t / p.Sq;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const __bf16* o = reinterpret_cast<const __bf16*>(p.o) + b * p.o_sb + r * p.o_ss + h * p.o_sh;
  const __bf16* g = reinterpret_cast<const __bf16*>(p.dout) + b * p.do_sb + r * p.do_ss + h * p.do_sh;
  float acc = 0.f;
  for (int c = 0; c < D / 8; ++c) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + c * 8);
    const uint4 e = *reinterpret_cast<const uint4*>(g + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = word4(a, i), y = word4(e, i);
      acc = fmaf(__uint_as_float(x << 16), __uint_as_float(y << 16), acc);
      acc = fmaf(__uint_as_float(x & 0xffff0000u), __uint_as_float(y & 0xffff0000u), acc);
    }
  }
  p.drow[t] = acc;
}

// log2-domain LSE for exp2(s*c - lse2); a row with no key (LSE = -inf) gives
// +inf, so every p of it is 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse == neg_inf() ? __builtin_inff() : lse * 1.4426950408889634f;  // log2(e)
}

template <int D, int NW, bool VL>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))  // two waves per SIMD up to d = 128
void bwd_dq_kernel(const BwdParams p) {
  constexpr int NT = NW * 64, TW = NW * 32;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int RM = D * 2 + 16, TR = kBwdT * 2 + 16;
  __shared__ __attribute__((aligned(16))) unsigned char Kb[kBwdT * RM];
  __shared__ __attribute__((aligned(16))) unsigned char Vb[kBwdT * RM];
  __shared__ __attribute__((aligned(16))) unsigned char KTb[D * TR];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
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
  const int arow = swap_b23(l32);

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
  Stage<D, NT> sk, sv;
  bool have = W.first();
  if (have) {
    const int nk = min(kBwdT, W.end - W.pos);
    sk.load(kb0 + (int64_t)W.pos * p.k_ss, p.k_ss, nk, tid);
    sv.load(vb0 + (int64_t)W.pos * p.v_ss, p.v_ss, nk, tid);
    sk.store(Kb, KTb, tid);
    sv.store(Vb, nullptr, tid);
  }
  __syncthreads();
  while (have) {
    const int list = W.list, j = W.id, k0 = W.pos, nk = min(kBwdT, W.end - W.pos);
    const bool more = W.next();
    if (more) {  // next sub-tile's reads in flight during this one's products
      const int nn = min(kBwdT, W.end - W.pos);
      sk.load(kb0 + (int64_t)W.pos * p.k_ss, p.k_ss, nn, tid);
      sv.load(vb0 + (int64_t)W.pos * p.v_ss, p.v_ss, nn, tid);
    }
    {
      f32x16_t s0, s1, d0, d1;
      tile_dot<D>(Kb, arow, h32, qf, s0, s1);
      tile_dot<D>(Vb, arow, h32, gf, d0, d1);
      uint32_t pk0[8], pk1[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        float v[4];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int reg = 2 * x + (y & 1);
          const f32x16_t& sv_ = y < 2 ? s0 : s1;
          const f32x16_t& dv_ = y < 2 ? d0 : d1;
          const int key = 16 * (reg >> 3) + 8 * h32 + (reg & 7) + (y < 2 ? 0 : 32);
          bool keep = key < nk;
          if (keep && list == 0)
            keep = keep_elem(p, sv0.kvv, row, k0 + key, j, k0 + key - j * p.block_kv);
          const float pr = keep ? __builtin_amdgcn_exp2f(fmaf(sv_[reg], p.c, -lse2)) : 0.f;
          v[y] = pr * (dv_[reg] - drow);
        }
        pk0[x] = pack_bf16x2(v[0], v[1]);
        pk1[x] = pack_bf16x2(v[2], v[3]);
      }
      tr_product<DB>(KTb, arow, h32, pk0, pk1, acc);
    }
    __syncthreads();  // every wave is done with this sub-tile
    if (more) {
      sk.store(Kb, KTb, tid);
      sv.store(Vb, nullptr, tid);
    }
    __syncthreads();
    have = more;
  }
  if (rvalid) {
    __bf16* dst = reinterpret_cast<__bf16*>(p.dq) + b * p.dq_sb + qtok * p.dq_ss + h * p.dq_sh;
    store_row<DB>(dst, h32, acc, p.scale);
  }
}

template <int D, int NW, bool VL>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(const BwdParams p) {
  constexpr int NT = NW * 64, TW = NW * 32;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int RM = D * 2 + 16, TR = kBwdT * 2 + 16;
  __shared__ __attribute__((aligned(16))) unsigned char Qb[kBwdT * RM];
  __shared__ __attribute__((aligned(16))) unsigned char Gb[kBwdT * RM];
  __shared__ __attribute__((aligned(16))) unsigned char QTb[D * TR];
  __shared__ __attribute__((aligned(16))) unsigned char GTb[D * TR];
  __shared__ float lse2s[kBwdT], drows[kBwdT];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
  const int ksub = cdiv(p.block_kv, TW);
  int t = blockIdx.x;
  const int s = t % ksub;
  t /= ksub;
  // nrow: the KV-major list row (batched: KV block j; varlen: global KV block id)
  const int nrow = t % p.N;
  t /= p.N;
  const int Hkv = p.H / p.hrep;
  const int hk = VL ? t : t % Hkv;
  const SeqView sv0 = seq_view<VL>(p, VL ? seq_of(p.cu_n, p.B, nrow) : t / Hkv);
  const int b = sv0.b;
  const int j = VL ? nrow - p.cu_n[b] : nrow;
  const int k0 = j * p.block_kv + s * TW;
  const int kend = min((j + 1) * p.block_kv, sv0.Sk);
  if (k0 >= kend) return;
  const int key = k0 + 32 * w + l32;  // sequence-local
  const bool kvalid = key < kend;

  const int64_t ktok = (int64_t)sv0.tk0 + key;
  const __bf16* krow = reinterpret_cast<const __bf16*>(p.k) + b * p.k_sb + ktok * p.k_ss + hk * p.k_sh;
  const __bf16* vrow = reinterpret_cast<const __bf16*>(p.v) + b * p.v_sb + ktok * p.v_ss + hk * p.v_sh;
  uint4 kf[DS], vf[DS];
  row_frags<D>(krow, kvalid, h32, kf);
  row_frags<D>(vrow, kvalid, h32, vf);

  f32x16_t dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }
  const int arow = swap_b23(l32);

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
    Stage<D, NT> sq, sg;
    float l2n = 0.f, drn = 0.f;  // this thread's row (tid < 64) of the next sub-tile
    auto load = [&]() {
      const int nr = min(kBwdT, W.end - W.pos), r0 = W.pos;
      sq.load(qb0 + (int64_t)r0 * p.q_ss, p.q_ss, nr, tid);
      sg.load(gb0 + (int64_t)r0 * p.do_ss, p.do_ss, nr, tid);
      if (tid < kBwdT) {
        l2n = tid < nr ? lse2_of(p.lse[lbase + r0 + tid]) : __builtin_inff();
        drn = tid < nr ? p.drow[lbase + r0 + tid] : 0.f;
      }
    };
    auto store = [&]() {
      sq.store(Qb, QTb, tid);
      sg.store(Gb, GTb, tid);
      if (tid < kBwdT) {
        lse2s[tid] = l2n;
        drows[tid] = drn;
      }
    };
    __syncthreads();  // the previous head's last sub-tile is done
    bool have = W.first();
    if (have) {
      load();
      store();
    }
    __syncthreads();
    while (have) {
      const int list = W.list, r0 = W.pos, nr = min(kBwdT, W.end - W.pos);
      const bool more = W.next();
      if (more) load();  // next sub-tile's reads in flight during this one's products
      f32x16_t s0, s1, d0, d1;
      tile_dot<D>(Qb, arow, h32, kf, s0, s1);
      tile_dot<D>(Gb, arow, h32, vf, d0, d1);
      uint32_t pk0[8], pk1[8], dk0[8], dk1[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        float pv[4], dsv[4];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int reg = 2 * x + (y & 1);
          const f32x16_t& sv = y < 2 ? s0 : s1;
          const f32x16_t& gv = y < 2 ? d0 : d1;
          const int rl = 16 * (reg >> 3) + 8 * h32 + (reg & 7) + (y < 2 ? 0 : 32);
          bool keep = kvalid && rl < nr;
          if (keep && list == 0)
            keep = keep_elem(p, sv0.kvv, r0 + rl, key, j, key - j * p.block_kv);
          const float pr = keep ? __builtin_amdgcn_exp2f(fmaf(sv[reg], p.c, -lse2s[rl])) : 0.f;
          pv[y] = pr;
          dsv[y] = pr * (gv[reg] - drows[rl]);
        }
        pk0[x] = pack_bf16x2(pv[0], pv[1]);
        pk1[x] = pack_bf16x2(pv[2], pv[3]);
        dk0[x] = pack_bf16x2(dsv[0], dsv[1]);
        dk1[x] = pack_bf16x2(dsv[2], dsv[3]);
      }
      tr_product<DB>(GTb, arow, h32, pk0, pk1, dv);
      tr_product<DB>(QTb, arow, h32, dk0, dk1, dk);
      __syncthreads();  // every wave is done with this sub-tile
      if (more) store();
      __syncthreads();
      have = more;
    }
  }

  if (kvalid) {
    __bf16* kdst = reinterpret_cast<__bf16*>(p.dk) + b * p.dk_sb + ktok * p.dk_ss + hk * p.dk_sh;
    __bf16* vdst = reinterpret_cast<__bf16*>(p.dv) + b * p.dv_sb + ktok * p.dv_ss + hk * p.dv_sh;
    store_row<DB>(kdst, h32, dk, p.scale);
    store_row<DB>(vdst, h32, dv, 1.f);
  }
}

template <int D, bool VL>
hipError_t launch_bwd_dv(const BwdParams& p, hipStream_t st) {
  // varlen: the row dots run over [H, total_q] as one sequence of Sq rows
  const int64_t rows = (VL ? 1 : (int64_t)p.B) * p.H * p.Sq;
  if (rows > 0) {
    BwdParams pr = p;
    if (VL) pr.B = 1;
    hipLaunchKernelGGL(bwd_rowdot_kernel<D>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       st, pr);
  }
  // batched: B*H*M Q-block rows and B*H_kv*N KV-block rows; varlen: the
  // M and N totals over the sequences carry the batch
  const int64_t nb = VL ? 1 : p.B;
  const int nwq = p.block_q % 128 == 0 ? 4 : 2, nwk = p.block_kv % 128 == 0 ? 4 : 2;
  const int64_t gq = nb * p.H * p.M * ((p.block_q + 32 * nwq - 1) / (32 * nwq));
  const int64_t gk = nb * (p.H / p.hrep) * p.N * ((p.block_kv + 32 * nwk - 1) / (32 * nwk));
  if (gq > 0) {
    if (nwq == 4)
      hipLaunchKernelGGL((bwd_dq_kernel<D, 4, VL>), dim3((unsigned)gq), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, 2, VL>), dim3((unsigned)gq), dim3(128), 0, st, p);
  }
  if (gk > 0) {
    if (nwk == 4)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, 4, VL>), dim3((unsigned)gk), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, 2, VL>), dim3((unsigned)gk), dim3(128), 0, st, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t st) {
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
