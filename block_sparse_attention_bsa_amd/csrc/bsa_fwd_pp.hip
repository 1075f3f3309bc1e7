// Block-sparse attention forward for gfx950 (CDNA4): bf16 Q/K/V, 256 query
// rows per workgroup, eight waves in a ping-pong schedule.
//
// The walk is the one of flash-attention PR #2224 ("[CuTe,Flex] varlen
// blocksparsity") and of "Dense FlashAttention vs Block-Sparse Attention"
// (sections 4 and 6): each workgroup reads its Q block's mask and full
// block lists, and only the listed K/V blocks are fetched, at addresses
// taken from the list, so skipped blocks are never touched.  Listed blocks
// are cut into 64-key sub-tiles ("items").
//
// Schedule.  Waves 0-3 (group 0) and 4-7 (group 1) share the four SIMDs,
// one wave of each group per SIMD.  Per item a wave has an MFMA phase
// (O += P_j V_j, then S_{j+1} = K_{j+1} Q^T: D/8 + D/8 MFMAs of 32 cycles)
// and a VALU phase (element mask, row max, lazy rescale, exp, P in bf16,
// row sum).  Between two workgroup barriers group 0 runs its MFMA phase
// first and group 1 its VALU phase first, so on every SIMD one wave keeps
// the matrix core busy while the other does its softmax; one barrier per
// item keeps the K/V ring consistent.
//
// K/V staging.  A four-stage LDS ring holds one item per stage; item j+3 is
// fetched while item j computes.  Each stage is K [64 keys][RSK slots] then
// V [64 keys][RSV slots] of 16 bytes.  For D = 64 and 128 the rows are not
// padded (RS = D/8) and the 16-byte chunk c of key r sits at position
// c ^ swz(r) of its row, an XOR swizzle that keeps both read patterns free
// of bank conflicts: K (ds_read_b128, 16 lanes read one chunk of 16 keys)
// uses swz = r & 15 (D = 128) or (r >> 1) & 7 (D = 64), so the 16 keys
// land on 16 different 16-byte bank groups; V (ds_read_b64_tr_b16, half a
// wave reads 64 bytes of each of 4 consecutive keys) uses swz = 4 * (r & 3)
// (D = 128) or 4 * ((r >> 1) & 1) (D = 64), so the 4 keys fill the 4
// quarters of the 64 banks.  The swizzle only touches address bits 4-7, so
// a lane keeps one address per K k-step and per V head-dim block and the
// DMA lanes fetch their chunks in permuted order.  D = 96 (12 chunks) pads
// instead: odd K stride, V stride 12 (mod 16).  The stage is cut into 1 KiB blocks dealt round-robin to the
// eight waves; each block is one buffer_load_dwordx4 ... lds (64 lanes x 16
// bytes straight into LDS) from a per-lane offset computed once, issued
// between two MFMAs of the MFMA phase.  Waves w < NFULLW own JMAX blocks of
// a stage, the others JMAX - 1, and each ends the interval with a vmcnt
// wait of its own count: "all but the newest item landed".  The buffer
// descriptor of an item spans only its visible keys, so rows past a partial
// item's key count read as zero: no clamping and no reads past the sequence
// end.  DMAs whose lanes are all out of range cost several times as much as
// in-range ones, so there are no padding DMAs, and an item past the end of
// the list reloads the sequence's first keys into a stage nobody reads.  Read geometry (odd K stride for ds_read_b128, V stride 4 or
// 12 mod 16 for ds_read_b64_tr_b16) is the same as in the other bf16
// kernel: no LDS bank conflicts.
//
// Softmax.  The running max m is lazy.  Each item's P = 2^(s*c - m) is
// taken against the current m first, with the lane's sum over its 32 keys;
// only if that sum leaves [0, kSumCap] (m stale by more than 16 in log2
// units, or still -inf before any key of the row was seen) does the wave
// take the row max, rescale O and l, and redo the item.  So the common item
// has no max reduction at all, P stays <= 2^16 (far inside fp32 and bf16
// range), and O, l and the LSE are all relative to the same m.  The row
// sum is taken over the fp32 P (so the LSE carries no bf16 rounding) and O
// is divided by it; P is rounded to bf16 only for the PV product.  Dividing
// O by the sum of the bf16 P instead (exact weights on rows dominated by
// one key) costs 13-20 % of the whole kernel here, however that sum is
// formed (v_dot2c_f32_bf16 per pair, or unpacking the pairs): the softmax
// phase already sets the length of the interval, and every VALU op added
// to it lengthens it.  So a row dominated by a few keys keeps the bf16
// rounding of their P (relative 2^-8) in O.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bsa_fwd_common.h"

namespace bsa {
namespace {

using namespace dev;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

// Word 3 of a raw (unstrided) buffer descriptor on the gfx9 family: 32-bit
// data format, no swizzle; accesses at or past num_records return zero.
constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ u32x4_t make_rsrc(uint64_t addr, uint32_t bytes) {
  u32x4_t r;
  r.x = (uint32_t)addr;
  r.y = (uint32_t)(addr >> 32) & 0xFFFFu;
  r.z = bytes;
  r.w = kRsrcWord3;
  return r;
}

// One wave-wide 16-byte-per-lane DMA: lane l's 16 bytes at descriptor
// offset `off` land at LDS byte address lds_addr + 16*l (lds_addr in M0).
// Issued from inline assembly so the compiler neither waits for it nor
// reorders LDS accesses across it; the kernel orders it with vmcnt waits and
// barriers.  The compiler's hazard checks do not see inside the asm: its
// s_nop 0 covers the M0 write only.  A VALU write of a descriptor SGPR
// (v_readlane restoring a spill) needs five wait states before a
// vector-memory read of it; this kernel builds its descriptors with scalar
// instructions and keeps them in SGPRs, which tests/test_asm_hazards.py
// checks in the compiled code (four more wait states per DMA cost 1.2 % of
// the video workload).
__device__ __forceinline__ void dma16(u32x4_t rsrc, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc),
               "{m0}"(lds_addr)
               : "memory");
}

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory ops in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint2 read_tr(const char* lds, int byte_off) {
  lds_char* base = (lds_char*)(lds);
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + byte_off));
  return __builtin_bit_cast(uint2, v);
}

// What the pipeline keeps of an item: first key, and the visible-key count
// (1..64) with the mask-list flag in bit 7.  nm == 0: no item (past the end).
struct Sub {
  int key0, nm;
  __device__ __forceinline__ int nk() const { return nm & 127; }
  __device__ __forceinline__ bool is_mask() const { return nm >> 7; }
};

// The items of one Q block: the mask list, then the full list, each listed
// KV block cut into 64-key items, blocks and items with no visible key
// skipped.  List entries are fetched 64 at a time, one per lane (its block's
// first key and visible-key count: the block size clipped to the sequence,
// for a mask-list block under the valid-count mask_mod also to its valid
// count, 0 for an id outside [0, num_n)), and read back with readlane.
struct ItemStream {
  const int32_t* mrow;
  const int32_t* frow;
  int64_t ms, fs;
  int mcnt, total, bk, Sk, num_n;
  const int32_t* kv_valid;  // non-null: valid-count mask_mod
  int g, st, base, key_base, vis;
  int ck, cv;  // lane chunk

  __device__ __forceinline__ void load(int gb, int lane) {
    base = gb;
    const int gg = gb + lane;
    int j = -1;
    if (gg < mcnt)
      j = mrow[gg * ms];
    else if (gg < total)
      j = frow[(gg - mcnt) * fs];
    int v = 0;
    if (gg < total && j >= 0 && j < num_n) {
      v = min(bk, Sk - j * bk);
      if (kv_valid != nullptr && gg < mcnt) v = min(v, kv_valid[j]);
    }
    ck = j * bk;
    cv = v;
  }
  // Next item; false (and out.nm = 0) past the end.
  __device__ __forceinline__ bool next(int lane, Sub& out) {
    int s = st + 1;
    while (s * kKvTile >= vis) {
      ++g;
      if (g >= total) {
        out.nm = 0;
        st = s;
        vis = 0;
        g = total;
        return false;
      }
      if (g >= base + 64) load(g, lane);
      key_base = __builtin_amdgcn_readlane(ck, g - base);
      vis = __builtin_amdgcn_readlane(cv, g - base);
      s = 0;
    }
    st = s;
    out.key0 = key_base + s * kKvTile;
    out.nm = min(vis - s * kKvTile, kKvTile) | (g < mcnt ? 128 : 0);
    return true;
  }
};

constexpr int NW_PP = 8;  // waves per workgroup

template <int D>
struct PPCfg {
  static constexpr int NW = NW_PP, TM = 256;
  static constexpr int DS = D / 16;  // QK^T k-steps
  static constexpr int DB = D / 32;  // O^T row blocks
  static constexpr int DC = D / 8;   // 16-byte chunks per row
  static constexpr bool SWZ = D == 64 || D == 128;  // unpadded, XOR-swizzled rows
  static constexpr int RSK = SWZ ? DC : DC + 1;     // else odd
  static constexpr int RSV = SWZ ? DC : (DC % 16 == 4 || DC % 16 == 12) ? DC : DC + 4;  // else 4/12 mod 16
  static constexpr int KBLK = RSK, VBLK = RSV;  // 1 KiB blocks: 64 keys x RS slots / 64 lanes
  static constexpr int NBLK = KBLK + VBLK;
  static constexpr int KSLOTS = 64 * RSK;
  static constexpr int STAGE_SLOTS = 64 * NBLK;
  static constexpr int STAGE_BYTES = STAGE_SLOTS * 16;
  static constexpr int STAGES = 4;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int JMAX = (NBLK + NW - 1) / NW;      // most DMA instructions of a wave per item
  static constexpr int NFULLW = NBLK - NW * (JMAX - 1);  // waves w < NFULLW issue JMAX
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(DC % 2 == 0 && (SWZ || (RSK % 2 == 1 && RSV % 16 != 0 && RSV % 4 == 0)),
                "stride rules");
  // chunk position swizzles of K and V rows (see the header)
  __device__ __forceinline__ static int kswz(int r) {
    return D == 128 ? (r & 15) : D == 64 ? ((r >> 1) & 7) : 0;
  }
  __device__ __forceinline__ static int vswz(int r) {
    return D == 128 ? 4 * (r & 3) : D == 64 ? 4 * ((r >> 1) & 1) : 0;
  }
};

template <int D, bool VARLEN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bsa_fwd_pp_kernel(const FwdParams p) {
  using C = PPCfg<D>;
  constexpr int DS = C::DS, DB = C::DB, DC = C::DC, RSK = C::RSK, RSV = C::RSV;
  constexpr int JMAX = C::JMAX;
  __shared__ uint4 smem[C::LDS_BYTES / 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, h32 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  const bool g1 = w >= 4;

  TileInfo ti;
  // Batched tiles in dispatch order: the GPU then works on about one head's Q
  // tiles at a time, whose K/V the 256 MB last-level cache holds (each XCD a
  // contiguous range, as the other kernels do, keeps eight heads in flight
  // and measured 2 % slower on the video workload); varlen keeps the XCD
  // ranges, which its longest-first order was measured with.
  if (!decode_tile<256, VARLEN ? 1 : 0>(p, VARLEN ? xcd_remap(blockIdx.x, p.num_tiles)
                                                   : (int)blockIdx.x, ti))
    return;
  // GQA packing: wave w holds rows (32*w) % R .. of head ti.h + 32*w / R
  // (R = 256 / gpack rows per head), and every head of the tile walks the
  // same items.  Without packing R = 256 and dh = 0.
  const int R = 256 / p.gpack;
  const int dh = (32 * w) / R;
  ti.qoff += dh * p.q_sh;
  ti.ooff += dh * p.o_sh;
  ti.lse_base += dh * ti.lse_hs;
  const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + ti.qoff;
  const uint64_t kaddr = reinterpret_cast<uint64_t>(reinterpret_cast<const __bf16*>(p.k) + ti.koff);
  const uint64_t vaddr = reinterpret_cast<uint64_t>(reinterpret_cast<const __bf16*>(p.v) + ti.voff);

  const int q0w = ti.q0 + (32 * w) % R;
  const int qrow = q0w + l32;
  uint4 qf[DS];
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = neg_inf(), l_a = 0.f, l_b = 0.f;

  // DMA geometry: block b = w + 8*jj of a stage (K blocks first, then V);
  // lane l fills slot 64*b + l, i.e. key slot / RS, chunk position slot % RS,
  // which holds chunk position ^ swz(key) (swizzled rows) or the chunk itself
  // (padded rows: a padding slot repeats the row's last chunk, never read).  Block
  // w + 8*(JMAX-1) exists only for waves w < NFULLW.
  const uint32_t kss2 = (uint32_t)(p.k_ss * 2), vss2 = (uint32_t)(p.v_ss * 2);
  const uint32_t lds_base = (uint32_t)(size_t)((lds_char*)smem);
  uint32_t doff[JMAX];
#pragma unroll
  for (int jj = 0; jj < JMAX; ++jj) {
    const int b = min(w + 8 * jj, C::NBLK - 1);
    const bool isk = b < C::KBLK;
    const int rs = isk ? RSK : RSV;
    const int slot = (isk ? b : b - C::KBLK) * 64 + lane;
    const int key = slot / rs, pos = slot % rs;
    const int chunk = C::SWZ ? pos ^ (isk ? C::kswz(key) : C::vswz(key)) : min(pos, DC - 1);
    doff[jj] = (uint32_t)key * (isk ? kss2 : vss2) + (uint32_t)chunk * 16u;
  }
  // descriptors of one item: K and V.  An item past the end (nm == 0)
  // points at the sequence's first keys; its stage is never read.
  struct Rsrc {
    u32x4_t k, v;
  };
  const int nk_none = min(kKvTile, ti.Sk);
  auto rsrc_of = [&](const Sub& it) {
    const uint32_t k0 = it.nm != 0 ? (uint32_t)it.key0 : 0u;
    const uint32_t nk = it.nm != 0 ? (uint32_t)it.nk() : (uint32_t)nk_none;
    Rsrc r;
    r.k = make_rsrc(kaddr + (uint64_t)k0 * kss2, nk * kss2);
    r.v = make_rsrc(vaddr + (uint64_t)k0 * vss2, nk * vss2);
    return r;
  };
  // DMA instruction jj of an item into a stage (the last jj only for w < NFULLW)
  auto dma_part = [&](const Rsrc& r, int stage, int jj) {
    const int b = w + 8 * jj;
    if (C::NFULLW < NW_PP && jj == JMAX - 1 && b >= C::NBLK) return;
    dma16(b < C::KBLK ? r.k : r.v, doff[jj],
          lds_base + (uint32_t)(stage * C::STAGE_BYTES + b * 1024));
  };
  auto issue = [&](const Sub& it, int stage) {
    const Rsrc r = rsrc_of(it);
#pragma unroll
    for (int jj = 0; jj < JMAX; ++jj) dma_part(r, stage, jj);
  };

  // per-lane LDS read geometry.  K: row arow (+32 for the second key half),
  // chunk 2*ks + h32.  V: key vkey + 16*ps (+4 for the second read), head
  // dims 32*db + vd .. +3.  Swizzled rows: the k-step and the head-dim block
  // enter as an XOR on address bits 4-7, so one address per ks (K) and per
  // db (V); the key offsets added after it leave those bits alone.
  const int arow = swap_b23(l32);
  const int kbase = (arow * RSK + h32) * 16;  // padded rows: + kh*32*RSK*16 + ks*32 bytes
  const int vs = lane & 15, vg = lane >> 4;
  const int vkey = 8 * h32 + (vs >> 2);
  const int vd = 16 * (vg & 1) + 4 * (((vs & 1) << 1) | ((vs >> 1) & 1));
  const int vbase = (vkey * RSV + (vd >> 3)) * 16 + 8 * ((vd >> 2) & 1);  // padded: + ps, db offsets
  int kx[C::SWZ ? DS : 1], vx[C::SWZ ? DB : 1];
  if constexpr (C::SWZ) {
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
      kx[ks] = (arow * RSK * 16 + 16 * (h32 ^ C::kswz(arow))) ^ (32 * ks);
#pragma unroll
    for (int db = 0; db < DB; ++db) vx[db] = (vbase + 16 * C::vswz(vkey)) ^ (64 * db);
  }

  f32x16_t s0, s1;          // S^T of the item after the one being accumulated
  uint32_t pk0[8], pk1[8];  // P^T (bf16 pairs) of the item being accumulated

  // MFMA phase: slots 0..NPV-1 are O^T += V^T P^T (ps = slot / DB, db =
  // slot % DB; A operand = two transposing reads of V), slots NPV.. are
  // S^T = K Q^T (ks = k / 2, key half = k % 2; A operand = one ds_read_b128
  // of K).  Operands are read kWin slots ahead of their MFMA so the LDS
  // latency hides behind the MFMAs in between; the slot order is pinned.
  constexpr int NPV = 4 * DB, NQK = 2 * DS, kWin = 5;
  // vl: the stage's V tile; kb: its K tile (+ kbase for padded rows)
  auto operand = [&](int i, const char* vl, const char* kb) -> uint4 {
    if (i < NPV) {
      const int ps = i / DB, db = i % DB;
      const int off = C::SWZ ? vx[C::SWZ ? db : 0] + 16 * ps * RSV * 16
                             : vbase + (16 * ps * RSV + 4 * db) * 16;
      const uint2 t0 = read_tr(vl, off);
      const uint2 t1 = read_tr(vl, off + 4 * RSV * 16);
      return make_uint4(t0.x, t0.y, t1.x, t1.y);
    }
    const int k = i - NPV;
    if constexpr (C::SWZ)
      return *reinterpret_cast<const uint4*>(kb + kx[k >> 1] + (k & 1) * 32 * RSK * 16);
    return *reinterpret_cast<const uint4*>(kb + (k & 1) * 32 * RSK * 16 + (k >> 1) * 32);
  };
  auto slot = [&](int i, const uint4& a) {
    if (i < NPV) {
      const int ps = i / DB, db = i % DB;
      oacc[db] = mfma32(a, p_operand(pk0, pk1, ps), oacc[db]);
    } else {
      const int k = i - NPV;
      if (k & 1)
        s1 = mfma32(a, qf[k >> 1], s1);
      else
        s0 = mfma32(a, qf[k >> 1], s0);
    }
  };
  // NS = NPV (accumulate only) or NPV + NQK (accumulate, then next scores).
  // With `dma`, DMA instruction jj of item `nxt` into stage `nstage` goes
  // right after MFMA slot jj + 1.
  auto mfma_phase = [&](auto ns_tag, int vstage, int kstage, bool dma, const Sub& nxt,
                        int nstage) {
    constexpr int NS = decltype(ns_tag)::value;
    const char* vl = reinterpret_cast<const char*>(smem + vstage * C::STAGE_SLOTS + C::KSLOTS);
    const char* kb = reinterpret_cast<const char*>(smem + kstage * C::STAGE_SLOTS) +
                     (C::SWZ ? 0 : kbase);
    if constexpr (NS > NPV) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = 0.f;
        s1[r] = 0.f;
      }
    }
    Rsrc r;
    uint4 op[kWin + 1];
#pragma unroll
    for (int i = 0; i < kWin && i < NS; ++i) op[i] = operand(i, vl, kb);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + kWin < NS) op[(i + kWin) % (kWin + 1)] = operand(i + kWin, vl, kb);
      __builtin_amdgcn_sched_barrier(0);
      slot(i, op[i % (kWin + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      if (dma) {
        if (i == 0) r = rsrc_of(nxt);
        if (i >= 1 && i <= JMAX) dma_part(r, nstage, i - 1);
      }
    }
  };
  auto qk_only = [&](int kstage) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
    const char* kb = reinterpret_cast<const char*>(smem + kstage * C::STAGE_SLOTS) +
                     (C::SWZ ? 0 : kbase);
#pragma unroll
    for (int k = 0; k < NQK; ++k) slot(NPV + k, operand(NPV + k, nullptr, kb));
  };
  // VALU phase of one item: s0/s1 -> pk0/pk1, running max and sum.
  const bool causal = p.mask_mod == kMaskCausal;
  const float c = p.c;
  auto softmax = [&](const Sub& it) {
    const bool diag = causal && it.is_mask() && it.key0 + kKvTile - 1 > q0w;
    if (it.nk() < kKvTile || diag) {
      // keep key k of the item iff k < lim; accumulator r of lane half h32
      // holds key 16*(r/8) + 8*h32 + r%8 (+32 for s1)
      int lim = it.nk();
      if (diag) lim = min(lim, qrow - it.key0 + 1);
      const int t = lim - 8 * h32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 16 * (r >> 3) + (r & 7);
        s0[r] = kr < t ? s0[r] : neg_inf();
        s1[r] = kr + 32 < t ? s1[r] : neg_inf();
      }
    }
    // P against the running max, and this lane's sum over its 32 keys.
    float la = 0.f, lb = 0.f;
    auto exps = [&](float mu) {
      la = 0.f;
      lb = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a0 = __builtin_amdgcn_exp2f(fmaf(s0[2 * i], c, -mu));
        const float a1 = __builtin_amdgcn_exp2f(fmaf(s0[2 * i + 1], c, -mu));
        const float b0 = __builtin_amdgcn_exp2f(fmaf(s1[2 * i], c, -mu));
        const float b1 = __builtin_amdgcn_exp2f(fmaf(s1[2 * i + 1], c, -mu));
        pk0[i] = pack_bf16x2(a0, a1);
        pk1[i] = pack_bf16x2(b0, b1);
        la += a0 + a1;
        lb += b0 + b1;
      }
    };
    exps(m_run);
    // Every P is at most the lane's sum, so a sum within kSumCap (it is
    // never NaN or inf then) bounds the whole item.  A larger sum means the
    // running max is stale by more than log2(kSumCap); inf or NaN means no
    // key of the row has been seen yet (m_run = -inf).  Both are rare: take
    // the row max, rescale, and redo the item.
    if (__any(!(la + lb <= kSumCap))) {
      float t3[11];
#pragma unroll
      for (int i = 0; i < 5; ++i) t3[i] = fmaxf(fmaxf(s0[3 * i], s0[3 * i + 1]), s0[3 * i + 2]);
#pragma unroll
      for (int i = 0; i < 5; ++i) t3[5 + i] = fmaxf(fmaxf(s1[3 * i], s1[3 * i + 1]), s1[3 * i + 2]);
      t3[10] = fmaxf(s0[15], s1[15]);
      float mx = fmaxf(fmaxf(fmaxf(fmaxf(t3[0], t3[1]), t3[2]), fmaxf(fmaxf(t3[3], t3[4]), t3[5])),
                       fmaxf(fmaxf(fmaxf(t3[6], t3[7]), t3[8]), fmaxf(t3[9], t3[10])));
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      // alpha = 2^(m_run - m_new); rows with nothing visible yet keep O = 0
      const float alpha = m_new == neg_inf() ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_a *= alpha;
      l_b *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
      exps(m_run == neg_inf() ? 0.f : m_run);
    }
    l_a += la;
    l_b += lb;
  };

  ItemStream L{ti.mrow, ti.frow, p.mi_s[3], p.fi_s[3], ti.mcnt, ti.mcnt + ti.fcnt,
               p.block_kv, ti.Sk, ti.num_n,
               p.mask_mod == kMaskKvValid ? ti.kvv : nullptr,
               -1, 0, -1000000, 0, 0, 0, 0};
  Sub t0, t1, t2, t3;
  const bool e0 = L.next(lane, t0);
  bool e1 = e0 && L.next(lane, t1);
  bool e2 = e1 && L.next(lane, t2);
  bool e3 = e2 && L.next(lane, t3);
  if (!e1) t1.nm = 0;
  if (!e2) t2.nm = 0;
  if (!e3) t3.nm = 0;

  // Rows past an item's visible keys are either zero-filled by the bounded
  // DMA or hold what an earlier item left: clearing the ring once keeps every
  // such V row finite (a masked key's P is 0, and 0 * finite = 0).
  for (int i = tid; i < C::LDS_BYTES / 16; i += 512) smem[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  // Items 0..2 (an item past the end loads nothing: empty descriptor).
  issue(t0, 0);
  issue(t1, 1);
  issue(t2, 2);
  // Q fragments (S^T MFMA B operand): Q[qrow][16*ks + 8*h32 .. +7].  Their
  // use right here makes the compiler wait for them (and so for the DMAs
  // issued above) before the loop, not inside it.
#pragma unroll
  for (int ks = 0; ks < DS; ++ks) {
    qf[ks] = qrow < ti.qend
                 ? *reinterpret_cast<const uint4*>(qp + (int64_t)qrow * p.q_ss + ks * 16 + h32 * 8)
                 : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int ks = 0; ks < DS; ++ks)
    asm volatile("" ::"v"(qf[ks].x), "v"(qf[ks].y), "v"(qf[ks].z), "v"(qf[ks].w));
  barrier();  // items 0..2 landed for every wave
  // Both groups take the scores of item 0; group 0 also its softmax (group 1
  // takes it at the start of its first interval).
  if (e0) {
    qk_only(0);
    if (!g1) softmax(t0);
  }
  // Interval j: group 0 runs [MFMA phase j, softmax j+1], group 1 runs
  // [softmax j, MFMA phase j], so on each SIMD one wave's MFMAs overlap the
  // other's softmax.  One barrier per interval: every wave's part of item
  // j+2 has landed, and no wave reads item j's stage any more (item j+4
  // refills it).  Items j and j+1 exist inside the loop; the last item's
  // accumulate-only phase is peeled off below (one MFMA-phase body keeps O
  // in one register set).  Every wave issues its JMAX or JMAX - 1 DMAs per
  // item, items past the end included, so "all but the newest item landed"
  // is vmcnt of that count.
  int j = 0;
  while (e1) {
    if (g1) softmax(t0);
    // MFMA phase of item j; item j+3 goes into the stage item j-1 used
    __builtin_amdgcn_s_setprio(1);
    mfma_phase(std::integral_constant<int, NPV + NQK>{}, j & 3, (j + 1) & 3, true, t3,
               (j + 3) & 3);
    __builtin_amdgcn_s_setprio(0);
    if (!g1) softmax(t1);
    // walk to item j+4
    t0 = t1;
    t1 = t2;
    e1 = e2;
    t2 = t3;
    e2 = e3;
    e3 = e3 && L.next(lane, t3);
    if (!e3) t3.nm = 0;
    if (w < C::NFULLW)  // item j+2 landed (this wave)
      wait_vmem<JMAX>();
    else
      wait_vmem<JMAX - 1>();
    barrier();
    ++j;
  }
  if (e0) {  // item j is the last one: accumulate only
    if (g1) softmax(t0);
    __builtin_amdgcn_s_setprio(1);
    mfma_phase(std::integral_constant<int, NPV>{}, j & 3, 0, false, t3, 0);
    __builtin_amdgcn_s_setprio(0);
  }
  wait_vmem<0>();      // no DMA of this workgroup outlives it
  epilogue<DB, __bf16>(p, ti, qrow, h32, m_run, l_a + l_b, l_a + l_b, oacc);
}

template <int D>
hipError_t launch_pp(const FwdParams& p, hipStream_t s) {
  FwdParams copy = p;
  void* args[] = {&copy};
  const void* k = p.varlen ? reinterpret_cast<const void*>(&bsa_fwd_pp_kernel<D, true>)
                           : reinterpret_cast<const void*>(&bsa_fwd_pp_kernel<D, false>);
  return hipLaunchKernel(k, dim3(p.num_tiles),
                         dim3(512), args, 0, s);
}

}  // namespace

hipError_t launch_fwd_pp(const FwdParams& p, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_pp<64>(p, s);
    case 96: return launch_pp<96>(p, s);
    case 128: return launch_pp<128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bsa
