// Block-sparse attention forward for gfx950 (CDNA4).
//
// One workgroup owns TM = 32*NW query rows of one (batch, head) and walks
// only the KV blocks named by its rows' block lists (mask list first, then
// the full list), as the block-sparse forward of flash-attention PR #2224
// ("[CuTe,Flex] varlen blocksparsity") and the runtime-indexed K/V fetch of
// "Dense FlashAttention vs Block-Sparse Attention" (sections 4 and 6)
// describe.  Each listed KV block is cut into 64-key sub-tiles; the next
// sub-tile's K and V rows are fetched from the block-index list into
// registers while the current one computes, then written into the other LDS
// stage (two stages, one barrier per sub-tile).  Skipped KV blocks are never
// touched.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64).  Each wave owns 32 query
// rows and computes everything transposed:
//     S^T[key, q] = K[key, :] . Q[q, :]          (A = K from LDS, B = Q in registers)
//     O^T[d, q]  += V^T[d, key] . P^T[key, q]    (A = V^T from LDS, B = P^T in registers)
// so every accumulator register of a lane belongs to the same query
// (q = lane % 32).  Row max needs one exchange between lane l and l^32 per
// sub-tile, the running sum needs none until the epilogue, and the O
// rescale is a per-lane scalar multiply.  The MFMA A-operand row i is
// loaded from K / V^T row swap_b23(i) (bits 2 and 3 of i exchanged) so that
// the 16 accumulator rows a lane receives form two runs of 8 consecutive
// keys (or head dims): P^T then feeds the PV MFMA straight from registers,
// V^T is read with 16-byte LDS loads, and O is stored in 16-byte pieces.
//
// Softmax runs in base 2 with the scale folded in (c = scale*log2 e), the
// running max is guarded so rows that see no key yet never form inf-inf,
// and P is rounded to bf16 for the PV MFMA.  Two running sums are kept: the
// rounded P (the same weights the PV product used) normalises O, and the
// fp32 P gives the LSE free of the bf16 rounding of P.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __builtin_bit_cast(float, x & 0xffff0000u); }

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Row permutation of the MFMA A operand: exchange bits 2 and 3.
__device__ __forceinline__ int swap_b23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// 8 consecutive input elements, held raw between the global load and the
// LDS store, and converted to 8 bf16 at store time.
template <bool F32> struct Chunk;
template <> struct Chunk<false> {
  uint4 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ uint4 bf16() const { return v; }
};
template <> struct Chunk<true> {
  // fp32 input is rounded to bf16 right at load (staging then matches the
  // bf16 path); fp32 inputs are a correctness path, not a fast one.
  uint4 v;
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                   pack_bf16x2(b.z, b.w));
  }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ uint4 bf16() const { return v; }
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Workgroups are dispatched round-robin over the 8 XCDs.  Renumber them so
// that each XCD receives one contiguous range of logical tiles: the Q tiles
// of one (batch, head) then share that XCD's L2 for their K/V blocks.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd, local = bid / kXcd;
  const int per = G / kXcd, rem = G % kXcd;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Concatenated (mask ++ full) block list of one Q-block row.  64 entries at
// a time are held one per lane and broadcast with readlane.
struct ListWalk {
  const int32_t* mrow;
  int64_t ms;
  int mcnt;
  const int32_t* frow;
  int64_t fs;
  int total;
  int base;
  int chunk;
  __device__ __forceinline__ int entry(int g, int lane) {
    if (g < base || g >= base + 64) {
      base = g;
      const int gg = g + lane;
      int val = -1;
      if (gg < mcnt)
        val = mrow[gg * ms];
      else if (gg < total)
        val = frow[(gg - mcnt) * fs];
      chunk = val;
    }
    return __builtin_amdgcn_readlane(chunk, g - base);
  }
};

// One unit of work: sub-tile st of the KV block listed at position g.
// blen is the number of leading keys of block j that can be visible: the
// block size, or for a mask-list block under the valid-count mask_mod its
// valid-token count (sub-tiles past it are never loaded).
struct Item {
  int g, st, j, blen, key0, nk, is_mask;
};

// Step to the next sub-tile that holds at least one key below Sk; entries
// with ids outside [0, num_n) are skipped.  Returns false at the end.
__device__ __forceinline__ bool advance(Item& it, ListWalk& L, int lane, int bk, int num_n,
                                        int Sk, int mask_mod, const int32_t* kv_valid) {
  int g = it.g, st = it.st + 1, j = it.j, blen = it.blen;
  while (true) {
    if (g >= 0 && st * kKvTile < blen) {
      const int key0 = j * bk + st * kKvTile;
      const int nk = min(min(kKvTile, blen - st * kKvTile), Sk - key0);
      if (nk > 0) {
        it.g = g;
        it.st = st;
        it.j = j;
        it.blen = blen;
        it.key0 = key0;
        it.nk = nk;
        it.is_mask = g < L.mcnt;
        return true;
      }
    }
    ++g;
    st = 0;
    if (g >= L.total) return false;
    j = L.entry(g, lane);
    blen = bk;
    if (j < 0 || j >= num_n)
      blen = 0;
    else if (mask_mod == 2 && g < L.mcnt)
      blen = min(bk, kv_valid[j]);
  }
}

template <int D, int NW, bool F32IN>
__global__ __launch_bounds__(NW * 64) void bsa_fwd_kernel(const FwdParams p) {
  using T = typename std::conditional<F32IN, float, __bf16>::type;
  constexpr int NT = NW * 64;
  constexpr int TM = NW * 32;
  constexpr int KT = kKvTile;
  constexpr int DS = D / 16;  // QK^T k-steps
  constexpr int DB = D / 32;  // O^T row blocks
  constexpr int KROW = D * 2 + 16;   // LDS bytes per K row (16 B pad)
  constexpr int VROW = KT * 2 + 16;  // LDS bytes per V^T row (16 B pad)
  constexpr int KBYTES = KT * KROW;
  constexpr int STAGE = KBYTES + D * VROW;
  constexpr int DC = D / 8;            // 16-byte chunks per row
  constexpr int KCH = KT * DC;         // K chunks per sub-tile
  constexpr int KC = (KCH + NT - 1) / NT;
  constexpr int VBL = (KT / 4) * DC;   // 4-key x 8-dim V blocks per sub-tile
  constexpr int VB = (VBL + NT - 1) / NT;
  static_assert(D % 32 == 0, "head_dim must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, h32 = lane >> 5;

  // ---- work tile -> (b, h, rows) and its block-list row
  const int t = xcd_remap(blockIdx.x, p.num_tiles);
  int h, q0, Sq_b, Sk_b, num_n;
  int64_t qoff, koff, voff, ooff, lse_base;
  const int32_t* mrow = nullptr;
  const int32_t* frow = nullptr;
  int mcnt = 0, fcnt = 0;
  if (!p.varlen) {
    const int qt = t % p.tiles_per_head;
    const int bh = t / p.tiles_per_head;
    h = bh % p.H;
    const int b = bh / p.H;
    const int hk = h / p.hrep;
    q0 = qt * TM;
    Sq_b = p.Sq;
    Sk_b = p.Sk;
    num_n = cdiv(Sk_b, p.block_kv);
    const int i = qt / p.qsub;
    qoff = b * p.q_sb + h * p.q_sh;
    koff = b * p.k_sb + hk * p.k_sh;
    voff = b * p.v_sb + hk * p.v_sh;
    ooff = b * p.o_sb + h * p.o_sh;
    lse_base = (int64_t)(b * p.H + h) * p.Sq;
    if (p.mcnt) {
      mcnt = p.mcnt[b * p.mc_s[0] + h * p.mc_s[1] + i * p.mc_s[2]];
      mrow = p.midx + b * p.mi_s[0] + h * p.mi_s[1] + i * p.mi_s[2];
    }
    if (p.fcnt) {
      fcnt = p.fcnt[b * p.fc_s[0] + h * p.fc_s[1] + i * p.fc_s[2]];
      frow = p.fidx + b * p.fi_s[0] + h * p.fi_s[1] + i * p.fi_s[2];
    }
  } else {
    const int tm = t % p.tiles_per_head;
    h = t / p.tiles_per_head;
    const int mg = tm / p.qsub, sub = tm % p.qsub;
    // sequence of Q block mg: largest b with cu_total_m_blocks[b] <= mg
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.cu_m[mid] <= mg)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int b = lo;
    const int m = mg - p.cu_m[b];
    const int sq0 = p.cu_q[b], sk0 = p.cu_k[b];
    Sq_b = p.cu_q[b + 1] - sq0;
    Sk_b = p.cu_k[b + 1] - sk0;
    num_n = cdiv(Sk_b, p.block_kv);
    q0 = m * p.block_q + sub * TM;
    if (m < 0 || m >= cdiv(Sq_b, p.block_q) || q0 >= Sq_b) return;  // whole workgroup
    const int64_t row_p = (int64_t)p.blk_off[b] + (int64_t)m * num_n;
    if (row_p < 0 || row_p + num_n > p.total_n) return;  // inconsistent bookkeeping
    const int hk = h / p.hrep;
    qoff = (int64_t)sq0 * p.q_ss + h * p.q_sh;
    koff = (int64_t)sk0 * p.k_ss + hk * p.k_sh;
    voff = (int64_t)sk0 * p.v_ss + hk * p.v_sh;
    ooff = (int64_t)sq0 * p.o_ss + h * p.o_sh;
    lse_base = (int64_t)h * p.lse_ld + sq0;
    if (p.mcnt) {
      mcnt = p.mcnt[h * p.mc_s[1] + mg * p.mc_s[2]];
      mrow = p.midx + h * p.mi_s[1] + row_p * p.mi_s[3];
    }
    if (p.fcnt) {
      fcnt = p.fcnt[h * p.fc_s[1] + mg * p.fc_s[2]];
      frow = p.fidx + h * p.fi_s[1] + row_p * p.fi_s[3];
    }
  }
  mcnt = min(max(mcnt, 0), num_n);
  fcnt = min(max(fcnt, 0), num_n);

  const T* qp = reinterpret_cast<const T*>(p.q) + qoff;
  const T* kp = reinterpret_cast<const T*>(p.k) + koff;
  const T* vp = reinterpret_cast<const T*>(p.v) + voff;

  // ---- Q fragments (MFMA B operand): Q[qrow][16*ks + 8*h32 .. +7]
  const int qrow = q0 + 32 * w + l32;
  uint4 qf[DS];
#pragma unroll
  for (int ks = 0; ks < DS; ++ks) {
    Chunk<F32IN> c;
    if (qrow < Sq_b)
      c.load(qp + (int64_t)qrow * p.q_ss + ks * 16 + h32 * 8);
    else
      c.zero();
    qf[ks] = c.bf16();
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = neg_inf();  // running max of scale*log2(e)*s over this row
  float l_run = 0.f;        // this lane's share of the sum of the bf16-rounded P (normalises O)
  float l_exact = 0.f;      // this lane's share of the sum of the fp32 P (gives LSE)

  // ---- staging of one K/V sub-tile through registers
  Chunk<F32IN> kst[KC];
  Chunk<F32IN> vst[VB][4];
  auto issue = [&](const Item& it) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int ci = tid + c * NT;
      if (KCH % NT == 0 || ci < KCH) {
        const int row = ci / DC, col = ci % DC;
        if (row < it.nk)
          kst[c].load(kp + (int64_t)(it.key0 + row) * p.k_ss + col * 8);
        else
          kst[c].zero();
      }
    }
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int bi = tid + vb * NT;
      if (VBL % NT == 0 || bi < VBL) {
        const int kg = bi / DC, dc = bi % DC;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = kg * 4 + rr;
          if (key < it.nk)
            vst[vb][rr].load(vp + (int64_t)(it.key0 + key) * p.v_ss + dc * 8);
          else
            vst[vb][rr].zero();
        }
      }
    }
  };
  auto store = [&](unsigned char* Kb, unsigned char* Vb) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int ci = tid + c * NT;
      if (KCH % NT == 0 || ci < KCH) {
        const int row = ci / DC, col = ci % DC;
        *reinterpret_cast<uint4*>(Kb + row * KROW + col * 16) = kst[c].bf16();
      }
    }
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int bi = tid + vb * NT;
      if (VBL % NT == 0 || bi < VBL) {
        const int kg = bi / DC, dc = bi % DC;
        const uint4 r0 = vst[vb][0].bf16(), r1 = vst[vb][1].bf16();
        const uint4 r2 = vst[vb][2].bf16(), r3 = vst[vb][3].bf16();
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const uint32_t x0 = word(r0, dd >> 1), x1 = word(r1, dd >> 1);
          const uint32_t x2 = word(r2, dd >> 1), x3 = word(r3, dd >> 1);
          uint2 out;
          if ((dd & 1) == 0) {
            out.x = (x0 & 0xffffu) | (x1 << 16);
            out.y = (x2 & 0xffffu) | (x3 << 16);
          } else {
            out.x = (x0 >> 16) | (x1 & 0xffff0000u);
            out.y = (x2 >> 16) | (x3 & 0xffff0000u);
          }
          *reinterpret_cast<uint2*>(Vb + (dc * 8 + dd) * VROW + kg * 8) = out;
        }
      }
    }
  };

  const int arow = swap_b23(l32);
  const float c = p.c;
  auto compute = [&](const unsigned char* Kb, const unsigned char* Vb, const Item& it) {
    f32x16_t s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(Kb + arow * KROW + ks * 32 + h32 * 16);
      const uint4 a1 =
          *reinterpret_cast<const uint4*>(Kb + (arow + 32) * KROW + ks * 32 + h32 * 16);
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
    }
    // element mask: accumulator r of lane half h32 holds key
    // 16*(r/8) + 8*h32 + r%8 (+32 for s1) of the sub-tile.  Keys at or past
    // nk (block end, sequence end, or the valid-token count) are hidden.
    const bool causal = it.is_mask && p.mask_mod == 1;
    if (causal || it.nk < KT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 16 * (r >> 3) + 8 * h32 + (r & 7);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kk = key + 32 * half;
          bool keep = kk < it.nk;
          if (causal) keep = keep && (it.key0 + kk <= qrow);
          if (!keep) {
            if (half == 0)
              s0[r] = neg_inf();
            else
              s1[r] = neg_inf();
          }
        }
      }
    }
    float mx = neg_inf();
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    uint32_t pk0[8], pk1[8];
    float ls = 0.f, le = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a0 = __builtin_amdgcn_exp2f(fmaf(s0[2 * i], c, -m_use));
      const float a1 = __builtin_amdgcn_exp2f(fmaf(s0[2 * i + 1], c, -m_use));
      const float b0 = __builtin_amdgcn_exp2f(fmaf(s1[2 * i], c, -m_use));
      const float b1 = __builtin_amdgcn_exp2f(fmaf(s1[2 * i + 1], c, -m_use));
      pk0[i] = pack_bf16x2(a0, a1);
      pk1[i] = pack_bf16x2(b0, b1);
      ls += (bf16_lo(pk0[i]) + bf16_hi(pk0[i])) + (bf16_lo(pk1[i]) + bf16_hi(pk1[i]));
      le += (a0 + a1) + (b0 + b1);
    }
    l_run = l_run * alpha + ls;
    l_exact = l_exact * alpha + le;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    // PV step ps covers keys 16*ps .. 16*ps+15; lane half h32 supplies keys
    // 16*ps + 8*h32 .. +7, which are accumulators 8*(ps%2) .. +7 of s_{ps/2}.
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const uint32_t* src = (ps < 2) ? pk0 : pk1;
      const int o = 4 * (ps & 1);
      const uint4 bop = make_uint4(src[o], src[o + 1], src[o + 2], src[o + 3]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint4 a =
            *reinterpret_cast<const uint4*>(Vb + (db * 32 + arow) * VROW + ps * 32 + h32 * 16);
        oacc[db] = mfma32(a, bop, oacc[db]);
      }
    }
  };

  // ---- list walk with a two-stage LDS pipeline
  ListWalk L{mrow, p.mi_s[3], mcnt, frow, p.fi_s[3], mcnt + fcnt, -1000000, -1};
  unsigned char* buf0 = smem;
  unsigned char* buf1 = smem + STAGE;
  Item cur{-1, 0, 0, 0, 0, 0, 0};
  bool have = advance(cur, L, lane, p.block_kv, num_n, Sk_b, p.mask_mod, p.kv_valid);
  if (have) {
    issue(cur);
    store(buf0, buf0 + KBYTES);
  }
  __syncthreads();
  Item nxt = cur;
  bool have_nxt = have && advance(nxt, L, lane, p.block_kv, num_n, Sk_b, p.mask_mod, p.kv_valid);
  int sb = 0;
  while (have) {
    if (have_nxt) issue(nxt);
    unsigned char* cb = sb ? buf1 : buf0;
    unsigned char* ob = sb ? buf0 : buf1;
    compute(cb, cb + KBYTES, cur);
    if (have_nxt) store(ob, ob + KBYTES);
    __syncthreads();
    cur = nxt;
    have = have_nxt;
    if (have) have_nxt = advance(nxt, L, lane, p.block_kv, num_n, Sk_b, p.mask_mod, p.kv_valid);
    sb ^= 1;
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l); empty rows give 0, -inf
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float l_lse = l_exact + __shfl_xor(l_exact, 32);
  if (qrow < Sq_b) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T* op = reinterpret_cast<T*>(p.o) + ooff + (int64_t)qrow * p.o_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        T* dst = op + db * 32 + 16 * half + 8 * h32;
        const int r0 = 8 * half;
        if constexpr (F32IN) {
          float4* d4 = reinterpret_cast<float4*>(dst);
          d4[0] = make_float4(oacc[db][r0] * inv, oacc[db][r0 + 1] * inv, oacc[db][r0 + 2] * inv,
                              oacc[db][r0 + 3] * inv);
          d4[1] = make_float4(oacc[db][r0 + 4] * inv, oacc[db][r0 + 5] * inv,
                              oacc[db][r0 + 6] * inv, oacc[db][r0 + 7] * inv);
        } else {
          *reinterpret_cast<uint4*>(dst) =
              make_uint4(pack_bf16x2(oacc[db][r0] * inv, oacc[db][r0 + 1] * inv),
                         pack_bf16x2(oacc[db][r0 + 2] * inv, oacc[db][r0 + 3] * inv),
                         pack_bf16x2(oacc[db][r0 + 4] * inv, oacc[db][r0 + 5] * inv),
                         pack_bf16x2(oacc[db][r0 + 6] * inv, oacc[db][r0 + 7] * inv));
        }
      }
    }
    if (h32 == 0) p.lse[lse_base + qrow] = l_lse > 0.f ? (m_run + log2f(l_lse)) * kLn2 : neg_inf();
  }
}

template <int D, int NW, bool F32>
hipError_t launch_one(const FwdParams& p, hipStream_t s) {
  FwdParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW, F32>),
                         dim3(p.num_tiles), dim3(NW * 64), args, 0, s);
}

template <int D, bool F32>
hipError_t launch_tm(const FwdParams& p, int tile_m, hipStream_t s) {
  switch (tile_m) {
    case 128: return launch_one<D, 4, F32>(p, s);
    case 64: return launch_one<D, 2, F32>(p, s);
    case 32: return launch_one<D, 1, F32>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool F32>
hipError_t launch_d(const FwdParams& p, int D, int tile_m, hipStream_t s) {
  switch (D) {
    case 64: return launch_tm<64, F32>(p, tile_m, s);
    case 96: return launch_tm<96, F32>(p, tile_m, s);
    case 128: return launch_tm<128, F32>(p, tile_m, s);
    case 192: return launch_tm<192, F32>(p, tile_m, s);
    case 256: return launch_tm<256, F32>(p, tile_m, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int D, int tile_m, bool f32_in, hipStream_t s) {
  return f32_in ? launch_d<true>(p, D, tile_m, s) : launch_d<false>(p, D, tile_m, s);
}

}  // namespace bsa
