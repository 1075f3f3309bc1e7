// Proxy-compensated route, shared by the forward kernels that take it (the
// PrimTS page, "proxy-compensated block-sparse attention", flashinfer pull
// request 4872: description, proxy paragraph).  After a Q block's listed KV
// blocks, the kernel walks the caller's block summaries 64 at a time as if
// they were keys (mean K as the key, summed V as the value).  A bitmap in LDS
// of the listed blocks masks the summaries of blocks attended exactly,
// chunks whose blocks are all listed are skipped, and the row sum counts each
// summary at its block's token mass: one softmax over exact keys and proxies.
#pragma once

#include "bsa_fwd_common.h"

namespace bsa {
namespace dev {

// LDS words of the listed-block bitmap: one bit per block, plus one word so
// that a 64-block chunk can always read two.
constexpr int kProxyBitmapWords = kProxyMaxBlocks / 32 + 1;

// Clear the bitmap and set the bits of every block on either list of the Q
// block; ends with a barrier.  All nt threads of the workgroup call it.
__device__ __forceinline__ void build_listed_bitmap(uint32_t* xbits, const FwdParams& p,
                                                    const TileInfo& ti, int tid, int nt) {
  const int nwords = (ti.num_n + 31) / 32 + 1;
  for (int i = tid; i < nwords; i += nt) xbits[i] = 0u;
  __syncthreads();
  for (int e = tid; e < ti.mcnt; e += nt) {
    const int j = ti.mrow[(int64_t)e * p.mi_s[3]];
    if ((unsigned)j < (unsigned)ti.num_n) atomicOr(&xbits[j >> 5], 1u << (j & 31));
  }
  for (int e = tid; e < ti.fcnt; e += nt) {
    const int j = ti.frow[(int64_t)e * p.fi_s[3]];
    if ((unsigned)j < (unsigned)ti.num_n) atomicOr(&xbits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
}

// Next chunk of summaries (from block pn on) holding a block that is not
// listed; marks the item with is_mask = 2.  False when none is left.
__device__ __forceinline__ bool next_proxy_chunk(const uint32_t* xbits, int num_n, int& pn,
                                                 Item& it) {
  while (pn < num_n) {
    const int n0 = pn;
    pn += kKvTile;
    const int nk = min(kKvTile, num_n - n0);
    const uint64_t live = nk >= 64 ? ~0ull : ((1ull << nk) - 1);
    // the bitmap is the same for every lane: scalar copies keep the item
    // (and the DMA base address built from it) wave-uniform
    const uint32_t w0 = __builtin_amdgcn_readfirstlane(xbits[n0 >> 5]);
    const uint32_t w1 = __builtin_amdgcn_readfirstlane(xbits[(n0 >> 5) + 1]);
    const uint64_t ex = (uint64_t)w0 | ((uint64_t)w1 << 32);
    if ((~ex & live) == 0) continue;  // every block of the chunk is listed
    it.key0 = n0;
    it.nk = nk;
    it.is_mask = 2;
    return true;
  }
  return false;
}

// softmax_step for the kernels that carry the route (no element mask): one
// body for both kinds of item, so that only one copy is inlined.  A proxy
// item (is_mask == 2) holds summaries n0 .. n0+nk-1 (n0 = it.key0, a
// multiple of 64); a set bit n of the bitmap means block n is listed and its
// summary is masked, and the row sum adds mass(n) * p, where mass(n) is
// block_kv for every block but the last, whose mass is its true length.  An
// exact item takes weight 1 and no bitmap, which is softmax_step's
// arithmetic.  The PV product takes p as is.  As in softmax_step, l sums the
// fp32 p (the LSE) and lo the bf16 p of the PV product (the normaliser of
// O), both with the same mass weights.
template <int DB>
__device__ __forceinline__ void softmax_step_any(f32x16_t& s0, f32x16_t& s1, const Item& it,
                                                 const uint32_t* xbits, int block_kv, int num_n,
                                                 int Sk, int h32, float c, float& m_run,
                                                 float& l_run, float& lo_run,
                                                 f32x16_t (&oacc)[DB], uint32_t (&pk0)[8],
                                                 uint32_t (&pk1)[8]) {
  const bool px = it.is_mask == 2;
  if (px || it.nk < kKvTile) {
    const uint32_t ex0 = px ? xbits[it.key0 >> 5] : 0u;
    const uint32_t ex1 = px ? xbits[(it.key0 >> 5) + 1] : 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 16 * (r >> 3) + 8 * h32 + (r & 7);
      if (!(key < it.nk && ((ex0 >> key) & 1u) == 0)) s0[r] = neg_inf();
      if (!(key + 32 < it.nk && ((ex1 >> key) & 1u) == 0)) s1[r] = neg_inf();
    }
  }
  // row max: 32 values, a tree of 3-input maxes (v_max3_f32)
  float t[11];
#pragma unroll
  for (int i = 0; i < 5; ++i) t[i] = fmaxf(fmaxf(s0[3 * i], s0[3 * i + 1]), s0[3 * i + 2]);
#pragma unroll
  for (int i = 0; i < 5; ++i) t[5 + i] = fmaxf(fmaxf(s1[3 * i], s1[3 * i + 1]), s1[3 * i + 2]);
  t[10] = fmaxf(s0[15], s1[15]);
  float mx = fmaxf(fmaxf(fmaxf(fmaxf(t[0], t[1]), t[2]), fmaxf(fmaxf(t[3], t[4]), t[5])),
                   fmaxf(fmaxf(fmaxf(t[6], t[7]), t[8]), fmaxf(t[9], t[10])));
  mx = half_swap_max(mx);
  const float m_new = fmaxf(m_run, mx * c);
  if (__any(m_new > m_run)) {
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= alpha;
    lo_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == neg_inf()) ? 0.f : m_run;
  // p of the last block's summary, in fp32 (lt) and as rounded for the PV
  // product (lto).  Only the chunk that holds it does this (a wave-uniform
  // branch): chunk-local key tk is element 8 * ((tk >> 4) & 1) + (tk & 7) of
  // s0 (tk < 32) or s1, in the lanes of half (tk >> 3) & 1.
  float lt = 0.f, lto = 0.f;
  const int tk = num_n - 1 - it.key0;
  if (px && tk < kKvTile) {
    const int e = 8 * ((tk >> 4) & 1) + (tk & 7);
    float sv = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (r == e) sv = (tk & 32) ? s1[r] : s0[r];
    if (((tk >> 3) & 1) == h32) {
      lt = __builtin_amdgcn_exp2f(fmaf(sv, c, -m_use));
      lto = __uint_as_float(pack_bf16x2(lt, 0.f) << 16);
    }
  }
  float ls = 0.f, lo = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a0 = __builtin_amdgcn_exp2f(fmaf(s0[2 * i], c, -m_use));
    const float a1 = __builtin_amdgcn_exp2f(fmaf(s0[2 * i + 1], c, -m_use));
    const float b0 = __builtin_amdgcn_exp2f(fmaf(s1[2 * i], c, -m_use));
    const float b1 = __builtin_amdgcn_exp2f(fmaf(s1[2 * i + 1], c, -m_use));
    pk0[i] = pack_bf16x2(a0, a1);
    pk1[i] = pack_bf16x2(b0, b1);
    ls += (a0 + a1) + (b0 + b1);
    lo = add_bf16x2(pk1[i], add_bf16x2(pk0[i], lo));
  }
  const float wf = px ? (float)block_kv : 1.f;
  const float wt = px ? (float)(Sk - (num_n - 1) * block_kv) : 1.f;
  l_run += fmaf(wt - wf, lt, wf * ls);
  lo_run += fmaf(wt - wf, lto, wf * lo);
}

}  // namespace dev
}  // namespace bsa
