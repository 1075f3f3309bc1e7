// Device-side pieces shared by the two forward kernels (gfx950, wave64):
// work-tile decode, the block-list walk, the online-softmax step on the
// transposed MFMA accumulators, and the epilogue.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16).  Each wave owns 32 query rows and
// computes everything transposed:
//     S^T[key, q] = K[key, :] . Q[q, :]          (A = K from LDS, B = Q in registers)
//     O^T[d, q]  += V^T[d, key] . P^T[key, q]    (A = V^T from LDS, B = P^T in registers)
// so every accumulator register of a lane belongs to the same query
// (q = lane % 32): the row max needs one exchange between lanes l and l^32
// per sub-tile, the running sum none until the epilogue, and the O rescale
// is a per-lane scalar.  Accumulator r of lane half h = lane / 32 holds row
// 8*(r/4) + 4*h + r%4 of the 32-row block.  The A operand's row i is fetched
// from key (or head-dim) swap_b23(i) (bits 2 and 3 of i exchanged), so the
// 16 rows a lane receives are two runs of 8 consecutive keys (head dims):
// 16*(r/8) + 8*h + r%8.  P^T then feeds the PV MFMA straight from registers
// and O is written in 16-byte pieces.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_internal.h"

namespace bsa {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kMaskNone = 0, kMaskCausal = 1, kMaskKvValid = 2, kMaskLocal = 3;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed pair of bf16 values (v_dot2c_f32_bf16 against
// (1, 1)): sums exactly the P that feeds the PV product.
__device__ __forceinline__ float add_bf16x2(uint32_t pk, float acc) {
  const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), one, acc, false);
}

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Row permutation of the MFMA A operand: exchange bits 2 and 3.
__device__ __forceinline__ int swap_b23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Workgroups are dispatched round-robin over the 8 XCDs.  Renumber them so
// that each XCD receives one contiguous range of logical tiles: the Q tiles
// of one (batch, head) then share that XCD's L2 for their K/V blocks.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd, local = bid / kXcd;
  const int per = G / kXcd, rem = G % kXcd;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// What one workgroup works on: rows [q0, min(q0 + TM, qend)) of one
// (sequence, head), qend being the end of their sparse Q block (clipped to
// the sequence), and the block-list row of that Q block.
struct TileInfo {
  int h, q0, qend, Sq, Sk, num_n;
  const int32_t* kvv;  // valid-token counts of this sequence's KV blocks (or null)
  int64_t qoff, koff, voff, ooff, lse_base;  // element offsets of row 0 / LSE row 0 (head h)
  int64_t lse_hs;                              // LSE elements between two heads
  const int32_t* mrow;
  const int32_t* frow;
  int mcnt, fcnt;
};

// Varlen work order: Q block of rank q (0 <= q < total_m_blocks) in the
// order "block index within its sequence descending, then sequence
// ascending", so the blocks late in long sequences, which list the most KV
// blocks under a causal mask, are dispatched first and the short ones fill
// the tail.  With C(L) = sum_b max(0, num_m(b) - L) blocks at local index >=
// L, rank q lies at the level L where C(L+1) <= q < C(L) (binary search over
// L), and is the (q - C(L+1))-th sequence, counted from b = 0, that has a
// block at index L.  O(B log total_m) reads of cu_total_m_blocks.
__device__ __forceinline__ int blocks_at_or_above(const FwdParams& p, int L) {
  int c = 0;
  for (int b = 0; b < p.B; ++b) c += max(0, (p.cu_m[b + 1] - p.cu_m[b]) - L);
  return c;
}

__device__ __forceinline__ void varlen_block_by_rank(const FwdParams& p, int q, int& b, int& m) {
  int lo = 0, hi = p.total_m - 1;  // the largest L with C(L) > q
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (blocks_at_or_above(p, mid) > q)
      lo = mid;
    else
      hi = mid - 1;
  }
  int k = q - blocks_at_or_above(p, lo + 1);
  b = 0;
  for (int s = 0; s < p.B; ++s) {
    if (p.cu_m[s + 1] - p.cu_m[s] > lo) {
      if (k == 0) {
        b = s;
        break;
      }
      --k;
    }
  }
  m = lo;
}

// The two list lengths of a tile's Q-block row (an absent list has none),
// fetched together when both lists are given.
__device__ __forceinline__ void load_counts(const FwdParams& p, int64_t mo, int64_t fo,
                                            TileInfo& ti) {
  if (p.mcnt && p.fcnt) {
    ti.mcnt = p.mcnt[mo];
    ti.fcnt = p.fcnt[fo];
  } else if (p.mcnt) {
    ti.mcnt = p.mcnt[mo];
  } else if (p.fcnt) {
    ti.fcnt = p.fcnt[fo];
  }
}

// The same lookup for B < 64 sequences, one per lane: Q block q of the work
// order (rank q of the longest-first order when p.lpt, else global Q block
// q) -> sequence b, its local block m, global block mg, and the sequence's
// token and list-slot bounds.  Every lane loads entry `lane` of the four
// bookkeeping arrays at once; the level search evaluates C(L) for 64 levels
// per pass (lane = level), and ballots pick the sequence.  Same results as
// varlen_block_by_rank and the binary search over cu_total_m_blocks.
__device__ __forceinline__ void varlen_seq_lookup(const FwdParams& p, int q, int& b, int& m,
                                                  int& mg, int& sq0, int& sq1, int& sk0,
                                                  int& sk1, int& boff) {
  const int lane = (int)(threadIdx.x & 63);
  const bool in = lane <= p.B;
  const int cm = in ? p.cu_m[lane] : 0;
  const int cm1 = lane < p.B ? p.cu_m[lane + 1] : cm;
  const int cq = in ? p.cu_q[lane] : 0;
  const int ck = in ? p.cu_k[lane] : 0;
  const int bo = in ? p.blk_off[lane] : 0;
  const int nm = lane < p.B ? cm1 - cm : 0;  // Q blocks of sequence `lane`
  if (p.lpt) {
    // the largest level L with C(L) > q, C(L) = sum_s max(0, nm_s - L):
    // C(0) = total_m > q, and C is non-increasing, so the levels with C > q
    // are a prefix
    int L = 0;
    for (int c0 = 0;; c0 += 64) {
      int cl = 0;
      for (int s = 0; s < p.B; ++s) cl += max(0, __builtin_amdgcn_readlane(nm, s) - (c0 + lane));
      const int n_above = __popcll(__ballot(cl > q));
      if (n_above < 64) {
        L = c0 + n_above - 1;
        break;
      }
    }
    int c_next = 0;  // C(L + 1)
    for (int s = 0; s < p.B; ++s) c_next += max(0, __builtin_amdgcn_readlane(nm, s) - (L + 1));
    // the k-th sequence, counted from b = 0, that has a block at level L
    const int k = q - c_next;
    const uint64_t has = __ballot(nm > L);
    const int before = __popcll(has & ((1ull << lane) - 1ull));
    const uint64_t pick = __ballot(((has >> lane) & 1ull) != 0 && before == k);
    b = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)pick) - 1);
    m = L;
    mg = __builtin_amdgcn_readlane(cm, b) + m;
  } else {
    // the last sequence whose first global block is <= q (cu_m is non-decreasing)
    const uint64_t le = __ballot(lane < p.B && cm <= q);
    b = __builtin_amdgcn_readfirstlane(63 - __clzll((long long)le));
    mg = q;
    m = q - __builtin_amdgcn_readlane(cm, b);
  }
  sq0 = __builtin_amdgcn_readlane(cq, b);
  sq1 = __builtin_amdgcn_readlane(cq, b + 1);
  sk0 = __builtin_amdgcn_readlane(ck, b);
  sk1 = __builtin_amdgcn_readlane(ck, b + 1);
  boff = __builtin_amdgcn_readlane(bo, b);
}

// Logical tile t -> TileInfo.  A tile holds TM rows: R = TM / gpack rows
// of each of gpack consecutive Q heads h .. h + gpack - 1 (gpack > 1 packs
// the Q heads of one KV head, which then share their lists).  A sparse Q
// block of block_q rows is covered by qsub = ceil(block_q / R) tiles; tile
// sub of Q block i starts at row i*block_q + sub*R and its rows stop at the
// block end, so a block of any size (112, 80, 48 rows ...) is fitted rather
// than rejected (runguoli.com "FlashAttention - CuTe Kernels & Block
// Sparsity", the tile-fit change).
// Batched: t = ((b*H/gpack + h/gpack) * tiles_per_head + qt), qt = i*qsub + sub.
// Varlen (flash-attention PR #2224 layout): t = (h/gpack) * tiles_per_head + tm
// with tm = Q block * qsub + sub; the sequence is the largest b with
// cu_total_m_blocks[b] <= Q block (binary search), the list row starts at
// block_idx_offsets[b] + m * num_n(b).  The list head is h, or its KV head
// h / hrep when the lists are given per KV head.  Returns false when the
// tile holds no row of its sequence (the whole workgroup then exits).
// VL: 0 batched, 1 varlen (compile-time: the other layout's code is not in
// the kernel), 2 taken from p.varlen at run time.
template <int TM, int VL = 2>
__device__ __forceinline__ bool decode_tile(const FwdParams& p, int t, TileInfo& ti) {
  ti.mrow = nullptr;
  ti.frow = nullptr;
  ti.mcnt = ti.fcnt = 0;
  const int R = TM / p.gpack, HG = p.H / p.gpack;
  const bool varlen = VL == 2 ? p.varlen != 0 : VL == 1;
  if (!varlen) {
    const int qt = t % p.tiles_per_head;
    const int bh = t / p.tiles_per_head;
    const int h = (bh % HG) * p.gpack, b = bh / HG, hk = h / p.hrep;
    const int lh = p.kvh_lists ? hk : h;
    const int i = qt / p.qsub, sub = qt % p.qsub;
    ti.h = h;
    ti.q0 = i * p.block_q + sub * R;
    ti.qend = min(p.Sq, min(i * p.block_q + p.block_q, ti.q0 + R));
    if (ti.q0 >= ti.qend) return false;
    ti.Sq = p.Sq;
    ti.Sk = p.Sk;
    ti.num_n = cdiv(p.Sk, p.block_kv);
    ti.kvv = p.kv_valid;
    ti.qoff = b * p.q_sb + h * p.q_sh;
    ti.koff = b * p.k_sb + hk * p.k_sh;
    ti.voff = b * p.v_sb + hk * p.v_sh;
    ti.ooff = b * p.o_sb + h * p.o_sh;
    ti.lse_base = (int64_t)(b * p.H + h) * p.Sq;
    ti.lse_hs = p.Sq;
    load_counts(p, b * p.mc_s[0] + lh * p.mc_s[1] + i * p.mc_s[2],
                b * p.fc_s[0] + lh * p.fc_s[1] + i * p.fc_s[2], ti);
    if (p.mcnt) ti.mrow = p.midx + b * p.mi_s[0] + lh * p.mi_s[1] + i * p.mi_s[2];
    if (p.fcnt) ti.frow = p.fidx + b * p.fi_s[0] + lh * p.fi_s[1] + i * p.fi_s[2];
  } else {
    const int tm = t % p.tiles_per_head;
    const int h = (t / p.tiles_per_head) * p.gpack;
    const int sub = tm % p.qsub;
    int b, m, mg, sq0, sq1, sk0, sk1, boff;
    if (p.B < 64) {
      // one sequence per lane: its bookkeeping arrives in one round of loads,
      // and the search below runs on registers and ballots
      varlen_seq_lookup(p, tm / p.qsub, b, m, mg, sq0, sq1, sk0, sk1, boff);
    } else {
      if (p.lpt) {
        varlen_block_by_rank(p, tm / p.qsub, b, m);
      } else {
        const int mq = tm / p.qsub;
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (p.cu_m[mid] <= mq)
            lo = mid;
          else
            hi = mid - 1;
        }
        b = lo;
        m = mq - p.cu_m[b];
      }
      mg = p.cu_m[b] + m;
      sq0 = p.cu_q[b];
      sq1 = p.cu_q[b + 1];
      sk0 = p.cu_k[b];
      sk1 = p.cu_k[b + 1];
      boff = p.blk_off[b];
    }
    const int hk = h / p.hrep;
    const int lh = p.kvh_lists ? hk : h;
    ti.h = h;
    ti.Sq = sq1 - sq0;
    ti.Sk = sk1 - sk0;
    ti.num_n = cdiv(ti.Sk, p.block_kv);
    ti.q0 = m * p.block_q + sub * R;
    if (m < 0 || m >= cdiv(ti.Sq, p.block_q)) return false;
    ti.qend = min(ti.Sq, min(m * p.block_q + p.block_q, ti.q0 + R));
    if (ti.q0 >= ti.qend) return false;
    // valid-token counts: row b of a [B, kv_valid_ld] array (ld 0: one row for all)
    ti.kvv = p.kv_valid != nullptr ? p.kv_valid + (int64_t)b * p.kvv_ld : nullptr;
    const int64_t row_p = (int64_t)boff + (int64_t)m * ti.num_n;
    if (row_p < 0 || row_p + ti.num_n > p.total_n) return false;  // inconsistent bookkeeping
    ti.qoff = (int64_t)sq0 * p.q_ss + h * p.q_sh;
    ti.koff = (int64_t)sk0 * p.k_ss + hk * p.k_sh;
    ti.voff = (int64_t)sk0 * p.v_ss + hk * p.v_sh;
    ti.ooff = (int64_t)sq0 * p.o_ss + h * p.o_sh;
    ti.lse_base = (int64_t)h * p.lse_ld + sq0;
    ti.lse_hs = p.lse_ld;
    load_counts(p, lh * p.mc_s[1] + mg * p.mc_s[2], lh * p.fc_s[1] + mg * p.fc_s[2], ti);
    if (p.mcnt) ti.mrow = p.midx + lh * p.mi_s[1] + row_p * p.mi_s[3];
    if (p.fcnt) ti.frow = p.fidx + lh * p.fi_s[1] + row_p * p.fi_s[3];
  }
  ti.mcnt = min(max(ti.mcnt, 0), ti.num_n);
  ti.fcnt = min(max(ti.fcnt, 0), ti.num_n);
  return true;
}

// Concatenated (mask ++ full) block list of one Q-block row.  Entries are
// fetched 64 at a time, one per lane, together with the number of leading
// keys of that block that can be visible (the block size; for a mask-list
// block under the valid-count mask_mod its valid-token count; 0 for ids
// outside [0, num_n)), and broadcast with readlane.
struct ListWalk {
  const int32_t* mrow;
  int64_t ms;
  int mcnt;
  const int32_t* frow;
  int64_t fs;
  int total;
  int bk, num_n, mask_mod;
  const int32_t* kv_valid;
  int base;
  int chunk_j, chunk_len;

  // issue the loads of entries g .. g + 63 (one per lane)
  __device__ __forceinline__ void fetch(int g, int lane) {
    base = g;
    const int gg = g + lane;
    int j = -1;
    if (gg < mcnt)
      j = mrow[gg * ms];
    else if (gg < total)
      j = frow[(gg - mcnt) * fs];
    chunk_j = j;
  }
  // the visible lengths of the fetched entries (waits for them)
  __device__ __forceinline__ void lengths(int lane) {
    const int gg = base + lane, j = chunk_j;
    int len = 0;
    if (gg < total && j >= 0 && j < num_n) {
      len = bk;
      if (mask_mod == kMaskKvValid && gg < mcnt) len = min(bk, kv_valid[j]);
    }
    chunk_len = len;
  }
  __device__ __forceinline__ void load(int g, int lane) {
    fetch(g, lane);
    lengths(lane);
  }
  __device__ __forceinline__ void entry(int g, int lane, int& j, int& len) {
    if (g < base || g >= base + 64) load(g, lane);
    j = __builtin_amdgcn_readlane(chunk_j, g - base);
    len = __builtin_amdgcn_readlane(chunk_len, g - base);
  }
};

// One unit of work: sub-tile st (kKvTile keys) of the KV block listed at
// position g; its keys [key0, key0 + nk) are the ones that can be visible.
struct Item {
  int g, st, j, blen, key0, nk, is_mask;
  // packed items (advance_packed): item key r < nk is sequence key r + d_s,
  // s = (r >= e0) + (r >= e1) + (r >= e2); unused ends are kKvTile
  int e0, e1, e2, d0, d1, d2, d3;
};

// Route packing (the PrimTS page's fixed-width physical routes, here 64
// keys): the visible keys of consecutive listed blocks (the block size
// clipped to the sequence, and for a mask-list block under the valid-count
// mask_mod to its count) are packed into 64-key items of up to kPackSeg
// contiguous runs, so a block of 112, 80 or 16 keys leaves no MFMA slot
// empty except at the end of the list.  Runs from mask-list blocks under
// the causal mask are marked in bit s of it.is_mask, and the element mask
// tests their keys (softmax_step with SEG).  it.g / it.st hold the list
// position and the keys of block it.g already taken; it.j / it.blen that
// block's id and visible length.  Returns false past the end.
constexpr int kPackSeg = 4;

__device__ __forceinline__ bool advance_packed(Item& it, ListWalk& L, int lane, int Sk,
                                               bool causal_mask_list) {
  // The item's runs are the next (up to kPackSeg) list entries with a visible
  // key, the first one possibly part-taken.  They are found in the lanes that
  // hold the fetched entries (a ballot of the entries with keys left) and
  // read out with readlane; the run lengths are a running sum capped at 64.
  int first = (it.g >= 0 && it.st < it.blen) ? it.g : it.g + 1;
  int pos0 = first == it.g ? it.st : 0;
  uint64_t nz = 0;
  int av = 0;
  while (true) {
    if (first >= L.total) return false;  // past the end (the walk is not called again)
    // keep at least kPackSeg entries from `first` in the fetched window
    if (first < L.base || (first + kPackSeg > L.base + 64 && L.base + 64 < L.total))
      L.load(first, lane);
    const int rel = L.base + lane - first;  // candidate order of this lane's entry
    const int vis = max(0, min(L.chunk_len, Sk - L.chunk_j * L.bk));
    av = (rel >= 0 && L.base + lane < L.total) ? vis - (rel == 0 ? pos0 : 0) : 0;
    nz = __ballot(av > 0);
    if (nz != 0) break;
    // no visible key left in the window
    first = L.base + 64;
    pos0 = 0;
  }
  int nk = 0, cmask = 0, last_lane = 0, last_end = 0, last_vis = 0, last_j = 0;
  int d0 = 0, d1 = 0, d2 = 0, d3 = 0, e0 = kKvTile, e1 = kKvTile, e2 = kKvTile;
  // (unrolled, and no arrays: d and e stay in registers)
#pragma unroll
  for (int s = 0; s < kPackSeg; ++s) {
    if (nz != 0 && nk < kKvTile) {
      const int pl = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)nz) - 1);
      nz &= nz - 1;
      const int a = __builtin_amdgcn_readlane(av, pl);
      const int j = __builtin_amdgcn_readlane(L.chunk_j, pl);
      const int g = L.base + pl;
      const int start = g == first ? pos0 : 0;
      const int t = min(kKvTile - nk, a);
      const int dd = j * L.bk + start - nk;  // sequence key = item key + dd over this run
      if (s == 0) d0 = dd;
      if (s == 1) d1 = dd;
      if (s == 2) d2 = dd;
      if (s == 3) d3 = dd;
      if (causal_mask_list && g < L.mcnt) cmask |= 1 << s;
      last_lane = pl;
      last_end = start + t;
      last_vis = start + a;
      last_j = j;
      nk += t;
      if (nk < kKvTile) {  // the run ends inside the item
        if (s == 0) e0 = nk;
        if (s == 1) e1 = nk;
        if (s == 2) e2 = nk;
      }
    }
  }
  it.g = L.base + last_lane;
  it.st = last_end;
  it.j = last_j;
  it.blen = last_vis;
  it.nk = nk;
  it.key0 = d0;
  it.is_mask = cmask;
  it.e0 = e0;
  it.e1 = e1;
  it.e2 = e2;
  it.d0 = d0;
  it.d1 = d1;
  it.d2 = d2;
  it.d3 = d3;
  return true;
}

__device__ __forceinline__ bool advance(Item& it, ListWalk& L, int lane, int Sk) {
  int g = it.g, st = it.st + 1, j = it.j, blen = it.blen;
  while (true) {
    if (g >= 0 && st * kKvTile < blen) {
      const int key0 = j * L.bk + st * kKvTile;
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
    L.entry(g, lane, j, blen);
  }
}

// Cap on a lane's sum of P in the 256-row kernel's lazy running max.
constexpr float kSumCap = 65536.f;

// max over the two lane halves (lanes l and l ^ 32).  v_permlane32_swap
// trades the upper half of its first operand for the lower half of its
// second, so with x in both, one result holds x of the lower half in every
// lane and the other x of the upper half (no LDS round trip, unlike a
// shuffle through ds_bpermute).  The two results are copied out as scalars
// before the cast: a __builtin_bit_cast of a vector element reads the
// vector's first element, whatever the index.
__device__ __forceinline__ float half_swap_max(float x) {
  const uint32_t a = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const uint32_t lo = r[0], hi = r[1];
  return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

// Bits [max(lo, 0), min(hi, 63)] of a 64-bit mask (zero when empty).
__device__ __forceinline__ uint64_t key_bits(int lo, int hi) {
  lo = max(lo, 0);
  hi = min(hi, 63);
  if (hi < lo) return 0ull;
  const uint64_t upto = hi >= 63 ? ~0ull : (1ull << (hi + 1)) - 1;
  return upto & ~((1ull << lo) - 1);
}

// x - base clamped to [-1, 64] (computed in 64 bits: x may be an unbounded
// INT_MAX or a far negative window end, base negative): an item position
// for key_bits.
__device__ __forceinline__ int item_offset(int x, int base) {
  const int64_t v = (int64_t)x - base;
  return (int)(v < -1 ? -1 : v > kKvTile ? kKvTile : v);
}

// Online-softmax step for one 64-key sub-tile.  s0/s1 hold S^T for keys
// 0..31 / 32..63 of the sub-tile (raw dot products).  Applies the element
// mask, updates the running max m (base-2 units of scale*s), the running sum
// l of the fp32 P (for the LSE) and the running sum lo of P rounded to bf16
// (the P the PV product takes, so O = acc / lo weighs its rows by exactly
// those weights), rescales O only when some row's max grew, and returns P
// rounded to bf16 in pk0/pk1 (pairs of consecutive accumulators).
// masked: a mask-list sub-tile under the causal (RANGE false) or local
// (RANGE true) mask_mod; its kept keys of this lane's row are key <= mhi
// (causal: mhi = qrow) or mlo <= key <= mhi (local, absolute ids;
// row_key_range gives them).  The valid-count mask is already in it.nk.
// SEG: a packed item (advance_packed); bit s of it.is_mask marks run s as
// causal-masked, and item key k is sequence key k + d_s of its run s.
template <int DB, bool RANGE = false, bool SEG = false>
__device__ __forceinline__ void softmax_step(f32x16_t& s0, f32x16_t& s1, const Item& it,
                                             bool masked, int mlo, int mhi, int h32, float c,
                                             float& m_run, float& l_run, float& lo_run,
                                             f32x16_t (&oacc)[DB], uint32_t (&pk0)[8],
                                             uint32_t (&pk1)[8]) {
  if (masked || it.nk < kKvTile) {
    // the item's kept keys for this lane's row as bits of the lane's keys
    // (one bit test per element instead of a chain of compares): bit
    // 16*(r >> 3) + (r & 7) of the low (s0) and high (s1) words for
    // accumulator r
    uint64_t kb;
    if constexpr (SEG) {
      // runs [0, e0), [e0, e1), [e1, e2), [e2, nk): item key k of run s is
      // sequence key k + d_s; a run marked causal keeps k + d_s <= mhi
      auto run = [&](int a, int e, int d, int s) {
        int last = e - 1;
        if (masked && ((it.is_mask >> s) & 1)) last = min(last, item_offset(mhi, d));
        return key_bits(a, last);
      };
      kb = run(0, min(it.e0, it.nk), it.d0, 0) | run(it.e0, min(it.e1, it.nk), it.d1, 1) |
           run(it.e1, min(it.e2, it.nk), it.d2, 2) | run(it.e2, it.nk, it.d3, 3);
    } else {
      // [lo, hi]: within the visible count and, on a masked item, the row's
      // key range
      int lo = 0, hi = it.nk - 1;
      if (masked) {
        hi = min(hi, item_offset(mhi, it.key0));
        if constexpr (RANGE) lo = max(lo, item_offset(mlo, it.key0));
      }
      kb = key_bits(lo, hi);
    }
    {
      const uint64_t lm = kb >> (8 * h32);
      const uint32_t b0 = (uint32_t)lm, b1 = (uint32_t)(lm >> 32);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int bit = 16 * (r >> 3) + (r & 7);
        if (((b0 >> bit) & 1u) == 0) s0[r] = neg_inf();
        if (((b1 >> bit) & 1u) == 0) s1[r] = neg_inf();
      }
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
  l_run += ls;
  lo_run += lo;
}

// Keys [lo, hi] of row qrow that the causal (kMaskCausal: key <= qrow) or
// local (kMaskLocal: qrow - wl <= key <= qrow + wr, a negative bound
// unbounded) mask_mod keeps; [0, INT_MAX] for the others.
__device__ __forceinline__ void row_key_range(int mask_mod, int wl, int wr, int qrow, int& lo,
                                              int& hi) {
  lo = 0;
  hi = 0x7fffffff;
  if (mask_mod == kMaskCausal) {
    hi = qrow;
  } else if (mask_mod == kMaskLocal) {
    if (wl >= 0) lo = qrow - wl;
    if (wr >= 0) hi = qrow + min(wr, 0x7fffffff - qrow);
  }
}

// B operand of PV step ps (keys 16*ps .. 16*ps+15): lane half h32 supplies
// keys 16*ps + 8*h32 .. +7, i.e. accumulators 8*(ps%2) .. +7 of s_{ps/2}.
__device__ __forceinline__ uint4 p_operand(const uint32_t (&pk0)[8], const uint32_t (&pk1)[8],
                                           int ps) {
  const uint32_t* src = (ps < 2) ? pk0 : pk1;
  const int o = 4 * (ps & 1);
  return make_uint4(src[o], src[o + 1], src[o + 2], src[o + 3]);
}

// O = acc / lo (0 when lo == 0), LSE = ln2 * (m + log2 l) (-inf when l == 0):
// l sums the fp32 P, lo the normaliser of O (the bf16 P of the PV product).
template <int DB, typename T>
__device__ __forceinline__ void epilogue(const FwdParams& p, const TileInfo& ti, int qrow, int h32,
                                         float m_run, float l_run, float lo_run,
                                         const f32x16_t (&oacc)[DB]) {
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float lo_tot = lo_run + __shfl_xor(lo_run, 32);
  if (qrow >= ti.qend) return;
  const float inv = lo_tot > 0.f ? 1.f / lo_tot : 0.f;
  T* op = reinterpret_cast<T*>(p.o) + ti.ooff + (int64_t)qrow * p.o_ss;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      T* dst = op + db * 32 + 16 * half + 8 * h32;
      const int r0 = 8 * half;
      if constexpr (sizeof(T) == 4) {
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
  if (h32 == 0) p.lse[ti.lse_base + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : neg_inf();
}

}  // namespace dev
}  // namespace bsa
