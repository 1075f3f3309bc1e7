// Metadata kernels for gfx950: dense block mask or packed bitmap -> block
// lists (batched and packed varlen rows), the split of logical KV blocks into child tiles, and
// the full / partial classification of blocks under an element mask_mod.
//
// mask -> index follows the conversion "Dense FlashAttention vs Block-Sparse
// Attention" (section 2) describes: per Q-block row, the selected KV-block
// ids in descending order, then -1.  One wave compacts one row: lanes take
// 64 columns at a time from the top, a ballot gives the selected set and
// the popcount of the lower lanes' bits gives each id its slot, so the
// result is deterministic and bit-exact.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kWavesPerBlock = 4;

// sel(col) says whether KV block col of the row is selected.
template <class Sel>
__device__ __forceinline__ void compact_row_by(Sel sel_of, int N, int32_t* __restrict__ irow,
                                               int32_t* __restrict__ cnt, int lane) {
  int run = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < N; c0 += 64) {
    const int col = N - 1 - (c0 + lane);
    const bool sel = col >= 0 && sel_of(col);
    const uint64_t bal = __ballot(sel);
    if (sel) irow[run + __popcll(bal & below)] = col;
    run += __popcll(bal);
  }
  for (int s = run + lane; s < N; s += 64) irow[s] = -1;
  if (lane == 0) *cnt = run;
}

__device__ __forceinline__ void compact_row(const uint8_t* __restrict__ mrow, int N,
                                            int32_t* __restrict__ irow, int32_t* __restrict__ cnt,
                                            int lane) {
  compact_row_by([&](int col) { return mrow[col] != 0; }, N, irow, cnt, lane);
}

// Packed bitmap rows [B, Hkv, M, W] (W = ceil(N/32)): bit j of word w selects
// KV block 32*w + j; bits at or past N are never tested.  Q head h of the
// output reads KV head h / group.
__global__ __launch_bounds__(64 * kWavesPerBlock) void bitmask_to_index_kernel(
    const uint32_t* __restrict__ words, int64_t rows, int32_t H, int32_t group, int32_t M,
    int32_t N, int32_t W, int32_t* __restrict__ cnt, int32_t* __restrict__ idx) {
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t bh = row / M;
  const int32_t m = (int32_t)(row - bh * M);
  const int64_t b = bh / H;
  const int32_t h = (int32_t)(bh - b * H);
  const uint32_t* __restrict__ wrow = words + ((b * (H / group) + h / group) * M + m) * W;
  compact_row_by([&](int col) { return ((wrow[col >> 5] >> (col & 31)) & 1u) != 0; }, N,
                 idx + row * N, cnt + row, lane);
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void mask_to_index_kernel(
    const uint8_t* __restrict__ mask, int64_t rows, int32_t N, int32_t* __restrict__ cnt,
    int32_t* __restrict__ idx) {
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  compact_row(mask + row * N, N, idx + row * N, cnt + row, lane);
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void varlen_mask_to_index_kernel(
    const uint8_t* __restrict__ mask, int32_t H, int32_t B, const int32_t* __restrict__ cu_m,
    const int32_t* __restrict__ off, int32_t total_m, int32_t total_n, int32_t* __restrict__ cnt,
    int32_t* __restrict__ idx) {
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)H * total_m) return;
  const int h = (int)(row / total_m);
  const int mg = (int)(row % total_m);
  int lo = 0, hi = B - 1;  // largest b with cu_m[b] <= mg
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_m[mid] <= mg)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int b = lo;
  const int nm = cu_m[b + 1] - cu_m[b];
  const int m = mg - cu_m[b];
  if (nm <= 0 || m < 0 || m >= nm) return;
  const int64_t span = (int64_t)off[b + 1] - off[b];
  const int nn = (int)(span / nm);
  const int64_t start = (int64_t)off[b] + (int64_t)m * nn;
  if (nn < 0 || start < 0 || start + nn > total_n) return;
  const int64_t base = (int64_t)h * total_n + start;
  compact_row(mask + base, nn, idx + base, cnt + (int64_t)h * total_m + mg, lane);
}

__global__ __launch_bounds__(256) void expand_kv_blocks_kernel(
    const uint8_t* __restrict__ bm, const int32_t* __restrict__ bv, int32_t R, int32_t NL,
    int32_t f, int32_t child, uint8_t* __restrict__ full, uint8_t* __restrict__ part,
    int32_t* __restrict__ kvv) {
  const int64_t ncols = (int64_t)NL * f;
  const int64_t n = (int64_t)R * ncols;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n || x < ncols;
       x += stride) {
    if (x < ncols) {
      const int j = (int)(x / f), s = (int)(x % f);
      kvv[x] = min(max(bv[j] - s * child, 0), child);
    }
    if (x < n) {
      const int64_t r = x / ncols;
      const int jc = (int)(x % ncols);
      const int j = jc / f, s = jc % f;
      const int sz = min(max(bv[j] - s * child, 0), child);
      const bool sel = bm[r * NL + j] != 0;
      full[x] = (sel && sz == child) ? 1 : 0;
      part[x] = (sel && sz > 0 && sz < child) ? 1 : 0;
    }
  }
}

// Full / partial / empty class of block (m, n) under an element mask_mod
// (the role of flash-attention's compute_block_sparsity).  Causal and local
// masks keep a cell by the difference d = row - col alone: causal keeps
// d >= 0, local keeps -wr <= d <= wl (a negative bound is unbounded).  Over
// the block's rows [r0, r1) and columns [c0, c1) the differences are every
// integer in [r0 - (c1 - 1), (r1 - 1) - c0], so the block is full when that
// range lies inside the kept one and empty when the two do not meet.  The
// valid-count mask keeps the first kv_valid[n] columns of KV block n.
__global__ __launch_bounds__(256) void block_sparsity_kernel(
    int32_t mm, int32_t wl, int32_t wr, const int32_t* __restrict__ kv_valid, int32_t Sq,
    int32_t Sk, int32_t bq, int32_t bk, int32_t M, int32_t N, uint8_t* __restrict__ full,
    uint8_t* __restrict__ part) {
  const int64_t n_all = (int64_t)M * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n_all; x += stride) {
    const int m = (int)(x / N), n = (int)(x % N);
    const int64_t r0 = (int64_t)m * bq, r1 = min((int64_t)(m + 1) * bq, (int64_t)Sq);
    const int64_t c0 = (int64_t)n * bk, c1 = min((int64_t)(n + 1) * bk, (int64_t)Sk);
    bool all = true, any = true;
    if (mm == 1 || mm == 3) {
      const int64_t dmin = r0 - (c1 - 1), dmax = (r1 - 1) - c0;
      // kept differences [lo, hi]
      const int64_t lo = mm == 1 ? 0 : (wr < 0 ? INT64_MIN / 2 : -(int64_t)wr);
      const int64_t hi = mm == 1 ? INT64_MAX / 2 : (wl < 0 ? INT64_MAX / 2 : (int64_t)wl);
      all = dmin >= lo && dmax <= hi;
      any = dmax >= lo && dmin <= hi;
    } else if (mm == 2) {
      const int64_t v = kv_valid[n];
      all = v >= c1 - c0;
      any = v > 0;
    }
    full[x] = all ? 1 : 0;
    part[x] = (any && !all) ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_block_sparsity(int32_t mask_mod, int32_t win_left, int32_t win_right,
                                 const int32_t* kv_valid, int32_t Sq, int32_t Sk, int32_t block_q,
                                 int32_t block_kv, uint8_t* full, uint8_t* part, hipStream_t s) {
  const int32_t M = (int32_t)(((int64_t)Sq + block_q - 1) / block_q);
  const int32_t N = (int32_t)(((int64_t)Sk + block_kv - 1) / block_kv);
  const int64_t work = (int64_t)M * N;
  if (work <= 0) return hipSuccess;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(block_sparsity_kernel, dim3((unsigned)blocks), dim3(256), 0, s, mask_mod,
                     win_left, win_right, kv_valid, Sq, Sk, block_q, block_kv, M, N, full, part);
  return hipGetLastError();
}

hipError_t launch_mask_to_index(const uint8_t* mask, int64_t rows, int32_t N, int32_t* cnt,
                                int32_t* idx, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mask_to_index_kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0,
                     s, mask, rows, N, cnt, idx);
  return hipGetLastError();
}

hipError_t launch_bitmask_to_index(const uint32_t* words, int32_t B, int32_t Hkv, int32_t H,
                                  int32_t M, int32_t N, int32_t* cnt, int32_t* idx,
                                  hipStream_t s) {
  const int64_t rows = (int64_t)B * H * M;
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bitmask_to_index_kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock),
                     0, s, words, rows, H, H / Hkv, M, N, (N + 31) / 32, cnt, idx);
  return hipGetLastError();
}

// KV-major lists (for a pass that walks, per KV block, the Q blocks that list
// it): clear a dense transposed mask, scatter every list entry into it, then
// compact its rows like mask_to_index.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

__global__ __launch_bounds__(256) void scatter_transposed_kernel(
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ idx, int64_t rows, int32_t M,
    int32_t N, uint8_t* __restrict__ mt) {
  const int64_t total = rows * N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t row = e / N;  // (b*H + h)*M + i
    const int32_t s = (int32_t)(e - row * N);
    if (s >= min(max(cnt[row], 0), N)) continue;
    const int32_t j = idx[e];
    if (j < 0 || j >= N) continue;
    const int64_t bh = row / M;
    const int32_t i = (int32_t)(row - bh * M);
    mt[(bh * N + j) * M + i] = 1;
  }
}

hipError_t launch_kv_major_lists(const int32_t* cnt, const int32_t* idx, int32_t B, int32_t H,
                                 int32_t M, int32_t N, uint8_t* work, int32_t* cnt_t,
                                 int32_t* idx_t, hipStream_t s) {
  const int64_t rows = (int64_t)B * H * M;
  const int64_t cells = rows * N;
  if ((int64_t)B * H * N == 0) return hipSuccess;
  if (cells > 0) {
    const unsigned g = (unsigned)std::min<int64_t>((cells + 255) / 256, 65536);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(g), dim3(256), 0, s, work, cells);
    hipLaunchKernelGGL(scatter_transposed_kernel, dim3(g), dim3(256), 0, s, cnt, idx, rows, M,
                       N, work);
  }
  return launch_mask_to_index(work, (int64_t)B * H * N, M, cnt_t, idx_t, s);
}

// Varlen KV-major transposition: one thread per (head, list slot p) of the
// forward's packed lists; slot p of sequence b's Q-block row i (p = off[b] +
// i*N_b + s) that holds a listed KV block j marks cell (j, i) of the
// transposed row layout, at off[b] + j*M_b + i.
__global__ __launch_bounds__(256) void varlen_scatter_transposed_kernel(
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ idx, int32_t H, int32_t B,
    const int32_t* __restrict__ cu_m, const int32_t* __restrict__ cu_n,
    const int32_t* __restrict__ off, int32_t total_m, int32_t total_n, uint8_t* __restrict__ mt) {
  const int64_t total = (int64_t)H * total_n;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int h = (int)(e / total_n);
    const int pslot = (int)(e - (int64_t)h * total_n);
    int lo = 0, hi = B - 1;  // largest b with off[b] <= pslot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= pslot)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int b = lo;
    const int mb = cu_m[b + 1] - cu_m[b], nb = cu_n[b + 1] - cu_n[b];
    const int local = pslot - off[b];
    if (mb <= 0 || nb <= 0 || local < 0 || local >= mb * nb) continue;
    const int i = local / nb, s = local - i * nb;
    if (s >= min(max(cnt[(int64_t)h * total_m + cu_m[b] + i], 0), nb)) continue;
    const int32_t j = idx[e];
    if (j < 0 || j >= nb) continue;
    mt[(int64_t)h * total_n + off[b] + (int64_t)j * mb + i] = 1;
  }
}

hipError_t launch_varlen_kv_major_lists(const int32_t* cnt, const int32_t* idx, int32_t H,
                                        int32_t B, const int32_t* cu_m, const int32_t* cu_n,
                                        const int32_t* off, int32_t total_m, int32_t total_kv,
                                        int32_t total_n, uint8_t* work, int32_t* cnt_t,
                                        int32_t* idx_t, hipStream_t s) {
  const int64_t cells = (int64_t)H * total_n;
  if ((int64_t)H * total_kv == 0) return hipSuccess;
  if (cells > 0) {
    const unsigned g = (unsigned)std::min<int64_t>((cells + 255) / 256, 65536);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(g), dim3(256), 0, s, work, cells);
    hipLaunchKernelGGL(varlen_scatter_transposed_kernel, dim3(g), dim3(256), 0, s, cnt, idx, H, B,
                       cu_m, cu_n, off, total_m, total_n, work);
  }
  // the transposed rows: (b, j) over cu_n, width M_b = span / N_b
  return launch_varlen_mask_to_index(work, H, B, cu_n, off, total_kv, total_n, cnt_t, idx_t, s);
}

hipError_t launch_varlen_mask_to_index(const uint8_t* mask, int32_t H, int32_t B,
                                       const int32_t* cu_m, const int32_t* off, int32_t total_m,
                                       int32_t total_n, int32_t* cnt, int32_t* idx,
                                       hipStream_t s) {
  const int64_t rows = (int64_t)H * total_m;
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(varlen_mask_to_index_kernel, dim3((unsigned)blocks),
                     dim3(64 * kWavesPerBlock), 0, s, mask, H, B, cu_m, off, total_m, total_n,
                     cnt, idx);
  return hipGetLastError();
}

hipError_t launch_expand_kv_blocks(const uint8_t* block_mask, const int32_t* block_valid,
                                   int32_t R, int32_t NL, int32_t factor, int32_t child,
                                   uint8_t* full, uint8_t* part, int32_t* kv_valid,
                                   hipStream_t s) {
  const int64_t n = (int64_t)R * NL * factor;
  const int64_t ncols = (int64_t)NL * factor;
  const int64_t work = n > ncols ? n : ncols;
  if (work <= 0) return hipSuccess;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(expand_kv_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     block_mask, block_valid, R, NL, factor, child, full, part, kv_valid);
  return hipGetLastError();
}

}  // namespace bsa
