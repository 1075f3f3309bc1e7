// C-ABI entry points of libbsa.so: argument checks, the tile-fit rule,
// launch-parameter assembly and the optional host-side metadata check.
// No device allocation, no device->host copies on the normal path.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <cmath>
#include <limits>
#include <vector>

#include "../../include/bsa.h"
#include "bsa_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_head_dim(int D) { return D == 64 || D == 96 || D == 128 || D == 192 || D == 256; }

// Tile fit (runguoli.com "FlashAttention - CuTe Kernels & Block Sparsity":
// fit the forward tile to the sparse block instead of rejecting it).  A Q
// block that is a multiple of 32 rows takes the largest of 256/128/64/32
// rows dividing it (256 only for head_dim <= 128 with bf16 inputs, where
// eight waves of 32 rows fit two per SIMD).  Any other Q block takes the
// smallest of 32/64/128 rows that holds it, or 128-row tiles beyond 128
// rows; the rows of its last tile stop at the block end.  A Q block is
// covered by ceil(block_q / tile_m) workgroups sharing its block-list row.
// KV blocks of any size are cut into 64-key sub-tiles inside the kernel.
int fit_tile_m(int block_q, int D, bool f32_in, int mask_mod) {
  // the 256-row kernel knows the causal and valid-count masks only
  if (block_q % 256 == 0 && D <= 128 && !f32_in && mask_mod != BSA_MASK_LOCAL) return 256;
  if (block_q % 128 == 0) return 128;
  if (block_q % 64 == 0) return 64;
  if (block_q % 32 == 0) return 32;
  if (block_q < 32) return 32;
  if (block_q < 64) return 64;
  return 128;
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A list absent, or the same row for every head (head strides 0).
bool heads_broadcast(const bsa_block_list& L) {
  return L.cnt == nullptr || (L.cnt_stride[1] == 0 && L.idx_stride[1] == 0);
}

// GQA head packing: when every Q head of a KV head reads the same lists (the
// lists are given per KV head, or broadcast over heads) and the 256-row
// kernel serves the shape, one workgroup takes G = 256 / tile_m heads of
// that KV head, tile_m rows each, so every K/V item staged in LDS feeds G
// heads.  Returns G (1: no packing).
int gqa_pack(bool lists_shared, int tile_m, int hrep, int D, bool f32_in, int mask_mod,
             bool proxy) {
  if (!lists_shared || tile_m >= 256 || proxy || f32_in || D > 128 || mask_mod == BSA_MASK_LOCAL)
    return 1;
  const int G = 256 / tile_m;
  return hrep % G == 0 ? G : 1;
}

bool strides_ok(const int64_t* s, int n, int esize) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || (s[i] * esize) % 16 != 0) return false;
  return true;
}

// The bf16 kernel addresses one 64-key K/V sub-tile with 32-bit byte
// offsets from its first row.
bool subtile_offsets_fit(int64_t k_row_stride, int64_t v_row_stride, int esize) {
  const int64_t lim = (int64_t)1 << 31;
  return 64 * k_row_stride * esize < lim && 64 * v_row_stride * esize < lim;
}

bool list_ok(const bsa_block_list& L) {
  if (L.cnt == nullptr) return true;
  if (L.idx == nullptr) return false;
  for (int i = 0; i < 3; ++i)
    if (L.cnt_stride[i] < 0) return false;
  for (int i = 0; i < 4; ++i)
    if (L.idx_stride[i] < 0) return false;
  return true;
}

// ---- BSA_FLAG_VALIDATE: copy the lists to the host and check every row.
bsa_status fetch(const int32_t* dev, int64_t n, std::vector<int32_t>& host, hipStream_t s) {
  host.assign((size_t)(n > 0 ? n : 0), 0);
  if (n <= 0) return BSA_OK;
  if (hipMemcpyAsync(host.data(), dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return BSA_ERR_HIP;
  return BSA_OK;
}

// checks one Q-block row given its two (count, row-start) pairs
bool row_ok(const std::vector<int32_t>* hidx[2], const int64_t cnt[2], const int64_t start[2],
            const int64_t step[2], int64_t N, std::vector<char>& seen) {
  seen.assign((size_t)N, 0);
  for (int l = 0; l < 2; ++l) {
    if (cnt[l] < 0 || cnt[l] > N) return false;
    for (int64_t e = 0; e < cnt[l]; ++e) {
      const int64_t j = (*hidx[l])[(size_t)(start[l] + e * step[l])];
      if (j < 0 || j >= N || seen[(size_t)j]) return false;
      seen[(size_t)j] = 1;
    }
  }
  return true;
}

int64_t span3(const int64_t* st, int64_t d0, int64_t d1, int64_t d2) {
  return (d0 - 1) * st[0] + (d1 - 1) * st[1] + (d2 - 1) * st[2] + 1;
}

// H: the lists' head count (Q heads, or KV heads with BSA_FLAG_KV_HEAD_LISTS)
bsa_status validate_batched(const bsa_block_sparse& bs, int B, int H, int64_t M, int64_t N,
                            hipStream_t s) {
  const bsa_block_list* lists[2] = {&bs.mask, &bs.full};
  std::vector<int32_t> hc[2], hi[2];
  for (int l = 0; l < 2; ++l) {
    if (!lists[l]->cnt) continue;
    const int64_t nc = span3(lists[l]->cnt_stride, B, H, M);
    const int64_t ni = span3(lists[l]->idx_stride, B, H, M) + (N - 1) * lists[l]->idx_stride[3];
    bsa_status st = fetch(lists[l]->cnt, nc, hc[l], s);
    if (st == BSA_OK) st = fetch(lists[l]->idx, N > 0 ? ni : 0, hi[l], s);
    if (st != BSA_OK) return st;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return BSA_ERR_HIP;
  std::vector<char> seen;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int64_t m = 0; m < M; ++m) {
        int64_t cnt[2] = {0, 0}, start[2] = {0, 0}, step[2] = {0, 0};
        const std::vector<int32_t>* hidx[2] = {&hi[0], &hi[1]};
        for (int l = 0; l < 2; ++l) {
          const bsa_block_list& L = *lists[l];
          if (!L.cnt) continue;
          cnt[l] = hc[l][(size_t)(b * L.cnt_stride[0] + h * L.cnt_stride[1] + m * L.cnt_stride[2])];
          start[l] = b * L.idx_stride[0] + h * L.idx_stride[1] + m * L.idx_stride[2];
          step[l] = L.idx_stride[3];
        }
        if (!row_ok(hidx, cnt, start, step, N, seen)) return BSA_ERR_METADATA;
      }
  return BSA_OK;
}

bsa_status validate_varlen(const bsa_block_sparse& bs, int B, int H, const int32_t* cu_q,
                           const int32_t* cu_k, const int32_t* cu_m, const int32_t* off,
                           int32_t total_m, int32_t total_n, hipStream_t s) {
  std::vector<int32_t> hq, hk, hm, ho;
  bsa_status st = fetch(cu_q, B + 1, hq, s);
  if (st == BSA_OK) st = fetch(cu_k, B + 1, hk, s);
  if (st == BSA_OK) st = fetch(cu_m, B + 1, hm, s);
  if (st == BSA_OK) st = fetch(off, B + 1, ho, s);
  const bsa_block_list* lists[2] = {&bs.mask, &bs.full};
  std::vector<int32_t> hc[2], hi[2];
  for (int l = 0; l < 2 && st == BSA_OK; ++l) {
    if (!lists[l]->cnt) continue;
    const bsa_block_list& L = *lists[l];
    const int64_t nc = total_m > 0 ? (H - 1) * L.cnt_stride[1] + (total_m - 1) * L.cnt_stride[2] + 1 : 0;
    const int64_t ni = total_n > 0 ? (H - 1) * L.idx_stride[1] + (total_n - 1) * L.idx_stride[3] + 1 : 0;
    st = fetch(L.cnt, nc, hc[l], s);
    if (st == BSA_OK) st = fetch(L.idx, ni, hi[l], s);
  }
  if (st != BSA_OK) return st;
  if (hipStreamSynchronize(s) != hipSuccess) return BSA_ERR_HIP;
  // the cumulative arrays must be the ones the sequence lengths imply
  if (hq[0] != 0 || hk[0] != 0 || hm[0] != 0 || ho[0] != 0) return BSA_ERR_METADATA;
  for (int b = 0; b < B; ++b) {
    const int64_t sq = hq[b + 1] - hq[b], sk = hk[b + 1] - hk[b];
    if (sq < 0 || sk < 0) return BSA_ERR_METADATA;
    const int64_t nm = cdiv64(sq, bs.block_q), nn = cdiv64(sk, bs.block_kv);
    if (hm[b + 1] - hm[b] != nm || ho[b + 1] - ho[b] != nm * nn) return BSA_ERR_METADATA;
  }
  if (hm[B] != total_m || ho[B] != total_n) return BSA_ERR_METADATA;
  std::vector<char> seen;
  for (int h = 0; h < H; ++h)
    for (int b = 0; b < B; ++b) {
      const int64_t nm = hm[b + 1] - hm[b];
      const int64_t nn = nm > 0 ? (ho[b + 1] - ho[b]) / nm : 0;
      for (int64_t m = 0; m < nm; ++m) {
        int64_t cnt[2] = {0, 0}, start[2] = {0, 0}, step[2] = {0, 0};
        const std::vector<int32_t>* hidx[2] = {&hi[0], &hi[1]};
        for (int l = 0; l < 2; ++l) {
          const bsa_block_list& L = *lists[l];
          if (!L.cnt) continue;
          cnt[l] = hc[l][(size_t)(h * L.cnt_stride[1] + (hm[b] + m) * L.cnt_stride[2])];
          start[l] = h * L.idx_stride[1] + (ho[b] + m * nn) * L.idx_stride[3];
          step[l] = L.idx_stride[3];
        }
        if (!row_ok(hidx, cnt, start, step, nn, seen)) return BSA_ERR_METADATA;
      }
    }
  return BSA_OK;
}

void copy_lists(bsa::FwdParams& p, const bsa_block_sparse& bs) {
  p.mcnt = bs.mask.cnt;
  p.midx = bs.mask.idx;
  p.fcnt = bs.full.cnt;
  p.fidx = bs.full.idx;
  for (int i = 0; i < 3; ++i) {
    p.mc_s[i] = bs.mask.cnt_stride[i];
    p.fc_s[i] = bs.full.cnt_stride[i];
  }
  for (int i = 0; i < 4; ++i) {
    p.mi_s[i] = bs.mask.idx_stride[i];
    p.fi_s[i] = bs.full.idx_stride[i];
  }
}

}  // namespace

extern "C" {

const char* bsa_status_str(bsa_status s) {
  switch (s) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSA_ERR_MISALIGNED: return "misaligned pointer or stride (16-byte alignment required)";
    case BSA_ERR_METADATA: return "invalid block-sparse metadata";
    case BSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

bsa_status bsa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, bsa_dtype dt,
                   int32_t B, int32_t H, int32_t H_kv, int32_t Sq, int32_t Sk, int32_t D,
                   const int64_t q_str[3], const int64_t k_str[3], const int64_t v_str[3],
                   const int64_t o_str[3], const bsa_block_sparse* bs, bsa_mask_mod mask_mod,
                   const int32_t* kv_valid, float softmax_scale, uint32_t flags,
                   hipStream_t stream) {
  if (B < 0 || H <= 0 || H_kv <= 0 || Sq < 0 || Sk < 0 || H % H_kv != 0)
    return BSA_ERR_INVALID_ARGUMENT;
  if (dt != BSA_BF16 && dt != BSA_F32) return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod < BSA_MASK_NONE || mask_mod > BSA_MASK_LOCAL) return BSA_ERR_INVALID_ARGUMENT;
  if (!bs || !q_str || !k_str || !v_str || !o_str) return BSA_ERR_INVALID_ARGUMENT;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return BSA_ERR_INVALID_ARGUMENT;
  if (bs->block_q <= 0 || bs->block_kv <= 0) return BSA_ERR_INVALID_ARGUMENT;
  if (!list_ok(bs->mask) || !list_ok(bs->full)) return BSA_ERR_INVALID_ARGUMENT;
  if (!supported_head_dim(D)) return BSA_ERR_UNSUPPORTED;
  // proxy-compensated route: the staged bf16 kernel, 128-row tiles at most
  const bool proxy = bs->proxy_k != nullptr || bs->proxy_v != nullptr;
  if (proxy && (!bs->proxy_k || !bs->proxy_v)) return BSA_ERR_INVALID_ARGUMENT;
  if (proxy && (mask_mod != BSA_MASK_NONE || dt != BSA_BF16)) return BSA_ERR_UNSUPPORTED;
  int tile_m = fit_tile_m(bs->block_q, D, dt == BSA_F32, mask_mod);
  if (proxy && tile_m == 256) tile_m = 128;
  if (tile_m == 0) return BSA_ERR_UNSUPPORTED;
  const bool kvh = (flags & BSA_FLAG_KV_HEAD_LISTS) != 0;
  const int gpack = gqa_pack(kvh || (heads_broadcast(bs->mask) && heads_broadcast(bs->full)),
                             tile_m, H / H_kv, D, dt == BSA_F32, mask_mod, proxy);
  const int rows_per_head = tile_m;  // rows of one head in a tile
  if (gpack > 1) tile_m = 256;
  if ((int64_t)B * H * Sq == 0) return BSA_OK;  // nothing to write
  if (!q || !k || !v || !o || !lse) return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod == BSA_MASK_KV_VALID_COUNT && !kv_valid && bs->mask.cnt)
    return BSA_ERR_INVALID_ARGUMENT;
  const int es = dt == BSA_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return BSA_ERR_MISALIGNED;
  if (!strides_ok(q_str, 3, es) || !strides_ok(k_str, 3, es) || !strides_ok(v_str, 3, es) ||
      !strides_ok(o_str, 3, es))
    return BSA_ERR_MISALIGNED;
  if (!subtile_offsets_fit(k_str[1], v_str[1], es)) return BSA_ERR_UNSUPPORTED;
  const int64_t M = cdiv64(Sq, bs->block_q), N = cdiv64(Sk, bs->block_kv);
  if (proxy) {
    if (N > bsa::kProxyMaxBlocks) return BSA_ERR_UNSUPPORTED;
    if (!aligned16(bs->proxy_k) || !aligned16(bs->proxy_v) || !strides_ok(bs->proxy_k_str, 3, es) ||
        !strides_ok(bs->proxy_v_str, 3, es))
      return BSA_ERR_MISALIGNED;
    if (!subtile_offsets_fit(bs->proxy_k_str[1], bs->proxy_v_str[1], es))
      return BSA_ERR_UNSUPPORTED;
  }
  const int64_t qsub = cdiv64(bs->block_q, rows_per_head);
  const int64_t tiles_per_head = M * qsub;
  const int64_t tiles = (int64_t)B * (H / gpack) * tiles_per_head;
  if (tiles > std::numeric_limits<int32_t>::max() || N > std::numeric_limits<int32_t>::max() / 2)
    return BSA_ERR_UNSUPPORTED;
  if (flags & BSA_FLAG_VALIDATE) {
    const bsa_status st = validate_batched(*bs, B, kvh ? H_kv : H, M, N, stream);
    if (st != BSA_OK) return st;
  }
  bsa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.q_sb = q_str[0]; p.q_ss = q_str[1]; p.q_sh = q_str[2];
  p.k_sb = k_str[0]; p.k_ss = k_str[1]; p.k_sh = k_str[2];
  p.v_sb = v_str[0]; p.v_ss = v_str[1]; p.v_sh = v_str[2];
  p.o_sb = o_str[0]; p.o_ss = o_str[1]; p.o_sh = o_str[2];
  copy_lists(p, *bs);
  p.kv_valid = kv_valid;
  p.kvv_ld = 0;
  p.B = B;
  p.H = H;
  p.hrep = H / H_kv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.block_q = bs->block_q;
  p.block_kv = bs->block_kv;
  p.qsub = (int32_t)qsub;
  p.gpack = gpack;
  p.kvh_lists = kvh ? 1 : 0;
  p.mask_mod = mask_mod;
  p.win_left = bs->window_left;
  p.win_right = bs->window_right;
  p.varlen = 0;
  // Route packing where KV blocks are not a whole number of 64-key items
  // (with the run masks tested as bits, even the 12.5 % of empty slots of
  // 112-key blocks repays the gathered addresses: d128 sweep +0.5 %, d64
  // +5 %, d192 +3.5 %, d256 +2.5 %; 48 keys +12 %, 16 keys 3x): the
  // 128/64/32-row bf16 kernel (no local mask, no proxies; not the 32-row
  // tiles at head_dim >= 192, whose registers would spill) gathers K/V rows
  // by 31-bit byte offsets from the sequence's first row
  const int64_t lim = (int64_t)1 << 31;
  const int64_t bk_items = cdiv64(bs->block_kv, bsa::kKvTile) * bsa::kKvTile;
  p.pack = bk_items > bs->block_kv && tile_m <= 128 &&
           !(tile_m == 32 && D >= 192) && dt == BSA_BF16 &&
           mask_mod != BSA_MASK_LOCAL && !proxy && (int64_t)Sk * k_str[1] * 2 < lim &&
           (int64_t)Sk * v_str[1] * 2 < lim;
  p.tiles_per_head = (int32_t)tiles_per_head;
  p.lse_ld = Sq;
  p.num_tiles = (int32_t)tiles;
  p.c = softmax_scale * kLog2e;
  if (proxy) {
    p.ksum = bs->proxy_k;
    p.vsum = bs->proxy_v;
    p.ks_sb = bs->proxy_k_str[0]; p.ks_ss = bs->proxy_k_str[1]; p.ks_sh = bs->proxy_k_str[2];
    p.vs_sb = bs->proxy_v_str[0]; p.vs_ss = bs->proxy_v_str[1]; p.vs_sh = bs->proxy_v_str[2];
  }
  // the DMA kernel reuses K's and V's row offsets for the summaries
  const bool proxy_dma = proxy && bs->proxy_k_str[1] == k_str[1] && bs->proxy_v_str[1] == v_str[1];
  const hipError_t e = proxy && !proxy_dma ? bsa::launch_fwd_proxy_staged(p, D, tile_m, stream)
                                           : bsa::launch_fwd(p, D, tile_m, dt == BSA_F32, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

bsa_status bsa_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                          bsa_dtype dt, int32_t B, int32_t H, int32_t H_kv, int32_t D,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          const int32_t* cu_total_m_blocks, const int32_t* block_idx_offsets,
                          int32_t total_m_blocks, int32_t total_n_blocks, int32_t total_q,
                          const int64_t q_str[2], const int64_t k_str[2], const int64_t v_str[2],
                          const int64_t o_str[2], const bsa_block_sparse* bs,
                          bsa_mask_mod mask_mod, const int32_t* kv_valid,
                          int64_t kv_valid_ld, float softmax_scale, uint32_t flags,
                          hipStream_t stream) {
  if (bs && (bs->proxy_k || bs->proxy_v)) return BSA_ERR_UNSUPPORTED;  // batched only
  if (B < 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || total_m_blocks < 0 || total_n_blocks < 0 ||
      total_q < 0)
    return BSA_ERR_INVALID_ARGUMENT;
  if (dt != BSA_BF16 && dt != BSA_F32) return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod < BSA_MASK_NONE || mask_mod > BSA_MASK_LOCAL) return BSA_ERR_INVALID_ARGUMENT;
  if (kv_valid_ld < 0) return BSA_ERR_INVALID_ARGUMENT;
  if (!bs || !q_str || !k_str || !v_str || !o_str) return BSA_ERR_INVALID_ARGUMENT;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return BSA_ERR_INVALID_ARGUMENT;
  if (bs->block_q <= 0 || bs->block_kv <= 0) return BSA_ERR_INVALID_ARGUMENT;
  if (!list_ok(bs->mask) || !list_ok(bs->full)) return BSA_ERR_INVALID_ARGUMENT;
  if (!supported_head_dim(D)) return BSA_ERR_UNSUPPORTED;
  int tile_m = fit_tile_m(bs->block_q, D, dt == BSA_F32, mask_mod);
  if (tile_m == 0) return BSA_ERR_UNSUPPORTED;
  const bool kvh = (flags & BSA_FLAG_KV_HEAD_LISTS) != 0;
  const int gpack = gqa_pack(kvh || (heads_broadcast(bs->mask) && heads_broadcast(bs->full)),
                             tile_m, H / H_kv, D, dt == BSA_F32, mask_mod, false);
  const int rows_per_head = tile_m;
  if (gpack > 1) tile_m = 256;
  if (B == 0 || total_m_blocks == 0) return BSA_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k || !cu_total_m_blocks ||
      !block_idx_offsets)
    return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod == BSA_MASK_KV_VALID_COUNT && !kv_valid && bs->mask.cnt)
    return BSA_ERR_INVALID_ARGUMENT;
  const int es = dt == BSA_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return BSA_ERR_MISALIGNED;
  if (!strides_ok(q_str, 2, es) || !strides_ok(k_str, 2, es) || !strides_ok(v_str, 2, es) ||
      !strides_ok(o_str, 2, es))
    return BSA_ERR_MISALIGNED;
  if (!subtile_offsets_fit(k_str[0], v_str[0], es)) return BSA_ERR_UNSUPPORTED;
  const int qsub = (int)cdiv64(bs->block_q, rows_per_head);
  const int64_t tiles_per_head = (int64_t)total_m_blocks * qsub;
  const int64_t tiles = tiles_per_head * (H / gpack);
  if (tiles > std::numeric_limits<int32_t>::max()) return BSA_ERR_UNSUPPORTED;
  if (flags & BSA_FLAG_VALIDATE) {
    const bsa_status st = validate_varlen(*bs, B, kvh ? H_kv : H, cu_seqlens_q, cu_seqlens_k,
                                          cu_total_m_blocks,
                                          block_idx_offsets, total_m_blocks, total_n_blocks, stream);
    if (st != BSA_OK) return st;
  }
  bsa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.q_ss = q_str[0]; p.q_sh = q_str[1];
  p.k_ss = k_str[0]; p.k_sh = k_str[1];
  p.v_ss = v_str[0]; p.v_sh = v_str[1];
  p.o_ss = o_str[0]; p.o_sh = o_str[1];
  copy_lists(p, *bs);
  p.kv_valid = mask_mod == BSA_MASK_KV_VALID_COUNT ? kv_valid : nullptr;
  p.kvv_ld = kv_valid_ld;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.cu_m = cu_total_m_blocks;
  p.blk_off = block_idx_offsets;
  p.B = B;
  p.H = H;
  p.hrep = H / H_kv;
  p.block_q = bs->block_q;
  p.block_kv = bs->block_kv;
  p.qsub = qsub;
  p.gpack = gpack;
  p.kvh_lists = kvh ? 1 : 0;
  p.mask_mod = mask_mod;
  p.win_left = bs->window_left;
  p.win_right = bs->window_right;
  p.varlen = 1;
  // long-list-first order when its per-workgroup cost (B log total_m reads) is small
  p.lpt = B <= 64 ? 1 : 0;
  p.tiles_per_head = (int32_t)tiles_per_head;
  p.total_m = total_m_blocks;
  p.total_n = total_n_blocks;
  p.lse_ld = total_q;
  p.num_tiles = (int32_t)tiles;
  p.c = softmax_scale * kLog2e;
  const hipError_t e = bsa::launch_fwd(p, D, tile_m, dt == BSA_F32, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

bsa_status bsa_block_sparsity(bsa_mask_mod mask_mod, int32_t window_left, int32_t window_right,
                              const int32_t* kv_valid, int32_t Sq, int32_t Sk, int32_t block_q,
                              int32_t block_kv, uint8_t* full, uint8_t* part,
                              hipStream_t stream) {
  if (mask_mod < BSA_MASK_NONE || mask_mod > BSA_MASK_LOCAL) return BSA_ERR_INVALID_ARGUMENT;
  if (Sq < 0 || Sk < 0 || block_q <= 0 || block_kv <= 0) return BSA_ERR_INVALID_ARGUMENT;
  const int64_t M = cdiv64(Sq, block_q), N = cdiv64(Sk, block_kv);
  if (M * N == 0) return BSA_OK;
  if (M * N > std::numeric_limits<int32_t>::max()) return BSA_ERR_UNSUPPORTED;
  if (!full || !part) return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod == BSA_MASK_KV_VALID_COUNT && !kv_valid) return BSA_ERR_INVALID_ARGUMENT;
  const hipError_t e = bsa::launch_block_sparsity(mask_mod, window_left, window_right, kv_valid, Sq,
                                                  Sk, block_q, block_kv, full, part, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

bsa_status bsa_mask_to_index(const uint8_t* mask, int32_t B, int32_t H, int32_t M, int32_t N,
                             int32_t* cnt, int32_t* idx, hipStream_t stream) {
  if (B < 0 || H < 0 || M < 0 || N < 0) return BSA_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)B * H * M;
  if (rows == 0) return BSA_OK;
  if (!cnt || (N > 0 && (!mask || !idx))) return BSA_ERR_INVALID_ARGUMENT;
  const hipError_t e = bsa::launch_mask_to_index(mask, rows, N, cnt, idx, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

}  // extern "C"

namespace {

// The proxy route's extra inputs to the backward kernels (bsa_bwd_proxy):
// the bit sets of the summary positions each Q block takes ([B, H, M, w]
// words), the gradient outputs of the keys and values (strides of the
// caller's tensors, not of the extended K/V) and of the summaries, the
// number of original KV blocks n, of full blocks nreg, the KV block gl of
// the last block's summaries (-1 when that block is full), the original key
// count sk and the last block's token count.
struct ProxyBwd {
  const uint64_t* keep;
  void* dk;
  void* dv;
  void* dks;
  void* dvs;
  int64_t dk_str[3], dv_str[3], dks_str[3], dvs_str[3];
  int32_t n, nreg, gl, w, sk, c_last;
};

// The backward behind bsa_bwd and bsa_bwd_noalloc.  work == nullptr with
// noalloc: the row dots go to the library's static per-device array.
bsa_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, int32_t B, int32_t H,
                    int32_t H_kv, int32_t Sq, int32_t Sk, int32_t D, const int64_t q_str[3],
                    const int64_t k_str[3], const int64_t v_str[3], const int64_t o_str[3],
                    const bsa_block_sparse* bs, const bsa_block_list* mask_t,
                    const bsa_block_list* full_t, bsa_mask_mod mask_mod, const int32_t* kv_valid,
                    float softmax_scale, float* work, bool noalloc, hipStream_t stream,
                    bool check_only = false, const ProxyBwd* px = nullptr) {
  if (B < 0 || H <= 0 || H_kv <= 0 || Sq < 0 || Sk < 0 || H % H_kv != 0)
    return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod < BSA_MASK_NONE || mask_mod > BSA_MASK_LOCAL) return BSA_ERR_INVALID_ARGUMENT;
  if (!bs || !mask_t || !full_t || !q_str || !k_str || !v_str || !o_str)
    return BSA_ERR_INVALID_ARGUMENT;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return BSA_ERR_INVALID_ARGUMENT;
  if (bs->block_q <= 0 || bs->block_kv <= 0) return BSA_ERR_INVALID_ARGUMENT;
  if (!list_ok(bs->mask) || !list_ok(bs->full) || !list_ok(*mask_t) || !list_ok(*full_t))
    return BSA_ERR_INVALID_ARGUMENT;
  if (!supported_head_dim(D)) return BSA_ERR_UNSUPPORTED;
  if (bs->proxy_k || bs->proxy_v) return BSA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * (Sq + Sk) == 0) return BSA_OK;
  if (noalloc && (int64_t)B * H * Sq > bsa::kBwdNoallocMaxRows) return BSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || (!noalloc && !work))
    return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod == BSA_MASK_KV_VALID_COUNT && !kv_valid && (bs->mask.cnt || mask_t->cnt))
    return BSA_ERR_INVALID_ARGUMENT;
  for (const void* ptr : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(ptr)) return BSA_ERR_MISALIGNED;
  if (!strides_ok(q_str, 3, 2) || !strides_ok(k_str, 3, 2) || !strides_ok(v_str, 3, 2) ||
      !strides_ok(o_str, 3, 2))
    return BSA_ERR_MISALIGNED;
  // the tiles of 64 rows are staged with 32-bit byte offsets from their first row
  if (!subtile_offsets_fit(q_str[1], o_str[1], 2) || !subtile_offsets_fit(k_str[1], v_str[1], 2))
    return BSA_ERR_UNSUPPORTED;
  const int64_t M = cdiv64(Sq, bs->block_q), N = cdiv64(Sk, bs->block_kv);
  const int64_t gq = (int64_t)B * H * M * cdiv64(bs->block_q, 64);
  const int64_t gk = (int64_t)B * H_kv * N * cdiv64(bs->block_kv, 64);
  if (gq > std::numeric_limits<int32_t>::max() || gk > std::numeric_limits<int32_t>::max() ||
      M > std::numeric_limits<int32_t>::max() || N > std::numeric_limits<int32_t>::max())
    return BSA_ERR_UNSUPPORTED;
  bsa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse; p.drow = work;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.q_sb = q_str[0]; p.q_ss = q_str[1]; p.q_sh = q_str[2];
  p.k_sb = k_str[0]; p.k_ss = k_str[1]; p.k_sh = k_str[2];
  p.v_sb = v_str[0]; p.v_ss = v_str[1]; p.v_sh = v_str[2];
  p.o_sb = o_str[0]; p.o_ss = o_str[1]; p.o_sh = o_str[2];
  p.do_sb = o_str[0]; p.do_ss = o_str[1]; p.do_sh = o_str[2];
  p.dq_sb = q_str[0]; p.dq_ss = q_str[1]; p.dq_sh = q_str[2];
  p.dk_sb = k_str[0]; p.dk_ss = k_str[1]; p.dk_sh = k_str[2];
  p.dv_sb = v_str[0]; p.dv_ss = v_str[1]; p.dv_sh = v_str[2];
  p.mcnt = bs->mask.cnt; p.midx = bs->mask.idx; p.fcnt = bs->full.cnt; p.fidx = bs->full.idx;
  p.tmcnt = mask_t->cnt; p.tmidx = mask_t->idx; p.tfcnt = full_t->cnt; p.tfidx = full_t->idx;
  for (int i = 0; i < 3; ++i) {
    p.mc_s[i] = bs->mask.cnt_stride[i]; p.fc_s[i] = bs->full.cnt_stride[i];
    p.tmc_s[i] = mask_t->cnt_stride[i]; p.tfc_s[i] = full_t->cnt_stride[i];
  }
  for (int i = 0; i < 4; ++i) {
    p.mi_s[i] = bs->mask.idx_stride[i]; p.fi_s[i] = bs->full.idx_stride[i];
    p.tmi_s[i] = mask_t->idx_stride[i]; p.tfi_s[i] = full_t->idx_stride[i];
  }
  p.kv_valid = kv_valid;
  p.B = B; p.H = H; p.hrep = H / H_kv; p.Sq = Sq; p.Sk = Sk; p.M = (int32_t)M; p.N = (int32_t)N;
  p.block_q = bs->block_q; p.block_kv = bs->block_kv; p.mask_mod = mask_mod;
  p.win_left = bs->window_left; p.win_right = bs->window_right;
  p.c = softmax_scale * kLog2e;
  p.scale = softmax_scale;
  if (px) {  // the proxy route over the extended sequence (bsa_bwd_proxy)
    p.dk_sb = px->dk_str[0]; p.dk_ss = px->dk_str[1]; p.dk_sh = px->dk_str[2];
    p.dv_sb = px->dv_str[0]; p.dv_ss = px->dv_str[1]; p.dv_sh = px->dv_str[2];
    p.px_keep = px->keep;
    p.px_dks = px->dks;
    p.px_dvs = px->dvs;
    p.px_dks_sb = px->dks_str[0]; p.px_dks_sn = px->dks_str[1]; p.px_dks_sh = px->dks_str[2];
    p.px_dvs_sb = px->dvs_str[0]; p.px_dvs_sn = px->dvs_str[1]; p.px_dvs_sh = px->dvs_str[2];
    p.px_n = px->n;
    p.px_nreg = px->nreg;
    p.px_gl = px->gl;
    p.px_w = px->w;
    p.px_sk = px->sk;
    p.px_k0 = px->n * bs->block_kv;
    p.px_cl = px->c_last;
    p.px_lw = std::log2((float)bs->block_kv);
    p.px_lwl = std::log2((float)px->c_last);
  }
  if (check_only) return BSA_OK;  // the arguments pass; nothing is launched
  if (noalloc && bsa::bwd_noalloc_scratch(&p.drow) != hipSuccess) return BSA_ERR_HIP;
  // the dK/dV launch order follows the row dots in the workspace (the static
  // array of the allocation-free entry point holds it when it fits)
  const int64_t rows = (int64_t)B * H * Sq, items = (int64_t)B * H_kv * N;
  if (items <= bsa::kBwdOrderMaxItems && (!noalloc || rows + items <= bsa::kBwdNoallocMaxRows))
    p.kv_order = reinterpret_cast<int32_t*>(p.drow + rows);
  const hipError_t e = bsa::launch_bwd(p, D, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace

extern "C" {

bsa_status bsa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int32_t B, int32_t H,
                   int32_t H_kv, int32_t Sq, int32_t Sk, int32_t D, const int64_t q_str[3],
                   const int64_t k_str[3], const int64_t v_str[3], const int64_t o_str[3],
                   const bsa_block_sparse* bs, const bsa_block_list* mask_t,
                   const bsa_block_list* full_t, bsa_mask_mod mask_mod, const int32_t* kv_valid,
                   float softmax_scale, float* work, hipStream_t stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, Sq, Sk, D, q_str, k_str, v_str,
                  o_str, bs, mask_t, full_t, mask_mod, kv_valid, softmax_scale, work, false,
                  stream);
}

bsa_status bsa_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                       const float* lse, const float* dout, float* dq, float* dk, float* dv,
                       int32_t B, int32_t H, int32_t H_kv, int32_t Sq, int32_t Sk, int32_t D,
                       const int64_t q_str[3], const int64_t k_str[3], const int64_t v_str[3],
                       const int64_t o_str[3], const bsa_block_sparse* bs,
                       const bsa_block_list* mask_t, const bsa_block_list* full_t,
                       bsa_mask_mod mask_mod, const int32_t* kv_valid, float softmax_scale,
                       float* work, hipStream_t stream) {
  if (B < 0 || H <= 0 || H_kv <= 0 || Sq < 0 || Sk < 0 || H % H_kv != 0)
    return BSA_ERR_INVALID_ARGUMENT;
  if (!bs || !q_str || !k_str || !v_str || !o_str || bs->block_kv <= 0)
    return BSA_ERR_INVALID_ARGUMENT;
  if (!supported_head_dim(D)) return BSA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * (Sq + Sk) == 0) return BSA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !work)
    return BSA_ERR_INVALID_ARGUMENT;
  for (const void* ptr : {(const void*)q, (const void*)k, (const void*)v, (const void*)o,
                          (const void*)dout, (const void*)dq, (const void*)dk, (const void*)dv,
                          (const void*)work})
    if (!aligned16(ptr)) return BSA_ERR_MISALIGNED;
  if (!strides_ok(q_str, 3, 4) || !strides_ok(k_str, 3, 4) || !strides_ok(v_str, 3, 4) ||
      !strides_ok(o_str, 3, 4))
    return BSA_ERR_MISALIGNED;
  // work: the bf16 backward's entries, then contiguous bf16 copies of
  // q, o, dout, dq [B,Sq,H,D] and k, v, dk, dv [B,Sk,H_kv,D] (16-byte aligned:
  // every size below is a multiple of 8 elements)
  const int64_t N = cdiv64(Sk, bs->block_kv);
  const int64_t head = (int64_t)B * H * Sq + (int64_t)B * H_kv * N;
  const int64_t nq = (int64_t)B * Sq * H * D, nk = (int64_t)B * Sk * H_kv * D;
  uint16_t* base = reinterpret_cast<uint16_t*>(work + (head + 3) / 4 * 4);
  uint16_t *q16 = base, *o16 = q16 + nq, *do16 = o16 + nq, *dq16 = do16 + nq;
  uint16_t *k16 = dq16 + nq, *v16 = k16 + nk, *dk16 = v16 + nk, *dv16 = dk16 + nk;
  const int64_t sq16[3] = {(int64_t)Sq * H * D, (int64_t)H * D, D};
  const int64_t sk16[3] = {(int64_t)Sk * H_kv * D, (int64_t)H_kv * D, D};
  // every check of the bf16 backward first, so that nothing runs on bad arguments
  const bsa_status chk = bwd_impl(q16, k16, v16, o16, lse, do16, dq16, dk16, dv16, B, H, H_kv, Sq,
                                  Sk, D, sq16, sk16, sk16, sq16, bs, mask_t, full_t, mask_mod,
                                  kv_valid, softmax_scale, work, false, stream, true);
  if (chk != BSA_OK) return chk;
  if (bsa::launch_cast_f32_bf16(q, q_str, B, Sq, H, D, q16, stream) != hipSuccess ||
      bsa::launch_cast_f32_bf16(o, o_str, B, Sq, H, D, o16, stream) != hipSuccess ||
      bsa::launch_cast_f32_bf16(dout, o_str, B, Sq, H, D, do16, stream) != hipSuccess ||
      bsa::launch_cast_f32_bf16(k, k_str, B, Sk, H_kv, D, k16, stream) != hipSuccess ||
      bsa::launch_cast_f32_bf16(v, v_str, B, Sk, H_kv, D, v16, stream) != hipSuccess)
    return BSA_ERR_HIP;
  const bsa_status st = bwd_impl(q16, k16, v16, o16, lse, do16, dq16, dk16, dv16, B, H, H_kv, Sq,
                                 Sk, D, sq16, sk16, sk16, sq16, bs, mask_t, full_t, mask_mod,
                                 kv_valid, softmax_scale, work, false, stream);
  if (st != BSA_OK) return st;
  if (bsa::launch_cast_bf16_f32(dq16, q_str, B, Sq, H, D, dq, stream) != hipSuccess ||
      bsa::launch_cast_bf16_f32(dk16, k_str, B, Sk, H_kv, D, dk, stream) != hipSuccess ||
      bsa::launch_cast_bf16_f32(dv16, v_str, B, Sk, H_kv, D, dv, stream) != hipSuccess)
    return BSA_ERR_HIP;
  return BSA_OK;
}

// Workspace of bsa_bwd_proxy: the extended K/V (N blocks of keys and values,
// then Nc blocks of summary positions: one per full block, nreg of them, in
// order, and the last block's, when shorter than block_kv, first in a block
// of its own at position lastpos), the extended block mask, its Q-major and
// KV-major lists, the bit sets of the summary positions each Q block takes,
// and the backward's own entries; regions 256-byte aligned.
struct ProxyWork {
  int64_t N, Nc, NX, W, nreg, lastpos, c_last;
  int64_t kx, vx, mask, cnt, idx, cnt_t, idx_t, tr, keep, bwd, total;
};

ProxyWork proxy_work_layout(int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                            int64_t bq, int64_t bk) {
  ProxyWork w{};
  w.N = cdiv64(Sk, bk);
  w.c_last = w.N > 0 ? Sk - (w.N - 1) * bk : bk;
  if (w.c_last == bk) {
    w.nreg = w.N;
    w.Nc = cdiv64(w.N, bk);
    w.lastpos = -1;
  } else {
    w.nreg = w.N - 1;
    w.lastpos = cdiv64(w.nreg, bk) * bk;
    w.Nc = cdiv64(w.nreg, bk) + 1;
  }
  w.NX = w.N + w.Nc;
  w.W = cdiv64(w.Nc * bk, 64);
  const int64_t M = cdiv64(Sq, bq), NX = w.NX;
  const int64_t xb = B * NX * bk * Hkv * D * 2;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  int64_t at = 0;
  auto take = [&](int64_t bytes) { const int64_t o = at; at += up(bytes); return o; };
  w.kx = take(xb); w.vx = take(xb);
  w.mask = take(B * H * M * NX);
  w.cnt = take(B * H * M * 4); w.idx = take(B * H * M * NX * 4);
  w.cnt_t = take(B * H * NX * 4); w.idx_t = take(B * H * NX * M * 4); w.tr = take(B * H * NX * M);
  w.keep = take(B * H * M * w.W * 8);
  w.bwd = take((B * H * Sq + B * Hkv * NX) * 4);
  w.total = at;
  return w;
}

bsa_status bsa_bwd_proxy_work_size(int32_t B, int32_t H, int32_t H_kv, int32_t Sq, int32_t Sk,
                                   int32_t D, int32_t block_q, int32_t block_kv,
                                   int64_t* bytes) {
  if (!bytes || B < 0 || H <= 0 || H_kv <= 0 || Sq < 0 || Sk < 0 || D <= 0 || block_q <= 0 ||
      block_kv <= 0)
    return BSA_ERR_INVALID_ARGUMENT;
  *bytes = proxy_work_layout(B, H, H_kv, Sq, Sk, D, block_q, block_kv).total;
  return BSA_OK;
}

bsa_status bsa_bwd_proxy(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         void* dproxy_k, void* dproxy_v, int32_t B, int32_t H, int32_t H_kv,
                         int32_t Sq, int32_t Sk, int32_t D, const int64_t q_str[3],
                         const int64_t k_str[3], const int64_t v_str[3], const int64_t o_str[3],
                         const bsa_block_sparse* bs, float softmax_scale, void* work,
                         hipStream_t stream) {
  if (B < 0 || H <= 0 || H_kv <= 0 || Sq < 0 || Sk < 0 || H % H_kv != 0)
    return BSA_ERR_INVALID_ARGUMENT;
  if (!bs || !q_str || !k_str || !v_str || !o_str || !bs->proxy_k || !bs->proxy_v)
    return BSA_ERR_INVALID_ARGUMENT;
  if (bs->block_q <= 0 || bs->block_kv <= 0 || !list_ok(bs->mask) || !list_ok(bs->full))
    return BSA_ERR_INVALID_ARGUMENT;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return BSA_ERR_INVALID_ARGUMENT;
  if (!supported_head_dim(D)) return BSA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * (Sq + Sk) == 0) return BSA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !dproxy_k || !dproxy_v ||
      !work)
    return BSA_ERR_INVALID_ARGUMENT;
  for (const void* ptr : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv,
                          (const void*)dproxy_k, (const void*)dproxy_v, bs->proxy_k, bs->proxy_v,
                          (const void*)work})
    if (!aligned16(ptr)) return BSA_ERR_MISALIGNED;
  if (!strides_ok(q_str, 3, 2) || !strides_ok(k_str, 3, 2) || !strides_ok(v_str, 3, 2) ||
      !strides_ok(o_str, 3, 2) || !strides_ok(bs->proxy_k_str, 3, 2) ||
      !strides_ok(bs->proxy_v_str, 3, 2))
    return BSA_ERR_MISALIGNED;
  const ProxyWork L = proxy_work_layout(B, H, H_kv, Sq, Sk, D, bs->block_q, bs->block_kv);
  const int64_t M = cdiv64(Sq, bs->block_q), NX = L.NX;
  const int64_t Sx = NX * bs->block_kv;
  if (Sx > std::numeric_limits<int32_t>::max() / 2 || NX > std::numeric_limits<int32_t>::max())
    return BSA_ERR_UNSUPPORTED;
  char* w = static_cast<char*>(work);
  // the extended problem: keys and values, then one summary key per block
  const int64_t sx[3] = {Sx * H_kv * D, (int64_t)H_kv * D, D};
  bsa_block_sparse bsx{};
  bsx.mask.cnt = reinterpret_cast<const int32_t*>(w + L.cnt);
  bsx.mask.idx = reinterpret_cast<const int32_t*>(w + L.idx);
  const int64_t cst[3] = {H * M, M, 1}, ist[4] = {H * M * NX, M * NX, NX, 1};
  for (int i = 0; i < 3; ++i) bsx.mask.cnt_stride[i] = cst[i];
  for (int i = 0; i < 4; ++i) bsx.mask.idx_stride[i] = ist[i];
  bsx.block_q = bs->block_q;
  bsx.block_kv = bs->block_kv;
  bsx.window_left = bsx.window_right = -1;
  bsa_block_list mt{}, ft{};
  mt.cnt = reinterpret_cast<const int32_t*>(w + L.cnt_t);
  mt.idx = reinterpret_cast<const int32_t*>(w + L.idx_t);
  const int64_t tcs[3] = {H * NX, NX, 1}, tis[4] = {H * NX * M, NX * M, M, 1};
  for (int i = 0; i < 3; ++i) mt.cnt_stride[i] = tcs[i];
  for (int i = 0; i < 4; ++i) mt.idx_stride[i] = tis[i];
  ProxyBwd px{};
  px.keep = reinterpret_cast<const uint64_t*>(w + L.keep);
  px.dk = dk; px.dv = dv; px.dks = dproxy_k; px.dvs = dproxy_v;
  for (int i = 0; i < 3; ++i) {
    px.dk_str[i] = k_str[i]; px.dv_str[i] = v_str[i];
    px.dks_str[i] = bs->proxy_k_str[i]; px.dvs_str[i] = bs->proxy_v_str[i];
  }
  px.n = (int32_t)L.N;
  px.nreg = (int32_t)L.nreg;
  px.gl = L.lastpos >= 0 ? (int32_t)(NX - 1) : -1;
  px.w = (int32_t)L.W;
  px.sk = Sk;
  px.c_last = (int32_t)L.c_last;
  // every check of the backward over the extended problem before anything runs
  bsa_status st = bwd_impl(q, w + L.kx, w + L.vx, o, lse, dout, dq, dk, dv, B, H, H_kv, Sq,
                           (int32_t)Sx, D, q_str, sx, sx, o_str, &bsx, &mt, &ft, BSA_MASK_NONE,
                           nullptr, softmax_scale, reinterpret_cast<float*>(w + L.bwd), false,
                           stream, true, &px);
  if (st != BSA_OK) return st;
  bsa::ProxyBwdParams pp{};
  pp.k = static_cast<const uint16_t*>(k); pp.v = static_cast<const uint16_t*>(v);
  pp.ks = static_cast<const uint16_t*>(bs->proxy_k); pp.vs = static_cast<const uint16_t*>(bs->proxy_v);
  pp.k_sb = k_str[0]; pp.k_ss = k_str[1]; pp.k_sh = k_str[2];
  pp.v_sb = v_str[0]; pp.v_ss = v_str[1]; pp.v_sh = v_str[2];
  pp.ks_sb = bs->proxy_k_str[0]; pp.ks_sn = bs->proxy_k_str[1]; pp.ks_sh = bs->proxy_k_str[2];
  pp.vs_sb = bs->proxy_v_str[0]; pp.vs_sn = bs->proxy_v_str[1]; pp.vs_sh = bs->proxy_v_str[2];
  pp.kx = reinterpret_cast<uint16_t*>(w + L.kx); pp.vx = reinterpret_cast<uint16_t*>(w + L.vx);
  pp.maskx = reinterpret_cast<uint8_t*>(w + L.mask);
  pp.keep = reinterpret_cast<uint64_t*>(w + L.keep);
  pp.mcnt = bs->mask.cnt; pp.midx = bs->mask.idx; pp.fcnt = bs->full.cnt; pp.fidx = bs->full.idx;
  for (int i = 0; i < 3; ++i) { pp.mc_s[i] = bs->mask.cnt_stride[i]; pp.fc_s[i] = bs->full.cnt_stride[i]; }
  for (int i = 0; i < 4; ++i) { pp.mi_s[i] = bs->mask.idx_stride[i]; pp.fi_s[i] = bs->full.idx_stride[i]; }
  pp.B = B; pp.H = H; pp.Hkv = H_kv; pp.M = (int32_t)M; pp.N = (int32_t)L.N;
  pp.Nc = (int32_t)L.Nc; pp.W = (int32_t)L.W;
  pp.bk = bs->block_kv; pp.Sk = Sk; pp.D = D;
  pp.nreg = (int32_t)L.nreg; pp.lastpos = (int32_t)L.lastpos;
  if (bsa::launch_proxy_bwd_prepare(pp, stream) != hipSuccess ||
      bsa::launch_mask_to_index(pp.maskx, (int64_t)B * H * M, (int32_t)NX,
                                reinterpret_cast<int32_t*>(w + L.cnt),
                                reinterpret_cast<int32_t*>(w + L.idx), stream) != hipSuccess ||
      bsa::launch_kv_major_lists(reinterpret_cast<const int32_t*>(w + L.cnt),
                                 reinterpret_cast<const int32_t*>(w + L.idx), B, H, (int32_t)M,
                                 (int32_t)NX, reinterpret_cast<uint8_t*>(w + L.tr),
                                 reinterpret_cast<int32_t*>(w + L.cnt_t),
                                 reinterpret_cast<int32_t*>(w + L.idx_t), stream) != hipSuccess)
    return BSA_ERR_HIP;
  return bwd_impl(q, w + L.kx, w + L.vx, o, lse, dout, dq, dk, dv, B, H, H_kv, Sq, (int32_t)Sx, D,
                  q_str, sx, sx, o_str, &bsx, &mt, &ft, BSA_MASK_NONE, nullptr, softmax_scale,
                  reinterpret_cast<float*>(w + L.bwd), false, stream, false, &px);
}

bsa_status bsa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int32_t B, int32_t H, int32_t H_kv, int32_t Sq, int32_t Sk, int32_t D,
                           const int64_t q_str[3], const int64_t k_str[3],
                           const int64_t v_str[3], const int64_t o_str[3],
                           const bsa_block_sparse* bs, const bsa_block_list* mask_t,
                           const bsa_block_list* full_t, bsa_mask_mod mask_mod,
                           const int32_t* kv_valid, float softmax_scale, hipStream_t stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, Sq, Sk, D, q_str, k_str, v_str,
                  o_str, bs, mask_t, full_t, mask_mod, kv_valid, softmax_scale, nullptr, true,
                  stream);
}

bsa_status bsa_varlen_bwd(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          int32_t B, int32_t H, int32_t H_kv, int32_t D,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          const int32_t* cu_total_m_blocks, const int32_t* cu_total_kv_blocks,
                          const int32_t* block_idx_offsets, int32_t total_m_blocks,
                          int32_t total_kv_blocks, int32_t total_q, const int64_t q_str[2],
                          const int64_t k_str[2], const int64_t v_str[2], const int64_t o_str[2],
                          const bsa_block_sparse* bs, const bsa_block_list* mask_t,
                          const bsa_block_list* full_t, bsa_mask_mod mask_mod,
                          const int32_t* kv_valid, int64_t kv_valid_ld, float softmax_scale,
                          float* work, hipStream_t stream) {
  if (B < 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || total_m_blocks < 0 ||
      total_kv_blocks < 0 || total_q < 0 || kv_valid_ld < 0)
    return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod < BSA_MASK_NONE || mask_mod > BSA_MASK_LOCAL) return BSA_ERR_INVALID_ARGUMENT;
  if (!bs || !mask_t || !full_t || !q_str || !k_str || !v_str || !o_str)
    return BSA_ERR_INVALID_ARGUMENT;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return BSA_ERR_INVALID_ARGUMENT;
  if (bs->block_q <= 0 || bs->block_kv <= 0) return BSA_ERR_INVALID_ARGUMENT;
  if (!list_ok(bs->mask) || !list_ok(bs->full) || !list_ok(*mask_t) || !list_ok(*full_t))
    return BSA_ERR_INVALID_ARGUMENT;
  if (!supported_head_dim(D)) return BSA_ERR_UNSUPPORTED;
  if (bs->proxy_k || bs->proxy_v) return BSA_ERR_UNSUPPORTED;
  if (B == 0 || (int64_t)total_m_blocks + total_kv_blocks == 0) return BSA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !work || !cu_seqlens_q ||
      !cu_seqlens_k || !cu_total_m_blocks || !cu_total_kv_blocks || !block_idx_offsets)
    return BSA_ERR_INVALID_ARGUMENT;
  if (mask_mod == BSA_MASK_KV_VALID_COUNT && !kv_valid && (bs->mask.cnt || mask_t->cnt))
    return BSA_ERR_INVALID_ARGUMENT;
  for (const void* ptr : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(ptr)) return BSA_ERR_MISALIGNED;
  if (!strides_ok(q_str, 2, 2) || !strides_ok(k_str, 2, 2) || !strides_ok(v_str, 2, 2) ||
      !strides_ok(o_str, 2, 2))
    return BSA_ERR_MISALIGNED;
  if (!subtile_offsets_fit(q_str[0], o_str[0], 2) || !subtile_offsets_fit(k_str[0], v_str[0], 2))
    return BSA_ERR_UNSUPPORTED;
  const int64_t gq = (int64_t)H * total_m_blocks * cdiv64(bs->block_q, 64);
  const int64_t gk = (int64_t)H_kv * total_kv_blocks * cdiv64(bs->block_kv, 64);
  if (gq > std::numeric_limits<int32_t>::max() || gk > std::numeric_limits<int32_t>::max())
    return BSA_ERR_UNSUPPORTED;
  bsa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse; p.drow = work;
  p.dq = dq; p.dk = dk; p.dv = dv;
  // token-major layouts: no batch stride, the sequence start moves the base
  p.q_ss = q_str[0]; p.q_sh = q_str[1];
  p.k_ss = k_str[0]; p.k_sh = k_str[1];
  p.v_ss = v_str[0]; p.v_sh = v_str[1];
  p.o_ss = o_str[0]; p.o_sh = o_str[1];
  p.do_ss = o_str[0]; p.do_sh = o_str[1];
  p.dq_ss = q_str[0]; p.dq_sh = q_str[1];
  p.dk_ss = k_str[0]; p.dk_sh = k_str[1];
  p.dv_ss = v_str[0]; p.dv_sh = v_str[1];
  p.mcnt = bs->mask.cnt; p.midx = bs->mask.idx; p.fcnt = bs->full.cnt; p.fidx = bs->full.idx;
  p.tmcnt = mask_t->cnt; p.tmidx = mask_t->idx; p.tfcnt = full_t->cnt; p.tfidx = full_t->idx;
  for (int i = 0; i < 3; ++i) {
    p.mc_s[i] = bs->mask.cnt_stride[i]; p.fc_s[i] = bs->full.cnt_stride[i];
    p.tmc_s[i] = mask_t->cnt_stride[i]; p.tfc_s[i] = full_t->cnt_stride[i];
  }
  for (int i = 0; i < 4; ++i) {
    p.mi_s[i] = bs->mask.idx_stride[i]; p.fi_s[i] = bs->full.idx_stride[i];
    p.tmi_s[i] = mask_t->idx_stride[i]; p.tfi_s[i] = full_t->idx_stride[i];
  }
  p.kv_valid = mask_mod == BSA_MASK_KV_VALID_COUNT ? kv_valid : nullptr;
  p.kvv_ld = kv_valid_ld;
  p.B = B; p.H = H; p.hrep = H / H_kv; p.Sq = total_q; p.Sk = 0;
  p.M = total_m_blocks; p.N = total_kv_blocks;
  p.block_q = bs->block_q; p.block_kv = bs->block_kv; p.mask_mod = mask_mod;
  p.win_left = bs->window_left; p.win_right = bs->window_right;
  p.c = softmax_scale * kLog2e;
  p.scale = softmax_scale;
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k; p.cu_m = cu_total_m_blocks;
  p.cu_n = cu_total_kv_blocks; p.boff = block_idx_offsets;
  p.varlen = true;
  // the dK/dV launch order follows the row dots in the workspace
  const int64_t items = (int64_t)H_kv * total_kv_blocks;
  if (items <= bsa::kBwdOrderMaxItems)
    p.kv_order = reinterpret_cast<int32_t*>(work + (int64_t)H * total_q);
  const hipError_t e = bsa::launch_bwd(p, D, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

bsa_status bsa_varlen_kv_major_lists(const int32_t* cnt, const int32_t* idx, int32_t H, int32_t B,
                                     const int32_t* cu_total_m_blocks,
                                     const int32_t* cu_total_kv_blocks,
                                     const int32_t* block_idx_offsets, int32_t total_m_blocks,
                                     int32_t total_kv_blocks, int32_t total_n_blocks,
                                     uint8_t* work, int32_t* cnt_t, int32_t* idx_t,
                                     hipStream_t stream) {
  if (H < 0 || B < 0 || total_m_blocks < 0 || total_kv_blocks < 0 || total_n_blocks < 0)
    return BSA_ERR_INVALID_ARGUMENT;
  if ((int64_t)H * total_kv_blocks == 0 || B == 0) return BSA_OK;
  if (!cnt_t || !cu_total_m_blocks || !cu_total_kv_blocks || !block_idx_offsets)
    return BSA_ERR_INVALID_ARGUMENT;
  if (total_n_blocks > 0 && (!cnt || !idx || !work || !idx_t)) return BSA_ERR_INVALID_ARGUMENT;
  const hipError_t e = bsa::launch_varlen_kv_major_lists(
      cnt, idx, H, B, cu_total_m_blocks, cu_total_kv_blocks, block_idx_offsets, total_m_blocks,
      total_kv_blocks, total_n_blocks, work, cnt_t, idx_t, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

bsa_status bsa_kv_major_lists(const int32_t* cnt, const int32_t* idx, int32_t B, int32_t H,
                              int32_t M, int32_t N, uint8_t* work, int32_t* cnt_t,
                              int32_t* idx_t, hipStream_t stream) {
  if (B < 0 || H < 0 || M < 0 || N < 0) return BSA_ERR_INVALID_ARGUMENT;
  if ((int64_t)B * H * N == 0) return BSA_OK;
  if (!cnt_t || (M > 0 && (!cnt || !idx || !work || !idx_t))) return BSA_ERR_INVALID_ARGUMENT;
  const hipError_t e = bsa::launch_kv_major_lists(cnt, idx, B, H, M, N, work, cnt_t, idx_t, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

bsa_status bsa_bitmask_to_index(const uint32_t* words, int32_t B, int32_t Hkv, int32_t H,
                                int32_t M, int32_t N, int32_t* cnt, int32_t* idx,
                                hipStream_t stream) {
  if (B < 0 || Hkv < 0 || H < 0 || M < 0 || N < 0) return BSA_ERR_INVALID_ARGUMENT;
  if (H > 0 && (Hkv == 0 || H % Hkv != 0)) return BSA_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)B * H * M;
  if (rows == 0) return BSA_OK;
  if (!cnt || (N > 0 && (!words || !idx))) return BSA_ERR_INVALID_ARGUMENT;
  const hipError_t e = bsa::launch_bitmask_to_index(words, B, Hkv, H, M, N, cnt, idx, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

bsa_status bsa_varlen_mask_to_index(const uint8_t* mask, int32_t H, int32_t B,
                                    const int32_t* cu_total_m_blocks,
                                    const int32_t* block_idx_offsets, int32_t total_m_blocks,
                                    int32_t total_n_blocks, int32_t* cnt, int32_t* idx,
                                    hipStream_t stream) {
  if (H < 0 || B < 0 || total_m_blocks < 0 || total_n_blocks < 0) return BSA_ERR_INVALID_ARGUMENT;
  if ((int64_t)H * total_m_blocks == 0 || B == 0) return BSA_OK;
  if (!cnt || !cu_total_m_blocks || !block_idx_offsets) return BSA_ERR_INVALID_ARGUMENT;
  if (total_n_blocks > 0 && (!mask || !idx)) return BSA_ERR_INVALID_ARGUMENT;
  const hipError_t e =
      bsa::launch_varlen_mask_to_index(mask, H, B, cu_total_m_blocks, block_idx_offsets,
                                       total_m_blocks, total_n_blocks, cnt, idx, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

bsa_status bsa_varlen_offsets(const int32_t* seqlens_q, const int32_t* seqlens_k, int32_t B,
                              int32_t block_q, int32_t block_kv, int32_t* cu_total_m_blocks,
                              int32_t* block_idx_offsets, int32_t* total_m_blocks,
                              int32_t* total_n_blocks) {
  if (B < 0 || block_q <= 0 || block_kv <= 0) return BSA_ERR_INVALID_ARGUMENT;
  if (!cu_total_m_blocks || !block_idx_offsets || !total_m_blocks || !total_n_blocks)
    return BSA_ERR_INVALID_ARGUMENT;
  if (B > 0 && (!seqlens_q || !seqlens_k)) return BSA_ERR_INVALID_ARGUMENT;
  int64_t cm = 0, co = 0;
  cu_total_m_blocks[0] = 0;
  block_idx_offsets[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seqlens_q[b] < 0 || seqlens_k[b] < 0) return BSA_ERR_INVALID_ARGUMENT;
    const int64_t nm = cdiv64(seqlens_q[b], block_q);
    const int64_t nn = cdiv64(seqlens_k[b], block_kv);
    cm += nm;
    co += nm * nn;
    if (cm > std::numeric_limits<int32_t>::max() || co > std::numeric_limits<int32_t>::max())
      return BSA_ERR_INVALID_ARGUMENT;
    cu_total_m_blocks[b + 1] = (int32_t)cm;
    block_idx_offsets[b + 1] = (int32_t)co;
  }
  *total_m_blocks = (int32_t)cm;
  *total_n_blocks = (int32_t)co;
  return BSA_OK;
}

bsa_status bsa_expand_kv_blocks(const uint8_t* block_mask, const int32_t* block_valid, int32_t R,
                                int32_t NL, int32_t factor, int32_t child, uint8_t* full,
                                uint8_t* part, int32_t* kv_valid, hipStream_t stream) {
  if (R < 0 || NL < 0 || factor <= 0 || child <= 0) return BSA_ERR_INVALID_ARGUMENT;
  if ((int64_t)NL * factor > std::numeric_limits<int32_t>::max()) return BSA_ERR_INVALID_ARGUMENT;
  if (NL == 0) return BSA_OK;
  if (!block_valid || !kv_valid) return BSA_ERR_INVALID_ARGUMENT;
  if (R > 0 && (!block_mask || !full || !part)) return BSA_ERR_INVALID_ARGUMENT;
  const hipError_t e = bsa::launch_expand_kv_blocks(block_mask, block_valid, R, NL, factor, child,
                                                    full, part, kv_valid, stream);
  return e == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

}  // extern "C"
