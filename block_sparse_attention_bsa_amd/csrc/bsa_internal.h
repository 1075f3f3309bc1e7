// Internal launch interface between the C-ABI layer (bsa_api.cpp) and the
// gfx950 kernels.  Not installed; not part of the ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace bsa {

// Keys per KV sub-tile staged through LDS.  A listed KV block of block_kv
// tokens is processed as ceil(block_kv / kKvTile) sub-tiles.
constexpr int kKvTile = 64;
constexpr int kProxyMaxBlocks = 16384;  // semantic KV blocks per row with proxies (LDS bitmap)

// Everything one forward launch needs, in element units of the input dtype.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  // strides: batched {batch, seq, head}; varlen {-, token, head}
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  // block lists (cnt == nullptr: list absent)
  const int32_t* mcnt;
  const int32_t* midx;
  const int32_t* fcnt;
  const int32_t* fidx;
  int64_t mc_s[3], mi_s[4], fc_s[3], fi_s[4];
  const int32_t* kv_valid;
  int64_t kvv_ld;  // varlen: entries between the kv_valid rows of two sequences (0: shared row)
  // varlen bookkeeping (device, [B+1]); null for batched
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* cu_m;
  const int32_t* blk_off;
  int32_t B, H, hrep, Sq, Sk;
  int32_t block_q, block_kv, qsub;
  int32_t mask_mod, varlen;
  int32_t tiles_per_head;  // batched: num_m_blocks*qsub; varlen: total_m_blocks*qsub
  int32_t total_m, total_n;  // varlen only
  int32_t lse_ld;          // batched: Sq; varlen: total_q
  int32_t num_tiles;       // grid size
  float c;                 // softmax_scale * log2(e)
  int32_t win_left, win_right;  // local mask_mod bounds (negative = unbounded)
  int32_t gpack;      // Q heads per tile (> 1: heads of one KV head packed, sharing lists)
  int32_t kvh_lists;  // lists indexed by KV head (cnt [B,H_kv,M] ...) instead of Q head
  int32_t lpt;        // varlen: Q blocks late in their sequence first (varlen_block_by_rank)
  int32_t pack;       // route packing: 64-key items gathered from consecutive listed blocks
  // proxy-compensated route: mean-K / summed-V block summaries [B, N, H_kv, D]
  const void* ksum;
  const void* vsum;
  int64_t ks_sb, ks_ss, ks_sh;
  int64_t vs_sb, vs_ss, vs_sh;
};

// Launch the forward kernel instance for (D, rows per workgroup, dtype):
// bf16 inputs use the DMA-pipelined kernel, fp32 inputs the register-staged
// one (which rounds to bf16 at load).  Returns hipSuccess or the launch
// error; unsupported combinations return hipErrorInvalidValue (the caller
// checks support first).
hipError_t launch_fwd(const FwdParams& p, int D, int tile_m, bool f32_in, hipStream_t s);
hipError_t launch_fwd_staged(const FwdParams& p, int D, int tile_m, bool f32_in, hipStream_t s);
// bf16 staged kernel with the proxy-compensated route (batched, no element
// mask, any summary strides); launch_fwd takes the route itself (p.ksum set)
// when the summaries share K's and V's row strides.
hipError_t launch_fwd_proxy_staged(const FwdParams& p, int D, int tile_m, hipStream_t s);
// 256-row ping-pong kernel (bf16, D in {64, 96, 128}).
hipError_t launch_fwd_pp(const FwdParams& p, int D, hipStream_t s);

// Backward (bf16, batched): inputs, gradients, the forward's lists (Q-major)
// and their KV-major transposes.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* drow;  // workspace [B,H,Sq]: rowsum(dO * O)
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_ss, q_sh, k_sb, k_ss, k_sh, v_sb, v_ss, v_sh, o_sb, o_ss, o_sh;
  int64_t do_sb, do_ss, do_sh, dq_sb, dq_ss, dq_sh, dk_sb, dk_ss, dk_sh, dv_sb, dv_ss, dv_sh;
  const int32_t* mcnt;
  const int32_t* midx;
  const int32_t* fcnt;
  const int32_t* fidx;
  int64_t mc_s[3], mi_s[4], fc_s[3], fi_s[4];
  const int32_t* tmcnt;
  const int32_t* tmidx;
  const int32_t* tfcnt;
  const int32_t* tfidx;
  int64_t tmc_s[3], tmi_s[4], tfc_s[3], tfi_s[4];
  const int32_t* kv_valid;
  int32_t B, H, hrep, Sq, Sk, M, N, block_q, block_kv, mask_mod, win_left, win_right;
  float c;      // softmax_scale * log2(e)
  float scale;  // softmax_scale
  // Packed varlen layout (the varlen kernel instances): B sequences, Sq =
  // total Q tokens (the LSE row length), M = total Q blocks, N = total KV
  // blocks; per-sequence token starts, block prefix sums and list-slot
  // offsets (sum of M_b*N_b); kv_valid row b at kv_valid + b*kvv_ld.
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* cu_m;
  const int32_t* cu_n;
  const int32_t* boff;
  int64_t kvv_ld;
  bool varlen;
  // dK/dV launch order (workspace, written by the launch): the KV-block
  // rows by decreasing KV-major list length, or nullptr for index order
  int32_t* kv_order;
  // Proxy route (batched; the PX kernel instances run when px_keep is set).
  // KV blocks 0 .. px_n-1 hold the keys and values (keys from px_sk on are
  // masked); the blocks after them hold one summary key per original block
  // (mean key, summed value / c_n; c_n the block's token count), whose
  // softmax weight c_n enters as log2 c_n added to its exponent.  Summary
  // position u (key px_k0 + u, px_k0 = px_n*block_kv) holds block u's
  // summaries for u < px_nreg (full blocks, weight log2 block_kv = px_lw);
  // a last block shorter than block_kv has a KV block of its own, px_gl,
  // whose first key holds its summaries (weight px_lwl = log2 c_last; px_gl
  // = -1 when there is none).  Q block i of (b, h) takes position u when bit
  // u % 64 of word px_keep[((b*H + h)*M + i)*px_w + u/64] is set.  dK/dV of
  // the keys go to dk/dv (rows < px_sk), those of the summaries to px_dks /
  // px_dvs ([B, px_n, H_kv, D], element strides), dV divided by c_n.
  const uint64_t* px_keep;
  void* px_dks;
  void* px_dvs;
  int64_t px_dks_sb, px_dks_sn, px_dks_sh, px_dvs_sb, px_dvs_sn, px_dvs_sh;
  int32_t px_n, px_nreg, px_gl, px_w, px_sk, px_k0, px_cl;
  float px_lw, px_lwl;
};
// Rows the dK/dV launch order covers at most (beyond it: index order).
constexpr int64_t kBwdOrderMaxItems = (int64_t)1 << 20;
// Backward of the proxy route: the extended K/V, contiguous [B, (N + Nc)*bk,
// Hkv, D]: rows t < N*bk the keys and values (zero past Sk), then summary
// positions u = t - N*bk: block u's mean key and summed value / c_n for
// u < nreg, the last block's at u = lastpos when it is shorter than bk
// (lastpos = ceil(nreg / bk)*bk, its own chunk; else lastpos = -1), zero
// elsewhere.  The extended block mask [B, H, M, N + Nc] marks block n < N
// when the row lists it and block N + g when the row takes any summary
// position of chunk g (positions g*bk .. g*bk + bk - 1); the positions a
// row takes (blocks it does not list) are bits, [B, H, M, W] words of 64
// (W = ceil(Nc*bk / 64)).  bf16 data as 16-bit patterns; element strides.
struct ProxyBwdParams {
  const uint16_t *k, *v, *ks, *vs;
  int64_t k_sb, k_ss, k_sh, v_sb, v_ss, v_sh;
  int64_t ks_sb, ks_sn, ks_sh, vs_sb, vs_sn, vs_sh;
  uint16_t *kx, *vx;
  uint8_t* maskx;
  uint64_t* keep;
  const int32_t *mcnt, *midx, *fcnt, *fidx;
  int64_t mc_s[3], mi_s[4], fc_s[3], fi_s[4];
  int32_t B, H, Hkv, M, N, Nc, W, bk, Sk, D, nreg, lastpos;
};
hipError_t launch_proxy_bwd_prepare(const ProxyBwdParams& p, hipStream_t s);

hipError_t launch_bwd(const BwdParams& p, int D, hipStream_t s);
// fp32 [B,S,H,D] (element strides str, unit head_dim stride) <-> contiguous bf16
// (bf16 as its 16-bit pattern)
hipError_t launch_cast_f32_bf16(const float* src, const int64_t str[3], int32_t B, int32_t S,
                                int32_t H, int32_t D, uint16_t* dst, hipStream_t st);
hipError_t launch_cast_bf16_f32(const uint16_t* src, const int64_t str[3], int32_t B, int32_t S,
                                int32_t H, int32_t D, float* dst, hipStream_t st);
// Rows (B*H*Sq) the allocation-free backward's static row-dot array holds.
constexpr int64_t kBwdNoallocMaxRows = (int64_t)1 << 22;
// Device address of that array on the current device (looked up once per
// device, then cached).
hipError_t bwd_noalloc_scratch(float** out);

hipError_t launch_kv_major_lists(const int32_t* cnt, const int32_t* idx, int32_t B, int32_t H,
                                 int32_t M, int32_t N, uint8_t* work, int32_t* cnt_t,
                                 int32_t* idx_t, hipStream_t s);
hipError_t launch_varlen_kv_major_lists(const int32_t* cnt, const int32_t* idx, int32_t H,
                                        int32_t B, const int32_t* cu_m, const int32_t* cu_n,
                                        const int32_t* off, int32_t total_m, int32_t total_kv,
                                        int32_t total_n, uint8_t* work, int32_t* cnt_t,
                                        int32_t* idx_t, hipStream_t s);
hipError_t launch_bitmask_to_index(const uint32_t* words, int32_t B, int32_t Hkv, int32_t H,
                                  int32_t M, int32_t N, int32_t* cnt, int32_t* idx, hipStream_t s);
hipError_t launch_mask_to_index(const uint8_t* mask, int64_t rows, int32_t N,
                                int32_t* cnt, int32_t* idx, hipStream_t s);

hipError_t launch_varlen_mask_to_index(const uint8_t* mask, int32_t H, int32_t B,
                                       const int32_t* cu_m, const int32_t* off,
                                       int32_t total_m, int32_t total_n,
                                       int32_t* cnt, int32_t* idx, hipStream_t s);

hipError_t launch_block_sparsity(int32_t mask_mod, int32_t win_left, int32_t win_right,
                                 const int32_t* kv_valid, int32_t Sq, int32_t Sk, int32_t block_q,
                                 int32_t block_kv, uint8_t* full, uint8_t* part, hipStream_t s);

hipError_t launch_expand_kv_blocks(const uint8_t* block_mask, const int32_t* block_valid,
                                   int32_t R, int32_t NL, int32_t factor, int32_t child,
                                   uint8_t* full, uint8_t* part, int32_t* kv_valid,
                                   hipStream_t s);

}  // namespace bsa
