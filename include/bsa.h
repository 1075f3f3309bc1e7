/*
 * bsa.h - block-sparse attention forward for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsa.so.  Plain device/host pointers and sizes only.  Every
 * device buffer is allocated, owned and freed by the caller; the library
 * keeps no state, allocates no device memory and enqueues all device work on
 * the caller's stream.  Without BSA_FLAG_VALIDATE no call synchronises.
 * Errors are returned as bsa_status codes; nothing is thrown across the ABI.
 *
 * The problem statement follows these pages:
 *  - flash-attention PR #2224 "[CuTe,Flex] varlen blocksparsity" (PR
 *    description and review thread): batched metadata *_block_cnt
 *    [B,H,num_m_blocks] / *_block_idx [B,H,num_m_blocks,num_n_blocks], the
 *    packed varlen layout [H,total_m_blocks] / [H,total_n_blocks], the
 *    cumulative arrays cu_total_m_blocks and block_idx_offsets, the ordered
 *    (mask_block_cnt, mask_block_idx, full_block_cnt, full_block_idx) tuple
 *    with the full list optional, and no device->host syncs at launch;
 *  - FastVideo PR #1354 "VSA-256 fastpath" (review thread): the per-KV-block
 *    valid-token-count mask_mod, LSE laid out [B,H,S], BSHD/BHSD inputs,
 *    256-token logical KV blocks run as 128-token tiles;
 *  - "Dense FlashAttention vs Block-Sparse Attention" (yiliu30.github.io),
 *    section 2: the boolean block mask becomes a reversed, -1 padded list of
 *    selected KV-block ids per Q-block row;
 *  - runguoli.com "FlashAttention - CuTe Kernels & Block Sparsity": forward
 *    tiles are fitted to the sparse block sizes instead of rejecting them.
 *
 * Semantics of one forward call (batch b, head h, row r of Q block
 * i = r / block_q; KV head = h / (H / H_kv)):
 *   visible columns C_r = { c < Sk : c / block_kv listed in full[b,h,i] }
 *                       U { c < Sk : c / block_kv listed in mask[b,h,i] and mask_mod(r,c) }
 *   O_r = sum_{c in C_r} softmax_c(scale * q_r.k_c) v_c,   LSE_r = ln sum_{c in C_r} exp(scale * q_r.k_c)
 *   An empty C_r gives O_r = 0 and LSE_r = -inf.
 * mask_mod applies to mask-list blocks only; columns >= Sk are never
 * visible; listed ids outside [0, num_n_blocks) are skipped.  A KV block
 * must not be listed twice for one row (within or across the two lists);
 * with BSA_FLAG_VALIDATE such metadata is rejected, without it the result
 * is undefined (memory stays safe).
 *
 * Arithmetic: Q/K/V are rounded to bf16 (round-to-nearest-even) if given as
 * fp32; QK^T and PV run on bf16 MFMA with fp32 accumulation; softmax is
 * fp32.  O has the input dtype; LSE is fp32 natural log.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size or shape */
  BSA_ERR_UNSUPPORTED = 2,      /* head_dim, block size or dtype without a kernel */
  BSA_ERR_MISALIGNED = 3,       /* base pointer or stride not 16-byte aligned */
  BSA_ERR_METADATA = 4,         /* BSA_FLAG_VALIDATE found bad block lists */
  BSA_ERR_HIP = 5               /* a HIP runtime call or launch failed */
} bsa_status;

typedef enum {
  BSA_BF16 = 0, /* Q,K,V,O bfloat16 */
  BSA_F32 = 1   /* Q,K,V,O float32; inputs rounded to bf16 at load, O written fp32 */
} bsa_dtype;

typedef enum {
  BSA_MASK_NONE = 0,           /* mask-list blocks behave like full blocks */
  BSA_MASK_CAUSAL = 1,         /* keep kv_idx <= q_idx (sequence-local ids in varlen) */
  BSA_MASK_KV_VALID_COUNT = 2, /* keep (kv_idx % block_kv) < kv_valid[kv_idx / block_kv] */
  BSA_MASK_LOCAL = 3           /* keep q_idx - window_left <= kv_idx <= q_idx + window_right
                                  (sequence-local ids in varlen); a negative bound is unbounded,
                                  so (-1, 0) is causal.  The causal/local range of "Dense
                                  FlashAttention vs Block-Sparse Attention", section 6. */
} bsa_mask_mod;

/* Copy the block lists to the host, check them (ids in range, no repeats
 * within or across the two lists of a row, 0 <= cnt <= num_n_blocks),
 * synchronising the stream.  Debug path. */
#define BSA_FLAG_VALIDATE 1u

/* The block lists are given per KV head: their head index is the KV head
 * (batched cnt [B,H_kv,M], idx [B,H_kv,M,N]; varlen cnt [H_kv,total_m],
 * idx [H_kv,total_n]) and Q head h reads the lists of KV head h/(H/H_kv),
 * as the packed bitmap of the PrimTS page is owned per KV head.  The Q
 * heads of one KV head then share their lists, and the forward packs them
 * (flash-attention PR #2224 review thread, pack_gqa): where the 256-row
 * kernel serves the shape (bf16, head_dim <= 128, no local mask, no
 * proxies) one workgroup covers G = 256/tile_m Q heads of tile_m rows each
 * when G divides H/H_kv, so each K/V tile staged on chip feeds G heads.
 * Lists broadcast over heads (head strides 0) are packed the same way
 * without the flag.  Results do not depend on the packing. */
#define BSA_FLAG_KV_HEAD_LISTS 2u

/* One block list (the mask list or the full list).  int32 device arrays.
 * cnt == NULL means the list is absent (no blocks).
 * Batched:  cnt[b,h,m]      at cnt + b*cnt_stride[0] + h*cnt_stride[1] + m*cnt_stride[2]
 *           idx[b,h,m,s]    at idx + b*idx_stride[0] + h*idx_stride[1] + m*idx_stride[2] + s*idx_stride[3]
 *           (stride 0 broadcasts the metadata over B or H).
 * Varlen:   cnt[h,mg]       at cnt + h*cnt_stride[1] + mg*cnt_stride[2]      (mg < total_m_blocks)
 *           idx[h,p]        at idx + h*idx_stride[1] + p*idx_stride[3]       (p < total_n_blocks)
 *           where row (b, m) of head h starts at p = block_idx_offsets[b] + m*num_n(b);
 *           cnt_stride[0], idx_stride[0], idx_stride[2] are ignored.
 * Only the first cnt entries of a row are read; their order is free. */
typedef struct {
  const int32_t* cnt;
  const int32_t* idx;
  int64_t cnt_stride[3];
  int64_t idx_stride[4];
} bsa_block_list;

/* The (mask, full) pair and the sparse block sizes (in tokens).
 * block_q and block_kv may be any positive size: the forward fits its tiles
 * to them (runguoli.com "FlashAttention - CuTe Kernels & Block Sparsity":
 * tiles fitted to the sparse block size instead of rejecting it).  A Q
 * block runs as ceil(block_q / tile_m) tiles of tile_m in {256, 128, 64,
 * 32} rows whose last one stops at the block end; a KV block runs as 64-key
 * sub-tiles whose last one stops at the block end.
 * window_left / window_right: the bounds of BSA_MASK_LOCAL (ignored by the
 * other mask_mods).
 *
 * proxy_k / proxy_v: optional summaries for the proxy-compensated route (the
 * PrimTS page, "proxy-compensated block-sparse attention", flashinfer pull
 * request 4872: description, proxy paragraph).  Both NULL: plain block-sparse
 * attention.  Both set: every KV block n that a Q-block row does not list
 * (in either list) enters that row's softmax once, with score
 * softmax_scale * q.proxy_k[n], value proxy_v[n], and weight c_n in the
 * denominator, where c_n = min(block_kv, Sk - n*block_kv) is its token count:
 *   O = (sum_exact e^s v + sum_omitted e^sbar Vsum) / (sum_exact e^s + sum_omitted c e^sbar),
 *   LSE = log of that denominator.
 * proxy_k holds the mean key and proxy_v the summed value of each block
 * (device, dtype dt = BSA_BF16, [B, N, H_kv, D] with N = ceil(Sk/block_kv),
 * element strides proxy_*_str = {batch, block, head}, head_dim stride 1,
 * 16-byte aligned like K and V).  Requires BSA_MASK_NONE, the batched
 * forward and N <= 16384; otherwise BSA_ERR_UNSUPPORTED.  A row whose blocks
 * are all listed has no proxy term. */
typedef struct {
  bsa_block_list mask;
  bsa_block_list full;
  int32_t block_q;
  int32_t block_kv;
  int32_t window_left;
  int32_t window_right;
  const void* proxy_k;
  const void* proxy_v;
  int64_t proxy_k_str[3];
  int64_t proxy_v_str[3];
} bsa_block_sparse;

/* Batched forward.
 *  q [B,Sq,H,D], k/v [B,Sk,H_kv,D], o [B,Sq,H,D]: device, dtype dt; element
 *    strides x_str = {batch, seq, head}; head_dim stride is 1.  BSHD and
 *    BHSD tensors are both expressed through these strides.
 *  lse: device fp32 [B,H,Sq], contiguous.
 *  D in {64, 96, 128, 192, 256}; H % H_kv == 0; Sq, Sk >= 0.
 *  bs: block lists, cnt [B,H,ceil(Sq/block_q)], idx [B,H,ceil(Sq/block_q),ceil(Sk/block_kv)].
 *  kv_valid: device int32 [ceil(Sk/block_kv)] for BSA_MASK_KV_VALID_COUNT, else ignored.
 *  softmax_scale: applied to q.k before the softmax (and inside LSE).
 * Requirements: 16-byte aligned base pointers; every stride times the
 * element size a multiple of 16 bytes.  O and LSE are overwritten for every
 * row < Sq. */
bsa_status bsa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   bsa_dtype dt, int32_t B, int32_t H, int32_t H_kv,
                   int32_t Sq, int32_t Sk, int32_t D,
                   const int64_t q_str[3], const int64_t k_str[3],
                   const int64_t v_str[3], const int64_t o_str[3],
                   const bsa_block_sparse* bs, bsa_mask_mod mask_mod,
                   const int32_t* kv_valid, float softmax_scale,
                   uint32_t flags, hipStream_t stream);

/* Packed variable-length forward (flash-attention PR #2224).
 *  q [Tq,H,D], k/v [Tk,H_kv,D], o [Tq,H,D]: device, strides {token, head}.
 *  lse: device fp32 [H,Tq] contiguous (Tq = cu_seqlens_q[B]).
 *  cu_seqlens_q/k: device int32 [B+1], exclusive prefix sums of lengths.
 *  cu_total_m_blocks, block_idx_offsets: device int32 [B+1], as produced by
 *    bsa_varlen_offsets (Q-block and packed-slot prefix sums).
 *  total_m_blocks, total_n_blocks: their last entries, and total_q =
 *    cu_seqlens_q[B] (the LSE row length), passed from the host so the
 *    launch needs no device->host copy.
 *  Block ids in the lists are sequence-local; mask_mod uses sequence-local
 *  (q_idx, kv_idx).
 *  kv_valid, kv_valid_ld: the valid-token counts of BSA_MASK_KV_VALID_COUNT
 *    (FastVideo PR #1354 review thread: keep kv_off < valid of the KV
 *    block), per sequence-local KV block: sequence b's KV block j (j <
 *    ceil(seqlen_k(b)/block_kv)) has count kv_valid[b*kv_valid_ld + j]
 *    (device int32; kv_valid_ld = 0 gives every sequence one shared row).
 *    Required when mask_mod is BSA_MASK_KV_VALID_COUNT and a mask list is
 *    given; ignored otherwise.  kv_valid_ld < 0 is BSA_ERR_INVALID_ARGUMENT.
 * Alignment rules as bsa_fwd. */
bsa_status bsa_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                          bsa_dtype dt, int32_t B, int32_t H, int32_t H_kv, int32_t D,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          const int32_t* cu_total_m_blocks, const int32_t* block_idx_offsets,
                          int32_t total_m_blocks, int32_t total_n_blocks, int32_t total_q,
                          const int64_t q_str[2], const int64_t k_str[2],
                          const int64_t v_str[2], const int64_t o_str[2],
                          const bsa_block_sparse* bs, bsa_mask_mod mask_mod,
                          const int32_t* kv_valid, int64_t kv_valid_ld,
                          float softmax_scale, uint32_t flags, hipStream_t stream);

/* Dense block mask -> block lists ("Dense FlashAttention vs Block-Sparse
 * Attention", section 2).  mask: device uint8 [B,H,M,N] contiguous (nonzero
 * = selected).  Writes cnt: device int32 [B,H,M] (number selected) and idx:
 * device int32 [B,H,M,N] (selected column ids in descending order, then -1).
 * Bit-exact; deterministic. */
bsa_status bsa_mask_to_index(const uint8_t* mask, int32_t B, int32_t H, int32_t M, int32_t N,
                             int32_t* cnt, int32_t* idx, hipStream_t stream);

/* Backward of the batched forward (bf16; D in {64, 96, 128, 192, 256}): the gradient of
 * O over the listed blocks (flash-attention pull request 2224 and the
 * FastVideo pull request 1354 review name it as the missing half; the
 * formulas are those of the forward's derivative):
 *   P = exp(scale*S - LSE), dV = P^T dO, dP = dO V^T, D = rowsum(dO*O),
 *   dS = P*(dP - D), dQ = scale*dS K, dK = scale*dS^T Q,
 * dK and dV summed over the Q heads of each KV head.
 *  q, o, dout, dq [B,Sq,H,D] and k, v, dk, dv [B,Sk,H_kv,D]: device bf16,
 *    element strides {batch, seq, head} (q_str also describes dq, k_str dk,
 *    v_str dv, o_str dout), head_dim stride 1, 16-byte aligned rows.
 *  lse: the forward's LSE, device fp32 [B,H,Sq] contiguous.
 *  bs: the forward's lists, block sizes and window (as for bsa_fwd).
 *  mask_t / full_t: their KV-major transposes (bsa_kv_major_lists):
 *    cnt [B,H,N], idx [B,H,N,M] through the same stride fields (cnt_stride
 *    over {b, h, j}, idx_stride over {b, h, j, s}); cnt == NULL: absent.
 *  work: device scratch of B*H*Sq + B*H_kv*ceil(Sk/block_kv) 4-byte
 *    entries (fp32 row dots, then the int32 order in which the dK/dV
 *    workgroups start: longest KV-major lists first), overwritten.
 * dq, dk, dv are overwritten everywhere (zero where nothing is listed).
 * Returns BSA_ERR_INVALID_ARGUMENT / BSA_ERR_UNSUPPORTED / BSA_ERR_MISALIGNED
 * for bad arguments, BSA_ERR_HIP if a launch fails.  Deterministic: no atomics. */
bsa_status bsa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int32_t B, int32_t H,
                   int32_t H_kv, int32_t Sq, int32_t Sk, int32_t D, const int64_t q_str[3],
                   const int64_t k_str[3], const int64_t v_str[3], const int64_t o_str[3],
                   const bsa_block_sparse* bs, const bsa_block_list* mask_t,
                   const bsa_block_list* full_t, bsa_mask_mod mask_mod, const int32_t* kv_valid,
                   float softmax_scale, float* work, hipStream_t stream);

/* Backward of the batched forward with fp32 tensors (bsa_fwd with BSA_F32:
 * its kernels round Q, K, V to bf16 at load), the same gradient as bsa_bwd
 * (same pages and formulas): q, k, v, o and dout are rounded to bf16 (round
 * to nearest even) into the workspace, bsa_bwd's kernels run on those copies
 * with fp32 accumulation, and dq, dk, dv are written back as fp32 (the
 * bf16 values widened exactly).  The gradient with respect to an fp32 input
 * is taken as that with respect to its bf16 rounding.
 *  q, o, dout, dq [B,Sq,H,D] and k, v, dk, dv [B,Sk,H_kv,D]: device fp32,
 *    element strides as for bsa_bwd, 16-byte aligned rows.
 *  lse, bs, mask_t, full_t, mask_mod, kv_valid, softmax_scale: as for bsa_bwd.
 *  work: device scratch, 16-byte aligned, of
 *    4*ceil((B*H*Sq + B*H_kv*ceil(Sk/block_kv))/4) + 2*(B*Sq*H*D + B*Sk*H_kv*D)
 *    4-byte entries (bsa_bwd's workspace, then the bf16 copies of the eight
 *    tensors), overwritten.
 * Errors and determinism as bsa_bwd. */
bsa_status bsa_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                       const float* lse, const float* dout, float* dq, float* dk, float* dv,
                       int32_t B, int32_t H, int32_t H_kv, int32_t Sq, int32_t Sk, int32_t D,
                       const int64_t q_str[3], const int64_t k_str[3], const int64_t v_str[3],
                       const int64_t o_str[3], const bsa_block_sparse* bs,
                       const bsa_block_list* mask_t, const bsa_block_list* full_t,
                       bsa_mask_mod mask_mod, const int32_t* kv_valid, float softmax_scale,
                       float* work, hipStream_t stream);

/* Backward of the proxy-compensated forward (bsa_fwd with bs->proxy_k and
 * proxy_v; the PrimTS page, "proxy-compensated block-sparse attention",
 * flashinfer pull request 4872: description, proxy paragraph; the backward
 * is that forward's derivative).  That forward is attention over keys rebuilt
 * token by token: each Q block's listed blocks with their own tokens, every
 * other block n as c_n copies of (proxy_k[n], proxy_v[n] / c_n), c_n its
 * token count.  The c_n copies of a key are one key whose exponential is
 * weighted by c_n, so this call builds an extended KV sequence in the
 * workspace (the N blocks of K and V, then one key per block holding its
 * summaries, the value divided by c_n, in chunks of block_kv; a last block
 * shorter than block_kv in a chunk of its own), marks per Q block the chunks
 * holding summaries it takes (the blocks it does not list) and those
 * summaries as bits, and runs bsa_bwd's kernels on it with log2 c_n added to
 * each summary's exponent.  dk, dv are the keys' and values' gradients;
 * dproxy_k[n] is the summary key's dK (the sum over its copies) and
 * dproxy_v[n] its dV over c_n.  Cost: that of the backward over every
 * listed block plus one key per omitted block (on the page's workload,
 * 84 of 512 blocks listed, 1.1-1.2 times the exact-only backward).
 *  q, k, v, o, lse, dout, dq, dk, dv, strides: as for bsa_bwd (bf16).
 *  bs: the forward's lists, block sizes and summaries (proxy_k, proxy_v
 *    [B,N,H_kv,D] with strides proxy_*_str over {batch, block, head});
 *    mask_mod NONE (the route has no element mask).
 *  dproxy_k, dproxy_v: device bf16, the summaries' layout and strides.
 *  work: device scratch, 16-byte aligned, of the size bsa_bwd_proxy_work_size
 *    returns (the extended K/V, its block mask, lists and their KV-major
 *    transposes, the bit sets, and bsa_bwd's workspace), overwritten.
 * Errors and determinism as bsa_bwd. */
bsa_status bsa_bwd_proxy_work_size(int32_t B, int32_t H, int32_t H_kv, int32_t Sq, int32_t Sk,
                                   int32_t D, int32_t block_q, int32_t block_kv,
                                   int64_t* bytes);
bsa_status bsa_bwd_proxy(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         void* dproxy_k, void* dproxy_v, int32_t B, int32_t H, int32_t H_kv,
                         int32_t Sq, int32_t Sk, int32_t D, const int64_t q_str[3],
                         const int64_t k_str[3], const int64_t v_str[3], const int64_t o_str[3],
                         const bsa_block_sparse* bs, float softmax_scale, void* work,
                         hipStream_t stream);

/* bsa_bwd without the `work` argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc.  The row dots (and, when they fit
 * beside them, the dK/dV start order) go to a static device array of
 * BSA_BWD_NOALLOC_MAX_ROWS 4-byte entries (16 MiB) that the library
 * holds on every GPU it runs on until the process ends; its address is looked
 * up once per device on the first call there.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  B*H*Sq above the
 * maximum returns BSA_ERR_UNSUPPORTED.  Every call on one GPU shares that
 * GPU's array, and each call overwrites all of it that it reads before
 * reading it: calls ordered on one stream are safe, calls that overlap on one
 * GPU (unordered streams) race and give undefined results.  Otherwise
 * exactly bsa_bwd (same kernels, bit-identical results). */
#define BSA_BWD_NOALLOC_MAX_ROWS (1 << 22)
bsa_status bsa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int32_t B, int32_t H, int32_t H_kv, int32_t Sq, int32_t Sk, int32_t D,
                           const int64_t q_str[3], const int64_t k_str[3],
                           const int64_t v_str[3], const int64_t o_str[3],
                           const bsa_block_sparse* bs, const bsa_block_list* mask_t,
                           const bsa_block_list* full_t, bsa_mask_mod mask_mod,
                           const int32_t* kv_valid, float softmax_scale, hipStream_t stream);

/* KV-major ("transposed") block lists: the per-KV-block view that a backward
 * pass walks (flash-attention pull request 2224, review thread: the backward
 * needs the block metadata transposed).  cnt: device int32 [B,H,M] and idx:
 * device int32 [B,H,M,N], contiguous, in the format of bsa_mask_to_index
 * (the first cnt entries of a row are read; ids outside [0,N) are skipped).
 * work: device scratch of B*H*N*M bytes, overwritten.  Writes cnt_t: device
 * int32 [B,H,N] (how many Q blocks list KV block j) and idx_t: device int32
 * [B,H,N,M] (those Q-block ids in descending order, then -1).  Convert the
 * mask and full lists separately.  Caller owns every buffer.  Returns
 * BSA_ERR_INVALID_ARGUMENT for negative sizes or a missing pointer,
 * BSA_ERR_HIP if a launch fails.  Bit-exact; deterministic. */
bsa_status bsa_kv_major_lists(const int32_t* cnt, const int32_t* idx, int32_t B, int32_t H,
                              int32_t M, int32_t N, uint8_t* work, int32_t* cnt_t,
                              int32_t* idx_t, hipStream_t stream);

/* Backward of the packed varlen forward (bsa_varlen_fwd's layout,
 * flash-attention pull request 2224: its review thread names the backward
 * over transposed metadata across the varlen features).  Each sequence is an
 * independent problem with sequence-local ids, so the gradients are those of
 * bsa_bwd per sequence (same formulas, bf16, same D set, same mask_mods).
 *  q, o, dout, dq [total_q,H,D] and k, v, dk, dv [total_k,H_kv,D]: device
 *    bf16, element strides {token, head} (q_str also describes dq, k_str dk,
 *    v_str dv, o_str dout), head_dim stride 1, 16-byte aligned rows.
 *  lse: the varlen forward's LSE, device fp32 [H,total_q] contiguous.
 *  cu_seqlens_q/k, cu_total_m_blocks, block_idx_offsets, total_m_blocks,
 *    total_q: as for bsa_varlen_fwd (device int32 arrays of B+1 entries).
 *  cu_total_kv_blocks: device int32 [B+1], [0, cumsum ceil(seqlen_k(b)/block_kv)]
 *    (bsa_varlen_offsets with the Q and KV roles swapped gives it as its
 *    cu_total_m_blocks), total_kv_blocks its last entry.
 *  bs: the forward's lists (cnt [H,total_m_blocks], idx [H,total_n_blocks]),
 *    block sizes and window.
 *  mask_t / full_t: their KV-major transposes (bsa_varlen_kv_major_lists):
 *    cnt [H,total_kv_blocks] through cnt_stride[1] (head) and cnt_stride[2]
 *    (global KV block), idx [H,total_n_blocks] through idx_stride[1] (head)
 *    and idx_stride[3] (slot), row (b, j) at slot block_idx_offsets[b] +
 *    j*num_m(b); cnt == NULL: absent.
 *  kv_valid, kv_valid_ld: as for bsa_varlen_fwd (per sequence-local KV block).
 *  work: device scratch of H*total_q + H_kv*total_kv_blocks 4-byte entries
 *    (fp32 row dots, then the int32 dK/dV start order), overwritten.
 * dq and dk, dv are overwritten on every token of the sequences (zero where
 * nothing is listed).  Errors as bsa_bwd.  Deterministic: no atomics. */
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
                          float* work, hipStream_t stream);

/* KV-major lists in the packed varlen layout (the transposed metadata of the
 * varlen backward, flash-attention pull request 2224 review thread).  cnt:
 * device int32 [H,total_m_blocks] and idx [H,total_n_blocks], contiguous, as
 * bsa_varlen_mask_to_index writes them (row (b,i) at block_idx_offsets[b] +
 * i*num_n(b); ids outside [0, num_n(b)) and entries past cnt are skipped).
 * cu_total_m_blocks, cu_total_kv_blocks, block_idx_offsets: device int32
 * [B+1] as for bsa_varlen_bwd.  work: device scratch of H*total_n_blocks
 * bytes, overwritten.  Writes cnt_t: device int32 [H,total_kv_blocks] (row
 * (b,j) at cu_total_kv_blocks[b] + j: how many Q blocks of sequence b list
 * its KV block j) and idx_t: device int32 [H,total_n_blocks] (row (b,j) at
 * block_idx_offsets[b] + j*num_m(b), width num_m(b): those sequence-local
 * Q-block ids in descending order, then -1).  Convert the mask and full
 * lists separately.  Caller owns every buffer.  Returns
 * BSA_ERR_INVALID_ARGUMENT for negative sizes or a missing pointer,
 * BSA_ERR_HIP if a launch fails.  Bit-exact; deterministic. */
bsa_status bsa_varlen_kv_major_lists(const int32_t* cnt, const int32_t* idx, int32_t H, int32_t B,
                                     const int32_t* cu_total_m_blocks,
                                     const int32_t* cu_total_kv_blocks,
                                     const int32_t* block_idx_offsets, int32_t total_m_blocks,
                                     int32_t total_kv_blocks, int32_t total_n_blocks,
                                     uint8_t* work, int32_t* cnt_t, int32_t* idx_t,
                                     hipStream_t stream);

/* Packed UInt32 block bitmap -> block lists (the bitmap input of the PrimTS
 * page, "proxy-compensated block-sparse attention", flashinfer pull request
 * 4872: description and test notes).  words: device uint32 [B,Hkv,M,W]
 * contiguous, W = ceil(N/32), one row per (batch, KV head, Q block); bit j
 * (value 1<<j) of word w selects KV block 32*w+j, and bits at or past N in
 * the final word are padding and ignored.  Q head h (H a multiple of Hkv)
 * takes the row of KV head h/(H/Hkv).  Writes cnt: device int32 [B,H,M] and
 * idx: device int32 [B,H,M,N] in the format of bsa_mask_to_index, so a
 * forward over these lists equals one over the lists of the same selection
 * given as a dense mask, bit for bit.  N == 0 writes cnt only and reads no
 * words.  Caller owns every buffer.  Returns BSA_ERR_INVALID_ARGUMENT for
 * negative sizes, H not a multiple of Hkv, or a missing pointer; BSA_ERR_HIP
 * if the launch fails.  Bit-exact; deterministic. */
bsa_status bsa_bitmask_to_index(const uint32_t* words, int32_t B, int32_t Hkv, int32_t H,
                                int32_t M, int32_t N, int32_t* cnt, int32_t* idx,
                                hipStream_t stream);

/* The same conversion for the packed varlen layout.  mask: device uint8
 * [H,total_n_blocks] laid out like idx (row (b,m) of head h at
 * block_idx_offsets[b] + m*num_n(b), width num_n(b)).  Writes cnt [H,total_m_blocks]
 * and idx [H,total_n_blocks] (device int32, contiguous).  num_n(b) is
 * recovered as (block_idx_offsets[b+1]-block_idx_offsets[b]) /
 * (cu_total_m_blocks[b+1]-cu_total_m_blocks[b]). */
bsa_status bsa_varlen_mask_to_index(const uint8_t* mask, int32_t H, int32_t B,
                                    const int32_t* cu_total_m_blocks,
                                    const int32_t* block_idx_offsets,
                                    int32_t total_m_blocks, int32_t total_n_blocks,
                                    int32_t* cnt, int32_t* idx, hipStream_t stream);

/* Host-only integer bookkeeping of the packed varlen layout (PR #2224):
 *   num_m(b) = ceil(seqlens_q[b]/block_q), num_n(b) = ceil(seqlens_k[b]/block_kv),
 *   cu_total_m_blocks = [0, cumsum num_m], block_idx_offsets = [0, cumsum num_m*num_n].
 * All pointers are host memory; the two outputs have B+1 entries.  Returns
 * BSA_ERR_INVALID_ARGUMENT on negative lengths, non-positive block sizes or
 * int32 overflow.  Touches no device. */
bsa_status bsa_varlen_offsets(const int32_t* seqlens_q, const int32_t* seqlens_k, int32_t B,
                              int32_t block_q, int32_t block_kv,
                              int32_t* cu_total_m_blocks, int32_t* block_idx_offsets,
                              int32_t* total_m_blocks, int32_t* total_n_blocks);

/* Split logical KV blocks into `factor` child tiles of `child` tokens
 * (FastVideo PR #1354: 256-token blocks run as 128-token tiles).
 * block_mask: device uint8 [R,NL] (R rows, e.g. B*H*M); block_valid: device
 * int32 [NL] valid-token counts in [0, factor*child].  Child s of block j
 * holds clamp(block_valid[j] - s*child, 0, child) tokens.  Writes device
 * uint8 full [R,NL*factor] (selected and child full), part [R,NL*factor]
 * (selected and 0 < size < child) and int32 kv_valid [NL*factor].
 * Counts outside the range are clamped the same way. */
bsa_status bsa_expand_kv_blocks(const uint8_t* block_mask, const int32_t* block_valid,
                                int32_t R, int32_t NL, int32_t factor, int32_t child,
                                uint8_t* full, uint8_t* part, int32_t* kv_valid,
                                hipStream_t stream);

/* Block classification of an element mask_mod, the role of flash-attention's
 * compute_block_sparsity (PR #2224 description and review thread): for Q block
 * m (rows [m*block_q, min((m+1)*block_q, Sq))) and KV block n (columns
 * [n*block_kv, min((n+1)*block_kv, Sk))) writes
 *   full[m,n] = 1 if mask_mod keeps every element of the block,
 *   part[m,n] = 1 if it keeps some but not all,
 *   both 0    if it keeps none,
 * as device uint8 [ceil(Sq/block_q), ceil(Sk/block_kv)] row-major masks.
 * With bsa_mask_to_index they become the full and mask lists whose forward
 * equals dense attention under the element mask (mask_mod applied to the
 * mask list).  mask_mod: BSA_MASK_NONE (every block full), BSA_MASK_CAUSAL,
 * BSA_MASK_LOCAL (window_left, window_right as in bsa_block_sparse) or
 * BSA_MASK_KV_VALID_COUNT (kv_valid: device int32 [ceil(Sk/block_kv)], else
 * ignored).  Sq, Sk >= 0, block sizes > 0.  Bit-exact; no synchronisation. */
bsa_status bsa_block_sparsity(bsa_mask_mod mask_mod, int32_t window_left, int32_t window_right,
                              const int32_t* kv_valid, int32_t Sq, int32_t Sk, int32_t block_q,
                              int32_t block_kv, uint8_t* full, uint8_t* part,
                              hipStream_t stream);

/* Static string for a status code. */
const char* bsa_status_str(bsa_status s);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
