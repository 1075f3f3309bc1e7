"""Seeded synthetic inputs for block-sparse attention forward.

This module only draws random tensors and random *dense block masks*; it
holds none of the attention arithmetic, none of the metadata encodings
(index lists, varlen offsets, 256->128 expansion) and imports neither the
oracle nor the HIP package.  Both sides consume what it returns.

Every workload follows the shapes the pages measure on:

* block-aligned causal BlockMask at B=2, H=4, S=1024 and a head_dim x block
  size sweep (runguoli.com "FlashAttention — CuTe Kernels & Block Sparsity",
  the H200 measurement paragraph of PR #2903);
* packed variable-length batches (flash-attention PR #2224 "[CuTe,Flex]
  varlen blocksparsity", PR description);
* video sparse attention with 4x8x8 = 256-token cubes, partial edge cubes
  and per-KV-block valid-token counts (FastVideo PR #1354, Summary and the
  valid-count mask_mod in the review thread).

Random draw order is always Q, K, V (fp32 N(0,1)) and then the metadata.
Tensors are float32 numpy arrays; callers round them to bf16 (RNE) before
use and both sides read the same rounded values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KV_VALID_COUNT = 2

SWEEP_HEAD_DIMS = (64, 96, 128, 192, 256)
SWEEP_BLOCKS = ((128, 128), (64, 128), (128, 64), (64, 64), (128, 112))


@dataclass
class BatchedWorkload:
    """Batched layout: q [B,Sq,H,D], k/v [B,Sk,Hkv,D] (BSHD, fp32).

    full / part are dense block masks [B,H,M,N] (bool), M=ceil(Sq/bq),
    N=ceil(Sk/bk).  `full` blocks take no element mask; `part` blocks take
    `mask_mod`.  kv_valid (int32 [N]) is the per-KV-block valid-token count
    used by MASK_KV_VALID_COUNT.
    """
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    full: np.ndarray
    part: np.ndarray
    block_q: int
    block_kv: int
    mask_mod: int
    scale: float
    kv_valid: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)


@dataclass
class VarlenWorkload:
    """Packed varlen layout: q/k/v [total_tokens, H, D] (THD, fp32).

    seqlens_q / seqlens_k: python int lists.  full[b] / part[b] are dense
    per-sequence block masks [H, M_b, N_b] with sequence-local block ids.
    kv_valid: per-sequence valid-token counts of the KV blocks (valid-count
    mask_mod only).
    """
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seqlens_q: List[int]
    seqlens_k: List[int]
    full: List[np.ndarray]
    part: List[np.ndarray]
    block_q: int
    block_kv: int
    mask_mod: int
    scale: float
    kv_valid: Optional[List[np.ndarray]] = None  # per sequence, int32 [N_b]


@dataclass
class WindowWorkload:
    """Sliding-window attention input: q/k/v [B,S,H,D] (BSHD, fp32) and the
    local mask_mod's (left, right) window.  No block masks: the lists come
    from classifying the window (bsa_block_sparsity on the GPU side,
    oracle.block_sparsity on the CPU side)."""
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    block_q: int
    block_kv: int
    window: tuple
    scale: float


@dataclass
class VideoWorkload:
    """Video sparse attention input at cube granularity.

    q/k/v: [1, n_cubes*cube_elems, H, D] fp32, cube-major, real tokens first
    inside each cube, padding rows zero.  cube_mask: [1, H, n_cubes, n_cubes]
    bool (per Q cube, its top-k KV cubes).  cube_valid: int32 [n_cubes].
    The attention runs on Q blocks of `cube_elems` rows and on KV tiles of
    `kv_tile` rows; the cube->tile expansion is not done here.
    """
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cube_mask: np.ndarray
    cube_valid: np.ndarray
    cube_elems: int
    kv_tile: int
    scale: float
    grid: tuple
    cube: tuple


def _qkv(rng, shape_q, shape_kv):
    q = rng.standard_normal(shape_q, dtype=np.float32)
    k = rng.standard_normal(shape_kv, dtype=np.float32)
    v = rng.standard_normal(shape_kv, dtype=np.float32)
    return q, k, v


def _cdiv(a, b):
    return -(-a // b)


def tiny(seed: int = 1001) -> BatchedWorkload:
    """B=1, H=1, S=256, D=64 fp32; 64x64 blocks; Bernoulli(0.5) blocks with
    the diagonal forced on; every selected block in the full list."""
    rng = np.random.default_rng(seed)
    B, H, S, D, bs = 1, 1, 256, 64, 64
    q, k, v = _qkv(rng, (B, S, H, D), (B, S, H, D))
    M = N = S // bs
    full = rng.random((B, H, M, N)) < 0.5
    for i in range(M):
        full[:, :, i, i] = True
    part = np.zeros_like(full)
    return BatchedWorkload("tiny", q, k, v, full, part, bs, bs, MASK_NONE,
                           1.0 / math.sqrt(D))


def causal_blocks(B=2, H=4, S=1024, D=128, bs=128, seed: int = 1002) -> BatchedWorkload:
    """Block-aligned causal mask: blocks strictly below the diagonal are full
    blocks, diagonal blocks are mask blocks with the causal mask_mod."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, (B, S, H, D), (B, S, H, D))
    M = N = _cdiv(S, bs)
    ii = np.arange(M)[:, None]
    jj = np.arange(N)[None, :]
    full = np.broadcast_to(jj < ii, (B, H, M, N)).copy()
    part = np.broadcast_to(jj == ii, (B, H, M, N)).copy()
    return BatchedWorkload("causal_blocks", q, k, v, full, part, bs, bs,
                           MASK_CAUSAL, 1.0 / math.sqrt(D))


def _diagonal_blocks(i, bq, bk, Sq, Sk):
    """KV blocks that hold both a causally visible (c <= r) and a causally
    hidden (c > r) element for some row r of Q block i."""
    r0, r1 = i * bq, min((i + 1) * bq, Sq) - 1
    out = []
    for j in range(_cdiv(Sk, bk)):
        c0, c1 = j * bk, min((j + 1) * bk, Sk) - 1
        if c0 <= r1 and c1 > r0:
            out.append(j)
    return out


def sparse_sweep(D: int, bq: int, bk: int, B=2, H=16, S=4096,
                 density: float = 0.25, seed: Optional[int] = None) -> BatchedWorkload:
    """Per Q block: the causal-diagonal KV blocks as causal mask blocks plus
    random other KV blocks as full blocks, floor(density*N) blocks in all."""
    blocks_id = SWEEP_BLOCKS.index((bq, bk)) if (bq, bk) in SWEEP_BLOCKS else 99
    rng = np.random.default_rng([1003, D, blocks_id] if seed is None else seed)
    q, k, v = _qkv(rng, (B, S, H, D), (B, S, H, D))
    M, N = _cdiv(S, bq), _cdiv(S, bk)
    k_total = int(math.floor(density * N))
    full = np.zeros((B, H, M, N), bool)
    part = np.zeros((B, H, M, N), bool)
    for i in range(M):
        diag = _diagonal_blocks(i, bq, bk, S, S)
        others = np.array([j for j in range(N) if j not in diag])
        n_pick = max(k_total - len(diag), 0)
        for b in range(B):
            for h in range(H):
                pick = rng.choice(others, size=n_pick, replace=False)
                full[b, h, i, pick] = True
                part[b, h, i, diag] = True
    return BatchedWorkload(f"sweep_d{D}_bq{bq}_bk{bk}", q, k, v, full, part, bq, bk,
                           MASK_CAUSAL, 1.0 / math.sqrt(D))


def gqa_sweep(D: int, bq: int, bk: int, Hkv: int, hrep: int, B=2, S=4096,
              density: float = 0.25, seed: Optional[int] = None) -> BatchedWorkload:
    """Grouped-query attention: H = Hkv * hrep Q heads over Hkv KV heads, with
    block masks per KV head (full / part [B, Hkv, M, N]) that the hrep Q heads
    of each KV head share, drawn as in sparse_sweep (causal diagonal blocks
    as mask blocks, random other blocks as full blocks, floor(density*N) in
    all).  extra["kv_head_lists"] marks the per-KV-head masks."""
    rng = np.random.default_rng([1009, D, bq, bk, Hkv, hrep] if seed is None else seed)
    H = Hkv * hrep
    q, k, v = _qkv(rng, (B, S, H, D), (B, S, Hkv, D))
    M, N = _cdiv(S, bq), _cdiv(S, bk)
    k_total = int(math.floor(density * N))
    full = np.zeros((B, Hkv, M, N), bool)
    part = np.zeros((B, Hkv, M, N), bool)
    for i in range(M):
        diag = _diagonal_blocks(i, bq, bk, S, S)
        others = np.array([j for j in range(N) if j not in diag], dtype=np.int64)
        n_pick = min(max(k_total - len(diag), 0), others.size)
        for b in range(B):
            for h in range(Hkv):
                full[b, h, i, rng.choice(others, size=n_pick, replace=False)] = True
                part[b, h, i, diag] = True
    return BatchedWorkload(f"gqa_d{D}_bq{bq}_bk{bk}_hkv{Hkv}x{hrep}", q, k, v, full, part, bq,
                           bk, MASK_CAUSAL, 1.0 / math.sqrt(D), extra={"kv_head_lists": True})


def varlen_packed(n_seq=8, H=16, D=128, bs=128, lo=128, hi=8192, p_below=0.3,
                  seed: int = 1004, seqlens: Optional[List[int]] = None) -> VarlenWorkload:
    """Packed batch of n_seq sequences (seqlen_q = seqlen_k ~ U{lo..hi}, or the
    given lengths).  Per sequence and head: diagonal blocks are causal mask
    blocks, each block strictly below the diagonal is a full block with
    probability p_below."""
    rng = np.random.default_rng(seed)
    if seqlens is None:
        seqlens = [int(x) for x in rng.integers(lo, hi + 1, size=n_seq)]
    seqlens = [int(x) for x in seqlens]
    total = sum(seqlens)
    q, k, v = _qkv(rng, (total, H, D), (total, H, D))
    full, part = [], []
    for s in seqlens:
        M = N = _cdiv(s, bs)
        ii = np.arange(M)[:, None]
        jj = np.arange(N)[None, :]
        below = rng.random((H, M, N)) < p_below
        full.append(below & (jj < ii)[None])
        part.append(np.broadcast_to((jj == ii)[None], (H, M, N)).copy())
    return VarlenWorkload("varlen_packed", q, k, v, seqlens, list(seqlens), full, part,
                          bs, bs, MASK_CAUSAL, 1.0 / math.sqrt(D))


def varlen_valid_count(n_seq=6, H=4, D=128, bq=256, bk=128, lo=300, hi=3000, p_sel=0.3,
                       seed: int = 1008) -> VarlenWorkload:
    """Packed varlen batch under the valid-count mask_mod (FastVideo PR #1354
    review thread, in the packed layout of flash-attention PR #2224): each
    sequence's KV blocks hold a random number of real tokens (valid counts
    drawn per sequence and block, the last block never past its sequence
    end).  Each (head, Q block, KV block) is selected with probability p_sel;
    a selected block whose count is the whole block goes to the full list,
    any other to the mask list.  `extra["kv_valid"]` holds the per-sequence
    counts."""
    rng = np.random.default_rng(seed)
    seqlens = [int(x) for x in rng.integers(lo, hi + 1, size=n_seq)]
    total = sum(seqlens)
    q, k, v = _qkv(rng, (total, H, D), (total, H, D))
    full, part, kvv = [], [], []
    for s in seqlens:
        M, N = _cdiv(s, bq), _cdiv(s, bk)
        cap = np.minimum(bk, s - np.arange(N) * bk)
        valid = rng.integers(0, cap + 1).astype(np.int32)  # 0 .. block size (or sequence end)
        whole = rng.random(N) < 0.5
        valid[whole] = cap[whole]
        sel = rng.random((H, M, N)) < p_sel
        is_full = (valid == bk)[None, None, :]
        full.append(sel & is_full)
        part.append(sel & ~is_full)
        kvv.append(valid)
    return VarlenWorkload("varlen_valid_count", q, k, v, seqlens, list(seqlens), full, part,
                          bq, bk, MASK_KV_VALID_COUNT, 1.0 / math.sqrt(D), kv_valid=kvv)


def sliding_window(B=2, H=16, S=8192, D=128, bs=128, window=(1024, 0),
                   seed: int = 1006) -> WindowWorkload:
    """Causal sliding window of `window[0]` keys back (the causal/local range
    of "Dense FlashAttention vs Block-Sparse Attention", section 6) at the
    sweep's batch, head and head_dim scale: 1024 of 8192 keys per row is
    about 12.5 % density, below the 25 % of the sweep."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, (B, S, H, D), (B, S, H, D))
    return WindowWorkload(f"sliding_window_w{window[0]}_{window[1]}", q, k, v, bs, bs,
                          tuple(window), 1.0 / math.sqrt(D))


def proxy_routes(B=1, S=32760, H=12, D=128, bs=64, per_row=84,
                 seed: int = 1007) -> BatchedWorkload:
    """The proxy-route workload of the PrimTS page (its proxy-overhead table):
    B1, 32760 tokens, 12 heads, d128, 64x64 blocks, 84 of the 512 KV blocks
    listed per Q-block row (16.4 %), drawn uniformly per (head, Q block), no
    element mask.  The last KV block holds 56 tokens."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, (B, S, H, D), (B, S, H, D))
    M = N = _cdiv(S, bs)
    full = np.zeros((B, H, M, N), bool)
    for b in range(B):
        for h in range(H):
            for i in range(M):
                full[b, h, i, rng.choice(N, per_row, replace=False)] = True
    return BatchedWorkload(f"proxy_routes_{per_row}of{N}", q, k, v, full, np.zeros_like(full),
                           bs, bs, MASK_NONE, 1.0 / math.sqrt(D))


def _cube_layout(grid, cube):
    """Valid-token count of each cube (cube-major order t, h, w) and, for each
    real token of the grid (t, h, w order), its padded row."""
    nc = [_cdiv(g, c) for g, c in zip(grid, cube)]
    ce = cube[0] * cube[1] * cube[2]
    valid = np.zeros(nc[0] * nc[1] * nc[2], np.int32)
    cid = 0
    for a in range(nc[0]):
        for b in range(nc[1]):
            for c in range(nc[2]):
                valid[cid] = (min(cube[0], grid[0] - a * cube[0]) *
                              min(cube[1], grid[1] - b * cube[1]) *
                              min(cube[2], grid[2] - c * cube[2]))
                cid += 1
    return valid, ce


def video(grid=(30, 48, 52), cube=(4, 8, 8), H=24, D=128, kv_tile=128,
          topk_frac=0.12, seed: int = 1005) -> VideoWorkload:
    """Video-style sparse attention at cube granularity.

    Tokens sit in a padded cube-major buffer (real tokens first in each cube,
    padding zero).  Each Q cube selects its top-k KV cubes by the mean-pooled
    (over real tokens) Q.K score, k = round(topk_frac * n_cubes), ties to the
    lower cube id.
    """
    rng = np.random.default_rng(seed)
    valid, ce = _cube_layout(grid, cube)
    n_cubes = len(valid)
    S = n_cubes * ce
    q, k, v = _qkv(rng, (1, S, H, D), (1, S, H, D))
    pad = np.ones(S, bool)
    for c in range(n_cubes):
        pad[c * ce: c * ce + valid[c]] = False
    q[:, pad] = 0.0
    k[:, pad] = 0.0
    v[:, pad] = 0.0
    # selection scores from mean-pooled real tokens (input generation only)
    qc = q[0].reshape(n_cubes, ce, H, D).astype(np.float64).sum(1) / valid[:, None, None]
    kc = k[0].reshape(n_cubes, ce, H, D).astype(np.float64).sum(1) / valid[:, None, None]
    topk = int(round(topk_frac * n_cubes))
    cube_mask = np.zeros((1, H, n_cubes, n_cubes), bool)
    cols = np.arange(n_cubes)
    for h in range(H):
        sc = qc[:, h, :] @ kc[:, h, :].T
        for i in range(n_cubes):
            order = np.lexsort((cols, -sc[i]))  # by score desc, then id asc
            cube_mask[0, h, i, order[:topk]] = True
    return VideoWorkload("video", q, k, v, cube_mask, valid, ce, kv_tile,
                         1.0 / math.sqrt(D), tuple(grid), tuple(cube))


def config(n: int, **kw):
    """The five named workloads: 1 tiny, 2 causal_blocks, 3 sparse_sweep
    (pass D, bq, bk), 4 varlen_packed, 5 video."""
    return {1: tiny, 2: causal_blocks, 3: sparse_sweep, 4: varlen_packed, 5: video}[n](**kw)
