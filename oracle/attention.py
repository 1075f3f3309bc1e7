"""CPU fp64 oracle for the block-sparse attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg use it.  It shares no code with the HIP library.

What is computed (flash-attention PR #2224, PR description: per (batch,
head, Q block) the kernel visits the KV blocks of a mask list and of a full
list; FastVideo PR #1354, review thread: the valid-count mask_mod; "Dense
FlashAttention vs Block-Sparse Attention", sections 1-4: only selected KV
blocks are computed):

  For batch b, head h (KV head h*Hkv//H), row r and its Q block i = r // bq,
  the visible columns are
      C_r = {c < Sk : c//bk in FULL[b,h,i]}
          U {c < Sk : c//bk in PART[b,h,i] and mask_mod(r, c)}
  s_rc = scale * <q_r, k_c>,  LSE_r = ln sum_{c in C_r} exp(s_rc),
  O_r  = sum_{c in C_r} exp(s_rc - LSE_r) v_c;  empty C_r -> O_r = 0, LSE_r = -inf.

The attention is written as the exact two-pass softmax over the gathered
columns (max, exp, sum, divide), deliberately not the kernel's online
recurrence.  All arithmetic is float64; callers pass inputs already rounded
to the kernel's input precision.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .metadata import cdiv, varlen_offsets

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KV_VALID_COUNT = 2
MASK_LOCAL = 3


def mask_mod_keep(mask_mod: int, rows: np.ndarray, cols: np.ndarray,
                  block_kv: int, kv_valid: Optional[np.ndarray],
                  window: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """Element mask of a mask-list block, keep[r, c] for the given absolute
    (sequence-local) row and column ids.

    causal: keep c <= r (q_idx >= kv_idx).  kv valid count (FastVideo PR
    #1354 review: kv_blk = n // block, kv_off = n % block, valid =
    kv_sizes[kv_blk]): keep kv_off < valid.  local ("Dense FlashAttention vs
    Block-Sparse Attention", section 6: the causal/local range a selected
    block must fall in), window = (left, right) in tokens: keep
    r - left <= c <= r + right; a negative bound is unbounded, so (-1, 0) is
    causal and (-1, -1) keeps everything.
    """
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    if mask_mod == MASK_NONE:
        return np.ones((rows.size, cols.size), bool)
    if mask_mod == MASK_CAUSAL:
        return cols[None, :] <= rows[:, None]
    if mask_mod == MASK_KV_VALID_COUNT:
        if kv_valid is None:
            raise ValueError("kv valid-count mask needs kv_valid")
        keep = (cols % block_kv) < np.asarray(kv_valid)[cols // block_kv]
        return np.broadcast_to(keep[None, :], (rows.size, cols.size)).copy()
    if mask_mod == MASK_LOCAL:
        if window is None:
            raise ValueError("local mask needs window=(left, right)")
        left, right = window
        d = rows[:, None].astype(np.int64) - cols[None, :].astype(np.int64)  # r - c
        keep = np.ones(d.shape, bool)
        if left >= 0:
            keep &= d <= left
        if right >= 0:
            keep &= -d <= right
        return keep
    raise ValueError(f"unknown mask_mod {mask_mod}")


def block_sparsity(mask_mod: int, Sq: int, Sk: int, block_q: int, block_kv: int,
                   window: Optional[Tuple[int, int]] = None,
                   kv_valid: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Classify every (Q block m, KV block n) of an Sq x Sk problem under an
    element mask_mod, the way flash-attention's compute_block_sparsity turns a
    mask_mod into block-sparse tensors (PR #2224 description and review):
    full[m, n] = 1 when every element of the block (clipped to Sq x Sk) is
    kept, part[m, n] = 1 when some but not all are, both 0 when none is.
    Element by element over each block; returns uint8 [M, N] masks."""
    M, N = cdiv(Sq, block_q), cdiv(Sk, block_kv)
    full = np.zeros((M, N), np.uint8)
    part = np.zeros((M, N), np.uint8)
    for m in range(M):
        rows = np.arange(m * block_q, min((m + 1) * block_q, Sq))
        for n in range(N):
            cols = np.arange(n * block_kv, min((n + 1) * block_kv, Sk))
            keep = mask_mod_keep(mask_mod, rows, cols, block_kv, kv_valid, window)
            if keep.all():
                full[m, n] = 1
            elif keep.any():
                part[m, n] = 1
    return full, part


def _softmax_rows(S: np.ndarray, V: np.ndarray):
    """Two-pass softmax over rows of S (entries -inf are hidden) times V.
    Returns (O, LSE, weights); rows with no visible entry give 0, -inf, 0."""
    m, n = S.shape
    O = np.zeros((m, V.shape[1]), np.float64)
    lse = np.full(m, -np.inf, np.float64)
    W = np.zeros((m, n), np.float64)
    if n == 0:
        return O, lse, W
    mx = S.max(axis=1)
    live = mx > -np.inf
    if live.any():
        E = np.exp(S[live] - mx[live, None])
        den = E.sum(axis=1)
        W[live] = E / den[:, None]
        O[live] = W[live] @ V
        lse[live] = mx[live] + np.log(den)
    return O, lse, W


def _q_block(q, k, v, b, h, i, full_row, part_row, bq, bk, Sq, Sk, mask_mod,
             kv_valid, scale, Hkv, H, want_weights=False, window=None):
    """One (b, h, Q block i): gather the listed KV blocks, mask, softmax."""
    hk = h * Hkv // H
    r0, r1 = i * bq, min((i + 1) * bq, Sq)
    rows = np.arange(r0, r1)
    cols_parts, keep_parts = [], []
    for j in range(len(full_row)):
        if full_row[j] and part_row[j]:
            raise ValueError(f"block ({b},{h},{i},{j}) is in both lists")
        if not (full_row[j] or part_row[j]):
            continue
        c0, c1 = j * bk, min((j + 1) * bk, Sk)
        if c0 >= c1:
            continue
        cols = np.arange(c0, c1)
        if full_row[j]:
            keep = np.ones((rows.size, cols.size), bool)
        else:
            keep = mask_mod_keep(mask_mod, rows, cols, bk, kv_valid, window)
        cols_parts.append(cols)
        keep_parts.append(keep)
    if cols_parts:
        C = np.concatenate(cols_parts)
        KEEP = np.concatenate(keep_parts, axis=1)
    else:
        C = np.zeros(0, np.int64)
        KEEP = np.zeros((rows.size, 0), bool)
    S = scale * (q[b, r0:r1, h, :] @ k[b, C, hk, :].T)
    S = np.where(KEEP, S, -np.inf)
    O, lse, W = _softmax_rows(S, v[b, C, hk, :])
    if want_weights:
        return rows, O, lse, W, C
    return rows, O, lse


def blocksparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                          full: np.ndarray, part: np.ndarray, block_q: int,
                          block_kv: int, mask_mod: int, scale: float,
                          kv_valid: Optional[np.ndarray] = None,
                          q_blocks: Optional[Iterable[Tuple[int, int, int]]] = None,
                          window: Optional[Tuple[int, int]] = None):
    """Batched block-sparse attention forward in float64.

    q [B,Sq,H,D], k/v [B,Sk,Hkv,D]; full/part dense block masks [B,H,M,N]
    with M = ceil(Sq/block_q), N = ceil(Sk/block_kv).
    q_blocks: optional iterable of (b, h, i) Q blocks to compute (others are
    left as NaN), for sampling large inputs.
    Returns O [B,Sq,H,D] float64 and LSE [B,H,Sq] float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sq, H, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    M, N = cdiv(Sq, block_q), cdiv(Sk, block_kv)
    if full.shape != (B, H, M, N) or part.shape != (B, H, M, N):
        raise ValueError(f"block masks must be {(B, H, M, N)}")
    O = np.full((B, Sq, H, D), np.nan)
    LSE = np.full((B, H, Sq), np.nan)
    if q_blocks is None:
        q_blocks = [(b, h, i) for b in range(B) for h in range(H) for i in range(M)]
    for (b, h, i) in q_blocks:
        rows, o, lse = _q_block(q, k, v, b, h, i, full[b, h, i], part[b, h, i],
                                block_q, block_kv, Sq, Sk, mask_mod, kv_valid,
                                scale, Hkv, H, window=window)
        O[b, rows, h, :] = o
        LSE[b, h, rows] = lse
    return O, LSE


def softmax_weights(q, k, v, full, part, block_q, block_kv, mask_mod, scale,
                    b, h, i, kv_valid=None, window=None):
    """Row softmax weights of one Q block over its gathered columns (for the
    sum-to-one invariant).  Returns (rows, cols, W)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sq, H, D = q.shape
    _, Sk, Hkv, _ = k.shape
    rows, _, _, W, C = _q_block(q, k, v, b, h, i, full[b, h, i], part[b, h, i],
                                block_q, block_kv, Sq, Sk, mask_mod, kv_valid,
                                scale, Hkv, H, want_weights=True, window=window)
    return rows, C, W


def expand_element_mask(full: np.ndarray, part: np.ndarray, block_q: int,
                        block_kv: int, Sq: int, Sk: int, mask_mod: int,
                        kv_valid: Optional[np.ndarray] = None,
                        window: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """Block masks -> dense element mask [B,H,Sq,Sk], element by element with
    plain Python loops (tiny inputs only)."""
    B, H = full.shape[:2]
    out = np.zeros((B, H, Sq, Sk), bool)
    for b in range(B):
        for h in range(H):
            for r in range(Sq):
                for c in range(Sk):
                    i, j = r // block_q, c // block_kv
                    if full[b, h, i, j]:
                        out[b, h, r, c] = True
                    elif part[b, h, i, j]:
                        if mask_mod == MASK_NONE:
                            out[b, h, r, c] = True
                        elif mask_mod == MASK_CAUSAL:
                            out[b, h, r, c] = c <= r
                        elif mask_mod == MASK_KV_VALID_COUNT:
                            out[b, h, r, c] = (c % block_kv) < kv_valid[j]
                        elif mask_mod == MASK_LOCAL:
                            left, right = window
                            out[b, h, r, c] = ((left < 0 or r - c <= left) and
                                               (right < 0 or c - r <= right))
    return out


def dense_attention(q, k, v, elem_mask: Optional[np.ndarray], scale: float):
    """Plain dense softmax attention with an element mask [B,H,Sq,Sk] (None =
    all visible), float64, brute force over the full score matrix."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sq, H, D = q.shape
    _, Sk, Hkv, _ = k.shape
    O = np.zeros((B, Sq, H, D))
    LSE = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            hk = h * Hkv // H
            S = scale * (q[b, :, h, :] @ k[b, :, hk, :].T)
            if elem_mask is not None:
                S = np.where(elem_mask[b, h], S, -np.inf)
            o, lse, _ = _softmax_rows(S, v[b, :, hk, :])
            O[b, :, h, :] = o
            LSE[b, h, :] = lse
    return O, LSE


def varlen_blocksparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                                 seqlens_q: Sequence[int], seqlens_k: Sequence[int],
                                 full: List[np.ndarray], part: List[np.ndarray],
                                 block_q: int, block_kv: int, mask_mod: int,
                                 scale: float, kv_valid=None,
                                 q_blocks: Optional[Iterable[Tuple[int, int, int]]] = None,
                                 window: Optional[Tuple[int, int]] = None):
    """Packed varlen forward (PR #2224): each sequence b is an independent
    batch-1 problem with sequence-local row/column ids.  q [Tq,H,D],
    k/v [Tk,Hkv,D]; full[b]/part[b] dense per-sequence block masks [H,M_b,N_b].
    kv_valid (valid-count mask_mod): one array of counts shared by every
    sequence, or one per sequence (a list, or the rows of a 2-D array), each
    indexed by the sequence-local KV block id.
    q_blocks: optional (b, h, i) with sequence-local i.  Returns O [Tq,H,D],
    LSE [H,Tq]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Tq, H, D = q.shape
    O = np.full((Tq, H, D), np.nan)
    LSE = np.full((H, Tq), np.nan)
    cq = np.concatenate([[0], np.cumsum(seqlens_q)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(seqlens_k)]).astype(np.int64)
    varlen_offsets(seqlens_q, seqlens_k, block_q, block_kv)  # shape checks
    sel = None
    if q_blocks is not None:
        sel = {}
        for (b, h, i) in q_blocks:
            sel.setdefault(b, []).append((0, h, i))
    for b in range(len(seqlens_q)):
        if sel is not None and b not in sel:
            continue
        qb = q[None, cq[b]:cq[b + 1]]
        kb = k[None, ck[b]:ck[b + 1]]
        vb = v[None, ck[b]:ck[b + 1]]
        per_seq = kv_valid is not None and (isinstance(kv_valid, (list, tuple)) or
                                            np.ndim(kv_valid) == 2)
        kvb = np.asarray(kv_valid[b]) if per_seq else kv_valid
        o, lse = blocksparse_attention(qb, kb, vb, full[b][None], part[b][None],
                                       block_q, block_kv, mask_mod, scale, kvb,
                                       q_blocks=None if sel is None else sel[b],
                                       window=window)
        O[cq[b]:cq[b + 1]] = o[0]
        LSE[:, cq[b]:cq[b + 1]] = lse[0]
    return O, LSE
