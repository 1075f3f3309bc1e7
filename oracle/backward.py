"""Backward of block-sparse attention and its KV-major block lists, float64 (CPU).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg use it.

The pages name the backward pass as the missing half (flash-attention pull
request 2224, description and review thread; FastVideo pull request 1354,
review findings; the tile-fit write-up, results) and say that it walks the
block lists transposed, per KV block.  They print no formula, so this is the
gradient of the forward as defined, written out: with the element mask of
the listed blocks, P = softmax(scale * Q K^T) over the kept keys of each row,
O = P V, and an upstream gradient dO,

    dV = P^T dO
    dP = dO V^T
    D  = rowsum(dO * O)              (= rowsum(P * dP))
    dS = P * (dP - D)
    dQ = scale * dS K
    dK = scale * dS^T Q

summed over the Q heads that share a KV head.  A row that keeps no key has
P = 0 and contributes nothing.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import MASK_NONE, mask_mod_keep
from .metadata import cdiv, mask_to_index


def element_mask(full, part, block_q: int, block_kv: int, Sq: int, Sk: int, mask_mod: int,
                 kv_valid: Optional[np.ndarray] = None,
                 window: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """Block masks [B,H,M,N] -> kept elements [B,H,Sq,Sk]: every element of a
    full block, the mask_mod's elements of a partial block."""
    B, H, M, N = full.shape
    out = np.zeros((B, H, Sq, Sk), bool)
    for b in range(B):
        for h in range(H):
            for i in range(M):
                rows = np.arange(i * block_q, min((i + 1) * block_q, Sq))
                for j in range(N):
                    cols = np.arange(j * block_kv, min((j + 1) * block_kv, Sk))
                    if full[b, h, i, j]:
                        out[b, h, rows[:, None], cols[None, :]] = True
                    elif part[b, h, i, j]:
                        keep = (np.ones((len(rows), len(cols)), bool) if mask_mod == MASK_NONE
                                else mask_mod_keep(mask_mod, rows, cols, block_kv, kv_valid,
                                                   window))
                        out[b, h, rows[:, None], cols[None, :]] = keep
    return out


def blocksparse_attention_bwd(q, k, v, full, part, block_q: int, block_kv: int, mask_mod: int,
                              scale: float, dout, kv_valid=None, window=None):
    """q [B,Sq,H,D], k/v [B,Sk,Hkv,D], dout [B,Sq,H,D]; block masks [B,H,M,N].
    Returns dq [B,Sq,H,D], dk and dv [B,Sk,Hkv,D], float64."""
    q, k, v, dout = (np.asarray(x, np.float64) for x in (q, k, v, dout))
    B, Sq, H, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    M, N = cdiv(Sq, block_q), cdiv(Sk, block_kv)
    if full.shape != (B, H, M, N) or part.shape != (B, H, M, N):
        raise ValueError(f"block masks must be {(B, H, M, N)}")
    keep = element_mask(full, part, block_q, block_kv, Sq, Sk, mask_mod, kv_valid, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            Q, K, V, dO = q[b, :, h], k[b, :, hk], v[b, :, hk], dout[b, :, h]
            S = np.where(keep[b, h], scale * Q @ K.T, -np.inf)
            m = S.max(axis=1, keepdims=True, initial=-np.inf)  # Sk = 0: no key
            has = np.isfinite(m[:, 0])
            E = np.where(keep[b, h], np.exp(S - np.where(has[:, None], m, 0.0)), 0.0)
            den = E.sum(axis=1, keepdims=True)
            P = np.where(has[:, None], E / np.where(den > 0, den, 1.0), 0.0)
            O = P @ V
            dP = dO @ V.T
            Dr = (dO * O).sum(axis=1, keepdims=True)
            dS = P * (dP - Dr)
            dq[b, :, h] = scale * dS @ K
            dk[b, :, hk] += scale * dS.T @ Q
            dv[b, :, hk] += P.T @ dO
    return dq, dk, dv


def kv_major_lists(mask: np.ndarray):
    """Block mask [B,H,M,N] -> the lists of the transposed mask, one row per
    KV block: (cnt [B,H,N], idx [B,H,N,M]) with the Q-block ids that list it,
    in the order of mask_to_index (descending, then -1)."""
    return mask_to_index(np.swapaxes(np.asarray(mask), -1, -2))


def varlen_blocksparse_attention_bwd(q, k, v, seqlens_q, seqlens_k, full, part, block_q: int,
                                     block_kv: int, mask_mod: int, scale: float, dout,
                                     kv_valid=None, window=None):
    """Backward of the packed varlen forward (flash-attention PR #2224
    layout): each sequence is its own batch-1 problem with sequence-local
    row and key ids, so its gradients are those of blocksparse_attention_bwd
    on its slices.  q, dout [Tq,H,D], k/v [Tk,Hkv,D]; full[b]/part[b] dense
    block masks [H,M_b,N_b]; kv_valid as for the varlen forward (one shared
    array, or one per sequence).  Returns dq [Tq,H,D], dk and dv [Tk,Hkv,D]."""
    q, k, v, dout = (np.asarray(x, np.float64) for x in (q, k, v, dout))
    cq = np.concatenate([[0], np.cumsum(seqlens_q)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(seqlens_k)]).astype(np.int64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    per_seq = kv_valid is not None and (isinstance(kv_valid, (list, tuple)) or
                                        np.ndim(kv_valid) == 2)
    for b in range(len(seqlens_q)):
        kvb = np.asarray(kv_valid[b]) if per_seq else kv_valid
        g = blocksparse_attention_bwd(q[None, cq[b]:cq[b + 1]], k[None, ck[b]:ck[b + 1]],
                                      v[None, ck[b]:ck[b + 1]], full[b][None], part[b][None],
                                      block_q, block_kv, mask_mod, scale,
                                      dout[None, cq[b]:cq[b + 1]], kvb, window)
        dq[cq[b]:cq[b + 1]] = g[0][0]
        dk[ck[b]:ck[b + 1]] = g[1][0]
        dv[ck[b]:ck[b + 1]] = g[2][0]
    return dq, dk, dv


def varlen_kv_major_lists(masks, seqlens_q, seqlens_k, block_q: int, block_kv: int):
    """Per-sequence block masks [H,M_b,N_b] -> KV-major lists in the packed
    varlen layout with the roles of Q and KV blocks swapped: cnt_t
    [H, sum_b N_b] (row (b, j) at sum_{b'<b} N_b' + j) and idx_t
    [H, sum_b M_b*N_b] (row (b, j) at offsets[b] + j*M_b, width M_b), holding
    the sequence-local Q-block ids that list KV block j, descending, then -1.
    The offsets sum M_b*N_b, the same as the forward's."""
    from .metadata import pack_varlen_lists
    return pack_varlen_lists([np.swapaxes(np.asarray(m), -1, -2) for m in masks],
                             seqlens_k, seqlens_q, block_kv, block_q)
