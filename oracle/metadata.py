"""Metadata oracle: block-mask -> index lists, packed bitmaps, varlen
offsets, KV-block expansion.  Pure integer work, plain Python/numpy, bit-exact by definition.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg use it.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def mask_to_index(mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Boolean block mask -> (cnt, idx), one row per leading index.

    Follows the conversion the Block-Sparse-Attention interface performs
    ("Dense FlashAttention vs Block-Sparse Attention", section 2: a boolean
    block-mask row becomes the selected KV-block ids in reversed order,
    padded with -1).  mask: [..., N], any nonzero entry counts as selected.
    Returns cnt int32 [...] and idx int32 [..., N].
    """
    mask = np.asarray(mask)
    lead, N = mask.shape[:-1], mask.shape[-1]
    flat = mask.reshape(int(np.prod(lead, dtype=np.int64)), N)
    cnt = np.zeros(flat.shape[0], np.int32)
    idx = np.full((flat.shape[0], N), -1, np.int32)
    for r in range(flat.shape[0]):
        sel = [j for j in range(N - 1, -1, -1) if flat[r, j] != 0]
        cnt[r] = len(sel)
        idx[r, :len(sel)] = sel
    return cnt.reshape(lead), idx.reshape(lead + (N,))


def bitmask_to_mask(words: np.ndarray, N: int, H: int | None = None) -> np.ndarray:
    """Packed UInt32 block bitmap -> boolean block mask.

    Follows the bitmap input of the PrimTS page ("proxy-compensated
    block-sparse attention", flashinfer pull request 4872: the description's
    bitmask paragraph and the test commit's notes): one row of 32-bit words
    per (batch, KV head, Q block),
    each bit selecting one KV block; bits at or beyond N in the final word
    are padding and are ignored.  Reading taken for the bit order, which the
    pages leave open: bit j (value 2**j) of word w selects KV block 32*w + j.

    words: integer array [B, Hkv, M, W] with W = ceil(N/32), any integer
    dtype holding the 32-bit pattern.  H: number of Q heads (a multiple of
    Hkv, default Hkv); Q head h reads the row of KV head h // (H // Hkv).
    Returns bool [B, H, M, N].
    """
    w = np.asarray(words).astype(np.int64) & 0xFFFFFFFF
    B, Hkv, M, W = w.shape
    if W != cdiv(N, 32):
        raise ValueError(f"{W} words per row for {N} blocks")
    H = Hkv if H is None else H
    if Hkv == 0 or H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    n = np.arange(N)
    bits = ((w[..., n // 32] >> (n % 32)) & 1).astype(bool)  # [B, Hkv, M, N]
    group = H // Hkv
    return bits[:, np.arange(H) // group]


def bitmask_to_index(words: np.ndarray, N: int, H: int | None = None):
    """Packed bitmap -> the (cnt, idx) block lists of mask_to_index: the
    bitmap and index formats describe the same selection."""
    return mask_to_index(bitmask_to_mask(words, N, H))


def index_to_mask(cnt: np.ndarray, idx: np.ndarray, N: int) -> np.ndarray:
    """Inverse of mask_to_index on the first cnt entries of each row (the
    padding beyond cnt is not read).  Raises on out-of-range or repeated ids."""
    lead = cnt.shape
    c = np.asarray(cnt).reshape(-1)
    ix = np.asarray(idx).reshape(len(c), -1)
    out = np.zeros((len(c), N), bool)
    for r in range(len(c)):
        for s in range(int(c[r])):
            j = int(ix[r, s])
            if not 0 <= j < N or out[r, j]:
                raise ValueError(f"row {r}: bad or repeated block id {j}")
            out[r, j] = True
    return out.reshape(lead + (N,))


def varlen_offsets(seqlens_q: Sequence[int], seqlens_k: Sequence[int],
                   block_q: int, block_kv: int):
    """Packed-varlen block bookkeeping, flash-attention PR #2224 ("[CuTe,Flex]
    varlen blocksparsity", PR description, and the review rename of
    cu_total_n_blocks to a cumulative sum of M_b*N_b offsets):

      num_m(b) = ceildiv(seqlen_q[b], block_q)
      num_n(b) = ceildiv(seqlen_k[b], block_kv)
      cu_total_m_blocks = [0, cumsum num_m]          (length B+1)
      block_idx_offsets = [0, cumsum num_m * num_n]  (length B+1)
      total_m_blocks = cu_total_m_blocks[-1], total_n_blocks = block_idx_offsets[-1]

    The sparse block sizes play the role of the pages' tile sizes.
    Returns python int lists (cu_m, offsets, total_m, total_n).
    """
    if len(seqlens_q) != len(seqlens_k):
        raise ValueError("seqlens_q and seqlens_k differ in length")
    cu_m, off = [0], [0]
    for sq, sk in zip(seqlens_q, seqlens_k):
        if sq < 0 or sk < 0:
            raise ValueError("negative sequence length")
        nm, nn = cdiv(sq, block_q), cdiv(sk, block_kv)
        cu_m.append(cu_m[-1] + nm)
        off.append(off[-1] + nm * nn)
    return cu_m, off, cu_m[-1], off[-1]


def pack_varlen_lists(masks: List[np.ndarray], seqlens_q, seqlens_k,
                      block_q: int, block_kv: int):
    """Per-sequence dense block masks [H, M_b, N_b] -> packed lists
    cnt [H, total_m_blocks], idx [H, total_n_blocks] (-1 where unused).

    Row (h, b, m) lives at cnt[h, cu_m[b] + m] and at
    idx[h, offsets[b] + m*N_b : offsets[b] + (m+1)*N_b]  (PR #2224 layout).
    """
    cu_m, off, tm, tn = varlen_offsets(seqlens_q, seqlens_k, block_q, block_kv)
    H = masks[0].shape[0] if masks else 0
    cnt = np.zeros((H, tm), np.int32)
    idx = np.full((H, tn), -1, np.int32)
    for b, m_b in enumerate(masks):
        nm, nn = cdiv(seqlens_q[b], block_q), cdiv(seqlens_k[b], block_kv)
        if m_b.shape != (H, nm, nn):
            raise ValueError(f"sequence {b}: mask shape {m_b.shape} != {(H, nm, nn)}")
        c, ix = mask_to_index(m_b)
        for h in range(H):
            for m in range(nm):
                cnt[h, cu_m[b] + m] = c[h, m]
                base = off[b] + m * nn
                idx[h, base: base + nn] = ix[h, m]
    return cnt, idx


def expand_kv_blocks(block_mask: np.ndarray, block_valid: np.ndarray,
                     factor: int, child: int):
    """Split each logical KV block into `factor` child tiles of `child` rows.

    FastVideo PR #1354 ("VSA-256 fastpath", Summary and the expanded_sizes
    review note) runs 256-token logical KV blocks as 128-token tiles and
    stores the two child sizes interleaved.  Reading (the children are not
    spelled out on the page): child s of a block with v valid tokens holds
    clamp(v - s*child, 0, child) valid tokens.  Children with child valid
    tokens are full blocks, 0 < size < child go to the mask list (valid-count
    mask_mod), size 0 children are dropped.

    block_mask [..., Nl] bool; block_valid int [Nl].
    Returns full [..., Nl*factor], part [..., Nl*factor], kv_valid int32 [Nl*factor].
    """
    block_mask = np.asarray(block_mask, bool)
    Nl = block_mask.shape[-1]
    if len(block_valid) != Nl:
        raise ValueError("block_valid length != number of logical KV blocks")
    sizes = np.zeros(Nl * factor, np.int32)
    for j in range(Nl):
        v = int(block_valid[j])
        if not 0 <= v <= factor * child:
            raise ValueError(f"block {j}: valid count {v} out of range")
        for s in range(factor):
            sizes[j * factor + s] = min(max(v - s * child, 0), child)
    full = np.zeros(block_mask.shape[:-1] + (Nl * factor,), bool)
    part = np.zeros_like(full)
    for jc in range(Nl * factor):
        sel = block_mask[..., jc // factor]
        if sizes[jc] == child:
            full[..., jc] = sel
        elif sizes[jc] > 0:
            part[..., jc] = sel
    return full, part, sizes
