"""Pins for the local (sliding-window) mask_mod and the block classifier of
the oracle (CPU only).

Independent anchors: the causal and unmasked special cases; the band built
with numpy's tril/triu; the closed-form block classification of a causal
mask on a square block grid; torch's scaled_dot_product_attention (float64,
CPU) with a boolean band mask for the forward over classified lists.
"""
import numpy as np
import pytest
import torch

import oracle

NONE, CAUSAL, KVV, LOCAL = (oracle.MASK_NONE, oracle.MASK_CAUSAL, oracle.MASK_KV_VALID_COUNT,
                            oracle.MASK_LOCAL)


def _band(Sq, Sk, left, right):
    """keep[r, c] for r - left <= c <= r + right (negative = unbounded) via tril/triu."""
    ones = np.ones((Sq, Sk), bool)
    keep = ones.copy()
    if right >= 0:
        keep &= np.tril(ones, k=right)
    if left >= 0:
        keep &= np.triu(ones, k=-left)
    return keep


def test_local_reduces_to_causal_and_none():
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 500, 40)
    cols = rng.integers(0, 500, 50)
    np.testing.assert_array_equal(
        oracle.mask_mod_keep(LOCAL, rows, cols, 64, None, (-1, 0)),
        oracle.mask_mod_keep(CAUSAL, rows, cols, 64, None))
    np.testing.assert_array_equal(
        oracle.mask_mod_keep(LOCAL, rows, cols, 64, None, (-1, -1)),
        oracle.mask_mod_keep(NONE, rows, cols, 64, None))


@pytest.mark.parametrize("left,right", [(0, 0), (5, 0), (0, 7), (31, 17), (-1, 3), (9, -1)])
def test_local_band_matches_tril_triu(left, right):
    Sq, Sk = 45, 60
    keep = oracle.mask_mod_keep(LOCAL, np.arange(Sq), np.arange(Sk), 16, None, (left, right))
    np.testing.assert_array_equal(keep, _band(Sq, Sk, left, right))


def test_block_sparsity_causal_square_closed_form():
    n, b = 7, 32
    full, part = oracle.block_sparsity(CAUSAL, n * b, n * b, b, b)
    m_idx, n_idx = np.indices((n, n))
    np.testing.assert_array_equal(full, (m_idx > n_idx).astype(np.uint8))
    np.testing.assert_array_equal(part, (m_idx == n_idx).astype(np.uint8))


@pytest.mark.parametrize("Sq,Sk,bq,bk,window", [(200, 260, 64, 48, (100, 0)),
                                                (130, 130, 32, 64, (40, 40)),
                                                (96, 300, 64, 128, (-1, 70)),
                                                (257, 129, 128, 64, (1, 1))])
def test_block_sparsity_lists_reproduce_the_element_mask(Sq, Sk, bq, bk, window):
    """The classified lists, expanded element by element with the mask_mod on
    the partial blocks, give back exactly the band; every partial block holds
    both kept and dropped elements and every full block only kept ones."""
    full, part = oracle.block_sparsity(LOCAL, Sq, Sk, bq, bk, window=window)
    assert not (full & part).any()
    band = _band(Sq, Sk, *window)
    em = oracle.expand_element_mask(full[None, None], part[None, None], bq, bk, Sq, Sk, LOCAL,
                                    window=window)[0, 0]
    np.testing.assert_array_equal(em, band)
    for m in range(full.shape[0]):
        for n in range(full.shape[1]):
            blk = band[m * bq:(m + 1) * bq, n * bk:(n + 1) * bk]
            if full[m, n]:
                assert blk.all()
            elif part[m, n]:
                assert blk.any() and not blk.all()
            else:
                assert not blk.any()


def test_block_sparsity_kv_valid_closed_form():
    Sq, Sk, bq, bk = 100, 330, 50, 64
    valid = np.array([64, 0, 10, 64, 63, 9], np.int32)  # last block is 330 - 320 = 10 wide
    full, part = oracle.block_sparsity(KVV, Sq, Sk, bq, bk, kv_valid=valid)
    width = np.minimum(bk, Sk - np.arange(len(valid)) * bk)
    exp_full = valid >= width
    exp_part = (valid > 0) & ~exp_full
    for m in range(full.shape[0]):
        np.testing.assert_array_equal(full[m], exp_full.astype(np.uint8))
        np.testing.assert_array_equal(part[m], exp_part.astype(np.uint8))


@pytest.mark.parametrize("window", [(64, 0), (20, 20), (-1, 33)])
def test_local_forward_equals_sdpa_with_band_mask(window):
    rng = np.random.default_rng(3)
    B, Sq, Sk, H, Hkv, D, bq, bk = 2, 96, 112, 2, 1, 16, 32, 48
    q = rng.standard_normal((B, Sq, H, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    full, part = oracle.block_sparsity(LOCAL, Sq, Sk, bq, bk, window=window)
    M, N = full.shape
    fullb = np.broadcast_to(full.astype(bool), (B, H, M, N))
    partb = np.broadcast_to(part.astype(bool), (B, H, M, N))
    O, L = oracle.blocksparse_attention(q, k, v, fullb, partb, bq, bk, LOCAL, 0.25, window=window)
    band = _band(Sq, Sk, *window)
    assert band.any(axis=1).all()  # every row keeps a key (SDPA would give NaN otherwise)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, H // Hkv, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, H // Hkv, axis=2)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(band), scale=0.25).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(O, ref, atol=1e-12)
    s = 0.25 * np.einsum("bqhd,bkhd->bhqk", q, np.repeat(k, H // Hkv, axis=2))
    s = np.where(band[None, None], s, -np.inf)
    m = s.max(-1, keepdims=True)
    ref_lse = (m + np.log(np.exp(s - m).sum(-1, keepdims=True)))[..., 0]
    np.testing.assert_allclose(L, ref_lse, atol=1e-12)
