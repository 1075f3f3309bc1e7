"""Pins for the attention oracle (CPU only).

Independent anchors: brute-force dense attention over an element mask built
element by element; torch's scaled_dot_product_attention (float64, CPU) as a
library routine for dense, causal and boolean-masked attention; scipy's
logsumexp for LSE; closed forms (one visible key, all-zero queries, empty
rows); row weights summing to one; list-semantics identities.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
import workloads

NONE, CAUSAL, KVV = oracle.MASK_NONE, oracle.MASK_CAUSAL, oracle.MASK_KV_VALID_COUNT


def _rand(rng, B, Sq, Sk, H, Hkv, D):
    q = rng.standard_normal((B, Sq, H, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    return q, k, v


def _rand_lists(rng, B, H, M, N, p_full=0.4, p_part=0.3):
    u = rng.random((B, H, M, N))
    full = u < p_full
    part = (u >= p_full) & (u < p_full + p_part)
    return full, part


def _sdpa(q, k, v, attn_mask=None, is_causal=False, scale=None):
    """torch SDPA in float64 on CPU; q [B,S,H,D] -> O [B,S,H,D]."""
    H, Hkv = q.shape[2], k.shape[2]
    rep = H // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, rep, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, rep, axis=2)).permute(0, 2, 1, 3)
    am = None if attn_mask is None else torch.from_numpy(attn_mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am,
                                                         is_causal=is_causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("mask_mod", [NONE, CAUSAL, KVV])
@pytest.mark.parametrize("shape", [(2, 70, 90, 2, 1, 16, 32, 16), (1, 64, 64, 4, 2, 8, 16, 16),
                                   (1, 33, 100, 1, 1, 8, 8, 24)])
def test_gathered_equals_bruteforce_dense(mask_mod, shape):
    B, Sq, Sk, H, Hkv, D, bq, bk = shape
    rng = np.random.default_rng(hash((mask_mod,) + shape) % (2 ** 32))
    q, k, v = _rand(rng, B, Sq, Sk, H, Hkv, D)
    M, N = -(-Sq // bq), -(-Sk // bk)
    full, part = _rand_lists(rng, B, H, M, N)
    kv_valid = rng.integers(0, bk + 1, N) if mask_mod == KVV else None
    scale = 1 / math.sqrt(D)
    O, L = oracle.blocksparse_attention(q, k, v, full, part, bq, bk, mask_mod, scale, kv_valid)
    em = oracle.expand_element_mask(full, part, bq, bk, Sq, Sk, mask_mod, kv_valid)
    Od, Ld = oracle.dense_attention(q, k, v, em, scale)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(L), np.isneginf(Ld))
    fin = np.isfinite(Ld)
    np.testing.assert_allclose(L[fin], Ld[fin], rtol=0, atol=1e-12)
    # LSE = logsumexp of the visible scaled scores (scipy)
    for b in range(B):
        for h in range(H):
            S = scale * q[b, :, h] @ k[b, :, h * Hkv // H].T
            ref = logsumexp(np.where(em[b, h], S, -np.inf), axis=1)
            np.testing.assert_allclose(L[b, h], ref, rtol=0, atol=1e-12)


def test_dense_masked_equals_sdpa():
    rng = np.random.default_rng(5)
    B, S, H, D = 2, 48, 3, 16
    q, k, v = _rand(rng, B, S, S, H, H, D)
    em = rng.random((B, H, S, S)) < 0.5
    em[..., 0] = True  # no empty rows: SDPA gives NaN there
    O, _ = oracle.dense_attention(q, k, v, em, 0.3)
    np.testing.assert_allclose(O, _sdpa(q, k, v, attn_mask=em, scale=0.3), atol=1e-12)


def test_all_blocks_full_equals_dense_sdpa():
    rng = np.random.default_rng(6)
    B, Sq, Sk, H, Hkv, D, bq, bk = 2, 100, 130, 4, 2, 32, 32, 64
    q, k, v = _rand(rng, B, Sq, Sk, H, Hkv, D)
    M, N = -(-Sq // bq), -(-Sk // bk)
    full = np.ones((B, H, M, N), bool)
    part = np.zeros_like(full)
    O, L = oracle.blocksparse_attention(q, k, v, full, part, bq, bk, NONE, 1 / math.sqrt(D))
    np.testing.assert_allclose(O, _sdpa(q, k, v), atol=1e-12)


def test_causal_block_layout_equals_causal_sdpa():
    w = workloads.causal_blocks(B=2, H=2, S=256, D=32, bs=64, seed=7)
    O, L = oracle.blocksparse_attention(w.q, w.k, w.v, w.full, w.part, w.block_q, w.block_kv,
                                        w.mask_mod, w.scale)
    ref = _sdpa(w.q.astype(np.float64), w.k.astype(np.float64), w.v.astype(np.float64),
                is_causal=True, scale=w.scale)
    np.testing.assert_allclose(O, ref, atol=1e-12)


def test_closed_forms_one_key_zero_query_empty_row():
    rng = np.random.default_rng(8)
    B, S, H, D, bs = 1, 32, 1, 8, 8
    q, k, v = _rand(rng, B, S, S, H, H, D)
    M = N = S // bs
    full = np.zeros((B, H, M, N), bool)
    part = np.zeros_like(full)
    # Q block 0: only block 0 under causal -> row 0 sees exactly key 0
    part[0, 0, 0, 0] = True
    # Q block 1: all-zero queries over blocks 1 and 3 (full) -> mean of those V rows
    q[0, 8:16] = 0.0
    full[0, 0, 1, [1, 3]] = True
    # Q block 2: nothing listed -> empty rows;  Q block 3: one full block
    full[0, 0, 3, 2] = True
    O, L = oracle.blocksparse_attention(q, k, v, full, part, bs, bs, CAUSAL, 0.5)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(L[0, 0, 0] - 0.5 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14
    cols = list(range(8, 16)) + list(range(24, 32))
    for r in range(8, 16):
        np.testing.assert_allclose(O[0, r, 0], v[0, cols, 0].mean(0), atol=1e-14)
        assert abs(L[0, 0, r] - math.log(16)) < 1e-14
    assert (O[0, 16:24] == 0).all() and np.isneginf(L[0, 0, 16:24]).all()
    assert np.isfinite(L[0, 0, 24:32]).all()


def test_row_weights_sum_to_one():
    w = workloads.sparse_sweep(32, 64, 32, B=1, H=2, S=256, seed=9)
    for i in range(4):
        rows, cols, W = oracle.softmax_weights(w.q, w.k, w.v, w.full, w.part, w.block_q,
                                               w.block_kv, w.mask_mod, w.scale, 0, 1, i)
        np.testing.assert_allclose(W.sum(1), 1.0, rtol=0, atol=1e-12)
        assert (W >= 0).all()


def test_list_semantics_identities():
    rng = np.random.default_rng(10)
    B, S, H, D, bs = 1, 128, 2, 16, 32
    q, k, v = _rand(rng, B, S, S, H, H, D)
    M = N = S // bs
    full, part = _rand_lists(rng, B, H, M, N)
    # full <-> mask list swap changes nothing under mask_mod NONE
    O1, L1 = oracle.blocksparse_attention(q, k, v, full, part, bs, bs, NONE, 0.25)
    O2, L2 = oracle.blocksparse_attention(q, k, v, part, full, bs, bs, NONE, 0.25)
    O3, L3 = oracle.blocksparse_attention(q, k, v, full | part, np.zeros_like(full), bs, bs,
                                          NONE, 0.25)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(O1, O3, atol=1e-13)
    np.testing.assert_allclose(L1, L3, atol=1e-13)
    # a causal mask block strictly below the diagonal equals a full block
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    below = np.broadcast_to(jj < ii, full.shape)
    fa = np.where(below, full | part, False)
    Oa, La = oracle.blocksparse_attention(q, k, v, fa, np.zeros_like(fa), bs, bs, CAUSAL, 0.25)
    Ob, Lb = oracle.blocksparse_attention(q, k, v, np.zeros_like(fa), fa, bs, bs, CAUSAL, 0.25)
    fin = np.isfinite(La)
    np.testing.assert_allclose(np.nan_to_num(Oa), np.nan_to_num(Ob), atol=1e-13)
    np.testing.assert_allclose(La[fin], Lb[fin], atol=1e-13)
    # overlapping lists are rejected
    bad = full.copy()
    bad[0, 0, 0, 0] = True
    pb = np.zeros_like(bad)
    pb[0, 0, 0, 0] = True
    with pytest.raises(ValueError):
        oracle.blocksparse_attention(q, k, v, bad, pb, bs, bs, NONE, 0.25)


def test_valid_count_mask_equals_token_masked_reference():
    # reduced video grid: 6x10x12 tokens in 2x4x4 cubes (32 tokens), 16-token tiles
    w = workloads.video(grid=(6, 10, 12), cube=(2, 4, 4), H=2, D=16, kv_tile=16,
                        topk_frac=0.3, seed=11)
    nc = len(w.cube_valid)
    full, part, kv = oracle.expand_kv_blocks(w.cube_mask, w.cube_valid, 2, 16)
    O, L = oracle.blocksparse_attention(w.q, w.k, w.v, full, part, w.cube_elems, 16, KVV,
                                        w.scale, kv_valid=kv)
    # token-masked reference: key token c is visible to query r iff its cube is
    # selected by r's cube and c is a real (non-padding) token of its cube
    S = nc * w.cube_elems
    cube_of = np.arange(S) // w.cube_elems
    real = (np.arange(S) % w.cube_elems) < w.cube_valid[cube_of]
    em = np.zeros((1, 2, S, S), bool)
    for h in range(2):
        em[0, h] = w.cube_mask[0, h][cube_of][:, cube_of] & real[None, :]
    Od, Ld = oracle.dense_attention(w.q, w.k, w.v, em, w.scale)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(L, Ld, atol=1e-12)


def test_varlen_equals_per_sequence_bruteforce():
    w = workloads.varlen_packed(n_seq=3, H=2, D=16, bs=32, lo=1, hi=150, seed=12)
    O, L = oracle.varlen_blocksparse_attention(w.q, w.k, w.v, w.seqlens_q, w.seqlens_k,
                                               w.full, w.part, w.block_q, w.block_kv,
                                               w.mask_mod, w.scale)
    off = 0
    for b, s in enumerate(w.seqlens_q):
        qb, kb, vb = (x[None, off:off + s].astype(np.float64) for x in (w.q, w.k, w.v))
        em = oracle.expand_element_mask(w.full[b][None], w.part[b][None], 32, 32, s, s, CAUSAL)
        Od, Ld = oracle.dense_attention(qb, kb, vb, em, w.scale)
        np.testing.assert_allclose(O[off:off + s], Od[0], atol=1e-12)
        np.testing.assert_allclose(L[:, off:off + s], Ld[0], atol=1e-12)
        # the same masked attention through torch SDPA (every row sees its diagonal key)
        np.testing.assert_allclose(Od, _sdpa(qb, kb, vb, attn_mask=em, scale=w.scale), atol=1e-12)
        off += s


def test_sampled_q_blocks_match_full_run():
    w = workloads.sparse_sweep(32, 128, 112, B=1, H=2, S=500, seed=13)
    O, L = oracle.blocksparse_attention(w.q, w.k, w.v, w.full, w.part, w.block_q, w.block_kv,
                                        w.mask_mod, w.scale)
    picks = [(0, 1, 3), (0, 0, 0)]
    Os, Ls = oracle.blocksparse_attention(w.q, w.k, w.v, w.full, w.part, w.block_q,
                                          w.block_kv, w.mask_mod, w.scale, q_blocks=picks)
    for (b, h, i) in picks:
        r = slice(i * 128, min(500, (i + 1) * 128))
        np.testing.assert_array_equal(Os[b, r, h], O[b, r, h])
        np.testing.assert_array_equal(Ls[b, h, r], L[b, h, r])


def test_varlen_per_sequence_valid_counts_equal_bruteforce():
    # packed batch under the valid-count mask_mod with counts of its own per
    # sequence: each sequence equals brute-force dense attention over the
    # element mask expanded with that sequence's counts, and SDPA with it
    w = workloads.varlen_valid_count(n_seq=3, H=2, D=16, bq=48, bk=32, lo=20, hi=150, seed=21)
    O, L = oracle.varlen_blocksparse_attention(w.q, w.k, w.v, w.seqlens_q, w.seqlens_k,
                                               w.full, w.part, w.block_q, w.block_kv,
                                               w.mask_mod, w.scale, kv_valid=w.kv_valid)
    assert np.isfinite(O).all()
    off = 0
    for b, s in enumerate(w.seqlens_q):
        qb, kb, vb = (x[None, off:off + s].astype(np.float64) for x in (w.q, w.k, w.v))
        em = oracle.expand_element_mask(w.full[b][None], w.part[b][None], 48, 32, s, s, KVV,
                                        kv_valid=w.kv_valid[b])
        Od, Ld = oracle.dense_attention(qb, kb, vb, em, w.scale)
        np.testing.assert_allclose(O[off:off + s], Od[0], atol=1e-12)
        np.testing.assert_allclose(L[:, off:off + s], Ld[0], atol=1e-12)
        live = em.any(-1)[0]  # rows with a visible key (SDPA gives NaN on empty rows)
        Os = _sdpa(qb, kb, vb, attn_mask=np.where(live[:, :, None], em[0], True)[None],
                   scale=w.scale)
        np.testing.assert_allclose(Od[0][live.T], Os[0][live.T], atol=1e-12)
        off += s
    # the counts are per sequence: giving every sequence the first one's row
    # (padded) changes the result wherever a later sequence's counts differ
    shared = np.concatenate([w.kv_valid[0], np.full(64, 32, np.int32)])
    O2, _ = oracle.varlen_blocksparse_attention(w.q, w.k, w.v, w.seqlens_q, w.seqlens_k,
                                                w.full, w.part, w.block_q, w.block_kv,
                                                w.mask_mod, w.scale, kv_valid=shared)
    assert not np.allclose(np.nan_to_num(O2), np.nan_to_num(O))
