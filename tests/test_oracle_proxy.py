"""Pins for the proxy-compensated oracle (CPU only).

Independent anchors: torch's scaled_dot_product_attention (float64, CPU) over
(a) the original K/V when every KV block holds identical tokens, where the
mean-K / summed-V proxy with token-mass weighting is exact, and (b) K/V whose
omitted blocks are rebuilt token by token from the summaries; numpy reshape
means and sums for the summaries; the all-selected case, which must reduce
to plain attention.
"""
import numpy as np
import pytest
import torch

import oracle


def _sdpa(q, k, v, scale, mask=None):
    """q [Sq,H,D], k/v [Sk,H,D] float64 -> O [Sq,H,D], LSE [H,Sq]."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).permute(1, 0, 2) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    s = scale * torch.einsum("hqd,hkd->hqk", tq, tk)
    return o.permute(1, 0, 2).numpy(), torch.logsumexp(s, dim=-1).numpy()


def _inputs(seed, B, Sq, Sk, H, Hkv, D, bq, bk, density):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, H, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    M, N = -(-Sq // bq), -(-Sk // bk)
    sel = rng.random((B, H, M, N)) < density
    split = rng.random((B, H, M, N)) < 0.5
    return q, k, v, sel & split, sel & ~split


def test_summaries_are_block_means_and_sums():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((2, 100, 3, 8))
    v = rng.standard_normal((2, 100, 3, 8))
    kbar, vsum = oracle.block_summaries(k, v, 32)
    assert kbar.shape == (2, 4, 3, 8)
    np.testing.assert_allclose(kbar[:, :3], k[:, :96].reshape(2, 3, 32, 3, 8).mean(axis=2), atol=1e-14)
    np.testing.assert_allclose(vsum[:, :3], v[:, :96].reshape(2, 3, 32, 3, 8).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(kbar[:, 3], k[:, 96:].sum(axis=1) / 4, atol=1e-14)  # tail of 4
    np.testing.assert_allclose(vsum[:, 3], v[:, 96:].sum(axis=1), atol=1e-14)


@pytest.mark.parametrize("Sk,bk", [(256, 32), (250, 32), (97, 16)])
def test_block_constant_kv_makes_the_proxy_exact(Sk, bk):
    """With identical tokens inside every KV block (the ragged tail included),
    the proxy of an omitted block equals its tokens exactly, so the output is
    plain attention over all keys whatever the selection."""
    B, Sq, H, Hkv, D, bq = 2, 70, 4, 2, 16, 32
    q, k, v, full, part = _inputs(1, B, Sq, Sk, H, Hkv, D, bq, bk, 0.3)
    N = -(-Sk // bk)
    rng = np.random.default_rng(2)
    kb = rng.standard_normal((B, N, Hkv, D))
    vb = rng.standard_normal((B, N, Hkv, D))
    owner = np.arange(Sk) // bk
    k, v = kb[:, owner], vb[:, owner]
    full[0, 0, 0] = False  # one row with no exact block at all
    part[0, 0, 0] = False
    kbar, vsum = oracle.block_summaries(k, v, bk)
    O, L = oracle.proxy_attention(q, k, v, full, part, kbar, vsum, bq, bk, 0.3)
    for b in range(B):
        ref_o, ref_l = _sdpa(q[b], np.repeat(k[b], H // Hkv, axis=1),
                             np.repeat(v[b], H // Hkv, axis=1), 0.3)
        np.testing.assert_allclose(O[b], ref_o, atol=1e-12)
        np.testing.assert_allclose(L[b], ref_l, atol=1e-12)


@pytest.mark.parametrize("seed,Sq,Sk,bq,bk,density", [(3, 96, 200, 32, 48, 0.3),
                                                       (4, 64, 64, 64, 16, 0.0),
                                                       (5, 130, 333, 64, 64, 0.5)])
def test_equals_attention_over_tokens_rebuilt_from_summaries(seed, Sq, Sk, bq, bk, density):
    """Omitted blocks' tokens replaced by (mean K, summed V / token count),
    exact blocks left as they are, then plain attention over all keys."""
    B, H, Hkv, D = 1, 2, 1, 8
    q, k, v, full, part = _inputs(seed, B, Sq, Sk, H, Hkv, D, bq, bk, density)
    kbar, vsum = oracle.block_summaries(k, v, bk)
    O, L = oracle.proxy_attention(q, k, v, full, part, kbar, vsum, bq, bk, 0.25)
    N = -(-Sk // bk)
    for h in range(H):
        for i in range(-(-Sq // bq)):
            rows = slice(i * bq, min((i + 1) * bq, Sq))
            kk, vv = k[0, :, 0].copy(), v[0, :, 0].copy()
            for n in range(N):
                if not (full[0, h, i, n] or part[0, h, i, n]):
                    sl = slice(n * bk, min((n + 1) * bk, Sk))
                    cnt = sl.stop - sl.start
                    kk[sl] = k[0, sl, 0].mean(axis=0)
                    vv[sl] = v[0, sl, 0].sum(axis=0) / cnt
            ref_o, ref_l = _sdpa(q[0, rows, h:h + 1], kk[:, None], vv[:, None], 0.25)
            np.testing.assert_allclose(O[0, rows, h], ref_o[:, 0], atol=1e-12)
            np.testing.assert_allclose(L[0, h, rows], ref_l[0], atol=1e-12)


def test_all_selected_is_plain_attention():
    B, Sq, Sk, H, Hkv, D, bq, bk = 1, 50, 90, 2, 2, 8, 32, 32
    q, k, v, full, part = _inputs(6, B, Sq, Sk, H, Hkv, D, bq, bk, 1.0)
    kbar, vsum = oracle.block_summaries(k, v, bk)
    O, L = oracle.proxy_attention(q, k, v, full, part, kbar, vsum, bq, bk, 0.5)
    ref_o, ref_l = _sdpa(q[0], k[0], v[0], 0.5)
    np.testing.assert_allclose(O[0], ref_o, atol=1e-12)
    np.testing.assert_allclose(L[0], ref_l, atol=1e-12)
