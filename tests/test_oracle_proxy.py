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


# ------------------------------------------ backward
def _rebuilt_autograd(q, k, v, kbar, vsum, full, part, bq, bk, scale, dout):
    """Gradients by torch autograd (float64) of attention over keys rebuilt
    token by token: per Q block, the exact blocks' tokens plus, for each
    omitted block n, c_n copies of (kbar_n, vsum_n / c_n)."""
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, kbar, vsum)]
    tq, tk, tv, tkb, tvs = t
    B, Sq, H, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    M, N = -(-Sq // bq), -(-Sk // bk)
    mass = [min(bk, Sk - n * bk) for n in range(N)]
    loss = torch.zeros((), dtype=torch.float64)
    g = torch.from_numpy(dout)
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            for i in range(M):
                rows = slice(i * bq, min((i + 1) * bq, Sq))
                keys, vals = [], []
                for n in range(N):
                    toks = slice(n * bk, min((n + 1) * bk, Sk))
                    if full[b, h, i, n] or part[b, h, i, n]:
                        keys.append(tk[b, toks, hk])
                        vals.append(tv[b, toks, hk])
                    else:
                        keys.append(tkb[b, n, hk].expand(mass[n], D))
                        vals.append((tvs[b, n, hk] / mass[n]).expand(mass[n], D))
                K, V = torch.cat(keys), torch.cat(vals)
                P = torch.softmax(scale * tq[b, rows, h] @ K.T, dim=-1)
                loss = loss + (P @ V * g[b, rows, h]).sum()
    loss.backward()
    return [np.zeros(x.shape) if x.grad is None else x.grad.numpy() for x in t]


@pytest.mark.parametrize("seed,Sq,Sk,bq,bk,density", [
    (3, 70, 96, 32, 16, 0.3), (4, 50, 100, 16, 32, 0.5), (5, 33, 65, 32, 8, 0.0)])
def test_backward_equals_autograd_over_rebuilt_tokens(seed, Sq, Sk, bq, bk, density):
    B, H, Hkv, D = 2, 4, 2, 8
    q, k, v, full, part = _inputs(seed, B, Sq, Sk, H, Hkv, D, bq, bk, density)
    rng = np.random.default_rng(seed + 100)
    N = -(-Sk // bk)
    kbar = rng.standard_normal((B, N, Hkv, D))
    vsum = rng.standard_normal((B, N, Hkv, D)) * 3
    dout = rng.standard_normal(q.shape)
    scale = 0.4
    got = oracle.proxy_attention_bwd(q, k, v, full, part, kbar, vsum, bq, bk, scale, dout)
    ref = _rebuilt_autograd(q, k, v, kbar, vsum, full, part, bq, bk, scale, dout)
    for name, a, r in zip(("dq", "dk", "dv", "dkbar", "dvsum"), got, ref):
        np.testing.assert_allclose(a, r, atol=1e-10, rtol=0, err_msg=name)


def test_backward_all_selected_is_the_plain_backward():
    B, Sq, Sk, H, Hkv, D, bq, bk = 1, 40, 48, 2, 1, 8, 16, 16
    q, k, v, _, _ = _inputs(6, B, Sq, Sk, H, Hkv, D, bq, bk, 0.0)
    M, N = -(-Sq // bq), -(-Sk // bk)
    full = np.ones((B, H, M, N), bool)
    part = np.zeros_like(full)
    kbar, vsum = oracle.block_summaries(k, v, bk)
    dout = np.random.default_rng(7).standard_normal(q.shape)
    dq, dk, dv, dkb, dvs = oracle.proxy_attention_bwd(q, k, v, full, part, kbar, vsum, bq, bk,
                                                      0.3, dout)
    rq, rk, rv = oracle.blocksparse_attention_bwd(q, k, v, full, part, bq, bk, oracle.MASK_NONE,
                                                  0.3, dout)
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, r, atol=1e-12, rtol=0)
    assert not dkb.any() and not dvs.any()


def test_backward_block_constant_tokens_match_dense_attention():
    """With identical tokens inside every KV block the proxy forward is plain
    attention over all keys; then dq is the dense dq, and for every block the
    dense gradient summed over its tokens equals the exact tokens' gradient
    plus that of its summary (dk: kbar is the block's key; dv: vsum is c_n
    times the block's value)."""
    B, Sq, Sk, H, Hkv, D, bq, bk = 1, 60, 90, 2, 1, 8, 20, 16
    q, _, _, full, part = _inputs(8, B, Sq, Sk, H, Hkv, D, bq, bk, 0.4)
    rng = np.random.default_rng(9)
    N = -(-Sk // bk)
    kb, vb = rng.standard_normal((B, N, Hkv, D)), rng.standard_normal((B, N, Hkv, D))
    owner = np.arange(Sk) // bk
    k, v = kb[:, owner], vb[:, owner]
    kbar, vsum = oracle.block_summaries(k, v, bk)
    dout = rng.standard_normal(q.shape)
    scale = 0.35
    dq, dk, dv, dkb, dvs = oracle.proxy_attention_bwd(q, k, v, full, part, kbar, vsum, bq, bk,
                                                      scale, dout)
    allf = np.ones_like(full)
    rq, rk, rv = oracle.blocksparse_attention_bwd(q, k, v, allf, np.zeros_like(allf), bq, bk,
                                                  oracle.MASK_NONE, scale, dout)
    np.testing.assert_allclose(dq, rq, atol=1e-11, rtol=0)
    mass = np.array([min(bk, Sk - n * bk) for n in range(N)], np.float64)
    for n in range(N):
        toks = slice(n * bk, min((n + 1) * bk, Sk))
        np.testing.assert_allclose(rk[:, toks].sum(1), dk[:, toks].sum(1) + dkb[:, n], atol=1e-11)
        np.testing.assert_allclose(rv[:, toks].sum(1), dv[:, toks].sum(1) + mass[n] * dvs[:, n],
                                   atol=1e-11)
