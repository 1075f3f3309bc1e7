"""Pins for the backward oracle and the KV-major block lists (CPU only).

Independent anchors: torch autograd (float64) through a dense masked softmax
attention; central finite differences of sum(O * dO) through the pinned
forward oracle; the plain-loop element mask; a hand-made transposition.
"""
import numpy as np
import pytest
import torch

import oracle

NONE, CAUSAL, KVV, LOCAL = (oracle.MASK_NONE, oracle.MASK_CAUSAL, oracle.MASK_KV_VALID_COUNT,
                            oracle.MASK_LOCAL)


def _case(seed, B, Sq, Sk, H, Hkv, D, bq, bk, density, mm):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, H, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    do = rng.standard_normal((B, Sq, H, D))
    M, N = -(-Sq // bq), -(-Sk // bk)
    sel = rng.random((B, H, M, N)) < density
    part = sel & (rng.random(sel.shape) < 0.5) if mm != NONE else np.zeros_like(sel)
    return q, k, v, do, sel & ~part, part


@pytest.mark.parametrize("mm,window", [(NONE, None), (CAUSAL, None), (LOCAL, (20, 5)), (KVV, None)])
def test_element_mask_matches_the_plain_loops(mm, window):
    q, k, v, do, full, part = _case(1, 1, 45, 70, 2, 1, 4, 16, 24, 0.6, mm)
    kvv = np.array([24, 10, 0], np.int32) if mm == KVV else None
    a = oracle.element_mask(full, part, 16, 24, 45, 70, mm, kvv, window)
    b = oracle.expand_element_mask(full, part, 16, 24, 45, 70, mm, kvv, window)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("mm,window", [(NONE, None), (CAUSAL, None), (LOCAL, (30, 0))])
def test_gradients_equal_torch_autograd(mm, window):
    B, Sq, Sk, H, Hkv, D, bq, bk = 2, 80, 96, 4, 2, 8, 32, 32
    q, k, v, do, full, part = _case(2, B, Sq, Sk, H, Hkv, D, bq, bk, 0.7, mm)
    keep = oracle.element_mask(full, part, bq, bk, Sq, Sk, mm, None, window)
    # rows that keep no key get zero gradient; torch's softmax would give NaN there
    empty = ~keep.any(axis=-1)
    dq, dk, dv = oracle.blocksparse_attention_bwd(q, k, v, full, part, bq, bk, mm, 0.3, do,
                                                  window=window)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(H // Hkv, dim=2)
    vv = tv.repeat_interleave(H // Hkv, dim=2)
    s = 0.3 * torch.einsum("bqhd,bkhd->bhqk", tq, kk)
    km = torch.from_numpy(keep)
    s = s.masked_fill(~km, -torch.inf)
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)
    o = torch.einsum("bhqk,bkhd->bqhd", p, vv)
    (o * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    assert (dq.transpose(0, 2, 1, 3)[empty] == 0).all()


def test_gradients_equal_finite_differences():
    B, Sq, Sk, H, Hkv, D, bq, bk = 1, 20, 24, 2, 1, 4, 8, 8
    q, k, v, do, full, part = _case(3, B, Sq, Sk, H, Hkv, D, bq, bk, 0.6, CAUSAL)
    f = lambda q_, k_, v_: float((oracle.blocksparse_attention(
        q_, k_, v_, full, part, bq, bk, CAUSAL, 0.5)[0] * do).sum())
    dq, dk, dv = oracle.blocksparse_attention_bwd(q, k, v, full, part, bq, bk, CAUSAL, 0.5, do)
    rng = np.random.default_rng(4)
    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for _ in range(6):
            idx = tuple(int(rng.integers(s)) for s in arr.shape)
            plus, minus = [x.copy() for x in (q, k, v)], [x.copy() for x in (q, k, v)]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            num = (f(*plus) - f(*minus)) / (2 * eps)
            assert abs(num - grad[idx]) < 1e-7, (which, idx, num, grad[idx])


def test_kv_major_lists_hand_example():
    mask = np.zeros((1, 1, 3, 4), bool)
    mask[0, 0, 0, [0, 2]] = True
    mask[0, 0, 2, [2, 3]] = True
    cnt, idx = oracle.kv_major_lists(mask)
    assert cnt.tolist() == [[[1, 0, 2, 1]]]
    assert idx[0, 0].tolist() == [[0, -1, -1], [-1, -1, -1], [2, 0, -1], [2, -1, -1]]
    rng = np.random.default_rng(5)
    m = rng.random((2, 3, 7, 5)) < 0.4
    c, i = oracle.kv_major_lists(m)
    np.testing.assert_array_equal(oracle.index_to_mask(c, i, 7), np.swapaxes(m, -1, -2))
