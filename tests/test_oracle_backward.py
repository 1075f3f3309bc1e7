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


def _varlen_case(seed, seqlens_q, seqlens_k, H, Hkv, D, bq, bk, density, mm):
    rng = np.random.default_rng(seed)
    Tq, Tk = sum(seqlens_q), sum(seqlens_k)
    q = rng.standard_normal((Tq, H, D))
    k = rng.standard_normal((Tk, Hkv, D))
    v = rng.standard_normal((Tk, Hkv, D))
    do = rng.standard_normal((Tq, H, D))
    full, part = [], []
    for sq, sk in zip(seqlens_q, seqlens_k):
        sel = rng.random((H, -(-sq // bq), -(-sk // bk))) < density
        pt = sel & (rng.random(sel.shape) < 0.5) if mm != NONE else np.zeros_like(sel)
        full.append(sel & ~pt)
        part.append(pt)
    return q, k, v, do, full, part


@pytest.mark.parametrize("mm", [CAUSAL, KVV, NONE])
def test_varlen_gradients_equal_torch_autograd_on_the_packed_batch(mm):
    # One masked attention over the whole packed batch, with a block-diagonal
    # element mask (no key of another sequence is visible), differentiated by
    # torch: the per-sequence slicing and offsets of the varlen backward must
    # reproduce it.  Includes a sequence with no tokens and one with no keys.
    sq, sk = [40, 0, 33, 17, 9], [52, 7, 29, 0, 30]
    H, Hkv, D, bq, bk = 4, 2, 8, 16, 12
    q, k, v, do, full, part = _varlen_case(6, sq, sk, H, Hkv, D, bq, bk, 0.7, mm)
    rng = np.random.default_rng(7)
    kvv = [rng.integers(0, bk + 3, size=-(-n // bk)).astype(np.int32) for n in sk] \
        if mm == KVV else None
    dq, dk, dv = oracle.varlen_blocksparse_attention_bwd(q, k, v, sq, sk, full, part, bq, bk, mm,
                                                         0.4, do, kv_valid=kvv)
    cq, ck = np.cumsum([0] + sq), np.cumsum([0] + sk)
    keep = np.zeros((H, sum(sq), sum(sk)), bool)
    for b in range(len(sq)):
        e = oracle.element_mask(full[b][None], part[b][None], bq, bk, sq[b], sk[b], mm,
                                None if kvv is None else kvv[b])
        keep[:, cq[b]:cq[b + 1], ck[b]:ck[b + 1]] = e[0]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(H // Hkv, dim=1)
    vv = tv.repeat_interleave(H // Hkv, dim=1)
    s = 0.4 * torch.einsum("qhd,khd->hqk", tq, kk)
    s = s.masked_fill(~torch.from_numpy(keep), -torch.inf)
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)
    o = torch.einsum("hqk,khd->qhd", p, vv)
    (o * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    assert np.abs(dk).sum() > 0 and np.abs(dq).sum() > 0


def test_varlen_kv_major_lists_hand_example():
    # sequence 0: 4 Q tokens (2 blocks of 2), 6 keys (3 blocks); Q block 0
    # lists KV blocks {0, 2}, Q block 1 lists {1, 2}.  Sequence 1: one Q block
    # listing its one KV block.  Per KV block, the Q blocks listing it:
    # (0,0): [0]; (0,1): [1]; (0,2): [1, 0]; (1,0): [0].  Rows of width M_b at
    # offsets [0, 6]: j*2 inside sequence 0, then 6.
    m0 = np.zeros((1, 2, 3), bool)
    m0[0, 0, [0, 2]] = True
    m0[0, 1, [1, 2]] = True
    m1 = np.ones((1, 1, 1), bool)
    cnt, idx = oracle.varlen_kv_major_lists([m0, m1], [4, 2], [6, 2], 2, 2)
    assert cnt.tolist() == [[1, 1, 2, 1]]
    assert idx.tolist() == [[0, -1, 1, -1, 1, 0, 0]]


def test_varlen_kv_major_lists_list_exactly_the_transposed_blocks():
    rng = np.random.default_rng(8)
    sq, sk, bq, bk, H = [300, 0, 129, 64], [250, 100, 1, 0], 64, 48, 3
    masks = [rng.random((H, -(-a // bq), -(-c // bk))) < 0.4 for a, c in zip(sq, sk)]
    cnt, idx = oracle.varlen_kv_major_lists(masks, sq, sk, bq, bk)
    _, off, _, _ = oracle.varlen_offsets(sq, sk, bq, bk)
    g = 0
    for b, m in enumerate(masks):
        M_b, N_b = m.shape[1], m.shape[2]
        for j in range(N_b):
            for h in range(H):
                want = sorted(np.nonzero(m[h, :, j])[0].tolist(), reverse=True)
                row = idx[h, off[b] + j * M_b: off[b] + (j + 1) * M_b].tolist()
                assert cnt[h, g + j] == len(want)
                assert row == want + [-1] * (M_b - len(want))
        g += N_b
    assert g == cnt.shape[1] and off[-1] == idx.shape[1]
