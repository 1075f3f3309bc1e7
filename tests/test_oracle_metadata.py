"""Pins for the metadata oracle (CPU only).

mask -> index:  the page's worked example, the traversal example, and a
brute force over every row of N <= 10 bits written with integer bit tricks.
varlen offsets: a hand-computed example of the page's formulas and a brute
enumeration of packed (b, m, n) slots.  KV-block expansion: token-level
equivalence by enumeration.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_mask_to_index_page_example():
    g = _golden("mask_to_index_example.json")
    cnt, idx = oracle.mask_to_index(np.array([g["mask_row"]], np.uint8))
    assert cnt.tolist() == [g["cnt"]]
    assert idx.tolist() == [g["idx_row"]]


def test_mask_to_index_traversal_example():
    g = _golden("traversal_example.json")
    row = np.zeros(g["n_blocks"], bool)
    row[g["selected"]] = True
    cnt, idx = oracle.mask_to_index(row[None])
    visit = idx[0, :cnt[0]].tolist()
    assert visit == g["visit_order"]
    assert [a - b for a, b in zip(visit[:-1], visit[1:])] == g["leaps"]


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 10])
def test_mask_to_index_bruteforce_all_rows(N):
    rows = np.array([[(x >> j) & 1 for j in range(N)] for x in range(1 << N)], np.uint8)
    cnt, idx = oracle.mask_to_index(rows)
    for x in range(1 << N):
        bits = [j for j in range(N) if (x >> j) & 1]
        assert cnt[x] == bin(x).count("1")
        expect = sorted(bits, reverse=True) + [-1] * (N - len(bits))
        assert idx[x].tolist() == expect


def test_mask_to_index_nonzero_counts_as_selected_and_shape():
    rng = np.random.default_rng(0)
    m = rng.integers(0, 4, size=(2, 3, 4, 7)).astype(np.uint8)
    cnt, idx = oracle.mask_to_index(m)
    assert cnt.shape == (2, 3, 4) and idx.shape == (2, 3, 4, 7)
    assert cnt.dtype == np.int32 and idx.dtype == np.int32
    np.testing.assert_array_equal(cnt, (m != 0).sum(-1))
    np.testing.assert_array_equal(oracle.index_to_mask(cnt, idx, 7), m != 0)


def test_index_to_mask_rejects_bad_lists():
    with pytest.raises(ValueError):
        oracle.index_to_mask(np.array([2]), np.array([[1, 1, -1]]), 3)
    with pytest.raises(ValueError):
        oracle.index_to_mask(np.array([1]), np.array([[3, -1, -1]]), 3)


def test_varlen_offsets_page_formula_example():
    g = _golden("varlen_layout_example.json")
    cu, off, tm, tn = oracle.varlen_offsets(g["seqlens_q"], g["seqlens_k"],
                                            g["block_q"], g["block_kv"])
    assert cu == g["cu_total_m_blocks"]
    assert off == g["block_idx_offsets"]
    assert (tm, tn) == (g["total_m_blocks"], g["total_n_blocks"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_varlen_offsets_brute_enumeration(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    sq = [int(x) for x in rng.integers(0, 700, B)]
    sk = [int(x) for x in rng.integers(0, 700, B)]
    bq, bk = int(rng.choice([32, 64, 128, 256])), int(rng.choice([16, 64, 112, 128]))
    cu, off, tm, tn = oracle.varlen_offsets(sq, sk, bq, bk)
    # enumerate every Q block and every (Q block, KV block) slot in packing order
    m_pos, slot = 0, 0
    for b in range(B):
        assert cu[b] == m_pos and off[b] == slot
        q_blocks = 0
        r = 0
        while r < sq[b]:
            q_blocks += 1
            r += bq
        kv_blocks = 0
        c = 0
        while c < sk[b]:
            kv_blocks += 1
            c += bk
        for _ in range(q_blocks):
            m_pos += 1
            for _ in range(kv_blocks):
                slot += 1
    assert (cu[B], off[B], tm, tn) == (m_pos, slot, m_pos, slot)


def test_pack_varlen_lists_roundtrip():
    rng = np.random.default_rng(3)
    sq, sk, H, bq, bk = [5, 300, 129], [70, 300, 1], 2, 64, 32
    masks = [rng.random((H, -(-a // bq), -(-b // bk))) < 0.4 for a, b in zip(sq, sk)]
    cnt, idx = oracle.pack_varlen_lists(masks, sq, sk, bq, bk)
    cu, off, tm, tn = oracle.varlen_offsets(sq, sk, bq, bk)
    assert cnt.shape == (H, tm) and idx.shape == (H, tn)
    for b, m in enumerate(masks):
        nm, nn = m.shape[1:]
        for h in range(H):
            for i in range(nm):
                row = idx[h, off[b] + i * nn: off[b] + (i + 1) * nn]
                c = cnt[h, cu[b] + i]
                assert c == m[h, i].sum()
                assert row[:c].tolist() == sorted(np.flatnonzero(m[h, i]).tolist(), reverse=True)
                assert (row[c:] == -1).all()


@pytest.mark.parametrize("factor,child", [(2, 128), (2, 16), (4, 8)])
def test_expand_kv_blocks_token_equivalence(factor, child):
    rng = np.random.default_rng(factor * 100 + child)
    NL = 9
    valid = rng.integers(0, factor * child + 1, NL)
    valid[0], valid[1] = factor * child, 0
    mask = rng.random((2, 3, NL)) < 0.6
    full, part, kv = oracle.expand_kv_blocks(mask, valid, factor, child)
    assert kv.shape == (NL * factor,)
    for j in range(NL):
        assert kv[j * factor:(j + 1) * factor].sum() == valid[j]
        # token p of logical block j is real iff p < valid[j]; after expansion it
        # sits in child p // child at offset p % child
        for p in range(factor * child):
            jc, o = j * factor + p // child, p % child
            assert (p < valid[j]) == (o < kv[jc])
    for jc in range(NL * factor):
        sel = mask[..., jc // factor]
        assert not (full[..., jc] & part[..., jc]).any()
        np.testing.assert_array_equal(full[..., jc] | part[..., jc], sel & (kv[jc] > 0))
        np.testing.assert_array_equal(full[..., jc], sel & (kv[jc] == child))


def test_expand_video_cube_counts():
    # 30x48x52 latent grid in 4x8x8 cubes: 336 cubes -> 672 tiles of 128
    import workloads
    valid, ce = workloads._cube_layout((30, 48, 52), (4, 8, 8))
    assert ce == 256 and len(valid) == 336 and int(valid.sum()) == 30 * 48 * 52
    _, _, kv = oracle.expand_kv_blocks(np.ones((1, 336), bool), valid, 2, 128)
    assert kv.shape == (672,)
    assert sorted(set(kv.tolist())) == [0, 64, 128]
    assert int(kv.sum()) == 74880


def test_mask_to_index_zero_width_rows():
    cnt, idx = oracle.mask_to_index(np.zeros((2, 3, 0), np.uint8))
    assert cnt.shape == (2, 3) and (cnt == 0).all() and idx.shape == (2, 3, 0)
