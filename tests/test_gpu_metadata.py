"""GPU metadata kernels vs the metadata oracle: bit-exact."""
import numpy as np
import pytest
import torch

import block_sparse_attention_bsa_amd as bsa
import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(1, 1, 1, 6), (2, 3, 5, 1), (2, 4, 8, 63), (1, 2, 7, 64),
                                   (1, 2, 9, 65), (2, 16, 32, 37), (1, 3, 4, 672), (1, 1, 3, 0)])
@pytest.mark.parametrize("p", [0.0, 0.3, 1.0])
def test_mask_to_index_bit_exact(shape, p):
    rng = np.random.default_rng(hash((shape, p)) % 2 ** 32)
    m = (rng.random(shape) < p).astype(np.uint8) * rng.integers(1, 255, shape).astype(np.uint8)
    cnt, idx = bsa.bsa_mask_to_index(torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    c_ref, i_ref = oracle.mask_to_index(m)
    np.testing.assert_array_equal(cnt.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(idx.cpu().numpy(), i_ref)


def test_mask_to_index_page_example():
    m = torch.tensor([[[[1, 0, 0, 1, 0, 1]]]], dtype=torch.uint8, device="cuda")
    cnt, idx = bsa.bsa_mask_to_index(m)
    assert cnt.cpu().tolist() == [[[3]]]
    assert idx.cpu().tolist() == [[[[5, 3, 0, -1, -1, -1]]]]


@pytest.mark.parametrize("seed", [0, 1])
def test_varlen_mask_to_index_bit_exact(seed):
    rng = np.random.default_rng(seed)
    sq = [int(x) for x in rng.integers(1, 900, 5)] + [0]
    sk = [int(x) for x in rng.integers(1, 900, 5)] + [7]
    H, bq, bk = 3, 64, 48
    masks = [rng.random((H, -(-a // bq), -(-b // bk))) < 0.35 for a, b in zip(sq, sk)]
    cu, off, tm, tn = bsa.bsa_varlen_offsets(sq, sk, bq, bk)
    assert (cu, off, tm, tn) == tuple(oracle.varlen_offsets(sq, sk, bq, bk))
    # the packed uint8 mask laid out like idx
    packed = np.zeros((H, tn), np.uint8)
    for b, m in enumerate(masks):
        nm, nn = m.shape[1:]
        for i in range(nm):
            packed[:, off[b] + i * nn: off[b] + (i + 1) * nn] = m[:, i]
    cnt, idx = bsa.bsa_varlen_mask_to_index(
        torch.from_numpy(packed).cuda(), torch.tensor(cu, dtype=torch.int32, device="cuda"),
        torch.tensor(off, dtype=torch.int32, device="cuda"), tm, tn)
    c_ref, i_ref = oracle.pack_varlen_lists(masks, sq, sk, bq, bk)
    np.testing.assert_array_equal(cnt.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(idx.cpu().numpy(), i_ref)


@pytest.mark.parametrize("factor,child", [(2, 128), (2, 16), (3, 40)])
def test_expand_kv_blocks_bit_exact(factor, child):
    rng = np.random.default_rng(factor + child)
    NL = 37
    valid = rng.integers(0, factor * child + 1, NL).astype(np.int32)
    valid[:3] = [factor * child, 0, child]
    bm = (rng.random((2, 5, NL)) < 0.5)
    full, part, kvv = bsa.bsa_expand_kv_blocks(torch.from_numpy(bm.astype(np.uint8)).cuda(),
                                               torch.from_numpy(valid).cuda(), factor, child)
    f_ref, p_ref, k_ref = oracle.expand_kv_blocks(bm, valid, factor, child)
    np.testing.assert_array_equal(full.cpu().numpy().astype(bool), f_ref)
    np.testing.assert_array_equal(part.cpu().numpy().astype(bool), p_ref)
    np.testing.assert_array_equal(kvv.cpu().numpy(), k_ref)


def test_mask_to_index_deterministic():
    rng = np.random.default_rng(9)
    m = torch.from_numpy((rng.random((2, 8, 64, 672)) < 0.12).astype(np.uint8)).cuda()
    a = bsa.bsa_mask_to_index(m)
    b = bsa.bsa_mask_to_index(m)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
