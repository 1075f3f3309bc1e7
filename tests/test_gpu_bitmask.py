"""GPU: the packed UInt32 block bitmap input and the KV-major block lists.  bsa_bitmask_to_index must match
oracle.bitmask_to_index bit for bit (padding bits set on purpose), and a
forward over bitmap-derived lists must equal, bit for bit, the forward over
the lists of the same selection given as a dense uint8 mask."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_bsa_amd as bsa
import oracle
from bsa_testlib import as_oracle, check_o_lse, to_dev

pytestmark = pytest.mark.gpu


def _words(rng, B, Hkv, M, N, density=0.4, pad_density=0.7):
    """Random selection plus random padding bits, packed LSB-first."""
    W = -(-N // 32)
    sel = rng.random((B, Hkv, M, N)) < density
    pad = rng.random((B, Hkv, M, 32 * W - N)) < pad_density
    bits = np.concatenate([sel, pad], axis=-1)
    return np.packbits(bits, axis=-1, bitorder="little").view("<u4").reshape(B, Hkv, M, W)


def _dev_words(words, as_uint32):
    t = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).cuda()
    return t.view(torch.uint32) if as_uint32 else t


@pytest.mark.parametrize("B,Hkv,H,M,N,u32", [(1, 1, 1, 1, 1, False), (2, 2, 2, 3, 31, True),
                                              (1, 2, 6, 4, 32, False), (2, 1, 4, 5, 33, True),
                                              (1, 3, 3, 7, 100, False), (2, 8, 16, 64, 512, True),
                                              (1, 1, 2, 3, 0, False), (1, 2, 4, 2, 64, False)])
def test_bitmask_to_index_matches_oracle_bit_exact(B, Hkv, H, M, N, u32):
    rng = np.random.default_rng(B * 1000 + H * 100 + N)
    words = _words(rng, B, Hkv, M, N)
    cnt, idx = bsa.bsa_bitmask_to_index(_dev_words(words, u32), N, H)
    torch.cuda.synchronize()
    c_ref, i_ref = oracle.bitmask_to_index(words, N, H)
    np.testing.assert_array_equal(cnt.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(idx.cpu().numpy(), i_ref)


def test_all_bits_set_and_none_set():
    B, Hkv, H, M, N = 1, 1, 2, 3, 70
    for fill, expect in ((0xFFFFFFFF, N), (0, 0)):
        words = np.full((B, Hkv, M, 3), fill, np.uint32)
        cnt, idx = bsa.bsa_bitmask_to_index(_dev_words(words, True), N, H)
        torch.cuda.synchronize()
        assert (cnt == expect).all()
        if expect:
            assert torch.equal(idx[0, 0, 0].cpu(), torch.arange(N - 1, -1, -1, dtype=torch.int32))
        else:
            assert (idx == -1).all()


@pytest.mark.parametrize("D,bq,bk,mm", [(128, 128, 128, bsa.MASK_CAUSAL), (64, 64, 64, bsa.MASK_NONE),
                                        (128, 64, 128, bsa.MASK_CAUSAL)])
def test_forward_over_bitmap_lists_equals_dense_mask_lists(D, bq, bk, mm):
    rng = np.random.default_rng(D + bq + bk)
    B, Hkv, H, S = 2, 2, 4, 700
    M, N = -(-S // bq), -(-S // bk)
    q = rng.standard_normal((B, S, H, D), dtype=np.float32)
    k = rng.standard_normal((B, S, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, S, Hkv, D), dtype=np.float32)
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    sel = _words(rng, B, Hkv, M, N, density=0.5)
    dense = oracle.bitmask_to_mask(sel, N, H)
    # partial blocks on the diagonal (causal) or none; the rest of the selection is full
    if mm == bsa.MASK_CAUSAL:
        f_cls, p_cls = oracle.block_sparsity(mm, S, S, bq, bk)
        full = dense & f_cls.astype(bool)
        part = p_cls.astype(bool)[None, None].repeat(B, 0).repeat(H, 1)
    else:
        full, part = dense, np.zeros_like(dense)
    # bitmaps of the two classes, per KV head (the class masks are equal over a group)
    def pack(m):
        kv = m[:, ::H // Hkv]
        W = -(-N // 32)
        padded = np.concatenate([kv, np.ones(kv.shape[:-1] + (32 * W - N,), bool)], axis=-1)
        return np.packbits(padded, axis=-1, bitorder="little").view("<u4").reshape(
            kv.shape[:-1] + (W,))
    fl_b = bsa.bsa_bitmask_to_index(_dev_words(pack(full), True), N, H)
    ml_b = bsa.bsa_bitmask_to_index(_dev_words(pack(part), False), N, H)
    fl_d = bsa.bsa_mask_to_index(torch.from_numpy(np.ascontiguousarray(full, np.uint8)).cuda())
    ml_d = bsa.bsa_mask_to_index(torch.from_numpy(np.ascontiguousarray(part, np.uint8)).cuda())
    scale = 1 / math.sqrt(D)
    has_part = bool(part.any())
    o1, l1 = bsa.bsa_fwd(qd, kd, vd, ml_b if has_part else None, fl_b, bq, bk, mm, None, scale,
                         validate=True)
    o2, l2 = bsa.bsa_fwd(qd, kd, vd, ml_d if has_part else None, fl_d, bq, bk, mm, None, scale,
                         validate=True)
    torch.cuda.synchronize()
    assert torch.equal(fl_b[0], fl_d[0]) and torch.equal(fl_b[1], fl_d[1])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O, L = oracle.blocksparse_attention(as_oracle(qd), as_oracle(kd), as_oracle(vd), full, part,
                                        bq, bk, mm, scale)
    check_o_lse(o1, l1, O, L, f"bitmap lists d{D} {bq}x{bk}")


def test_bad_bitmaps_are_rejected():
    w = torch.zeros((1, 2, 3, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        bsa.bsa_bitmask_to_index(w, 30)          # 2 words for 30 blocks
    with pytest.raises(ValueError):
        bsa.bsa_bitmask_to_index(w, 40, H=3)     # H not a multiple of Hkv
    with pytest.raises(ValueError):
        bsa.bsa_bitmask_to_index(w.to(torch.int64), 40)


@pytest.mark.parametrize("B,H,M,N,density", [(1, 1, 3, 4, 0.5), (2, 3, 17, 9, 0.3),
                                              (1, 2, 5, 130, 0.2), (2, 2, 64, 64, 0.0),
                                              (1, 4, 40, 33, 1.0), (1, 1, 1, 1, 1.0)])
def test_kv_major_lists_match_oracle_bit_exact(B, H, M, N, density):
    rng = np.random.default_rng(B * 100 + M + N)
    mask = rng.random((B, H, M, N)) < density
    cnt, idx = bsa.bsa_mask_to_index(torch.from_numpy(mask.astype(np.uint8)).cuda())
    cnt_t, idx_t = bsa.bsa_kv_major_lists((cnt, idx))
    torch.cuda.synchronize()
    c_ref, i_ref = oracle.kv_major_lists(mask)
    np.testing.assert_array_equal(cnt_t.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(idx_t.cpu().numpy(), i_ref)
