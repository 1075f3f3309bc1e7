"""Pins for the packed UInt32 bitmap input of the oracle (CPU only).

Independent anchors: a hand-decoded two-row example with set padding bits;
numpy's packbits (little bit order) as the encoder of random masks; the
Q-head to KV-head group mapping checked head by head.
"""
import numpy as np
import pytest

import oracle


def test_hand_decoded_two_rows_with_padding_bits():
    # N = 40 blocks -> 2 words per row; bits 40..63 of each row are padding.
    words = np.array([[[[0x80000005, 0xFFFFFF80],     # blocks 0, 2, 31; 39; padding 40..63
                        [0x00000000, 0x00000101]]]],  # block 32; bit 8 = block 40 is padding
                     dtype=np.uint32)
    mask = oracle.bitmask_to_mask(words, 40)
    assert mask.shape == (1, 1, 2, 40)
    assert sorted(np.flatnonzero(mask[0, 0, 0])) == [0, 2, 31, 39]
    assert sorted(np.flatnonzero(mask[0, 0, 1])) == [32]
    cnt, idx = oracle.bitmask_to_index(words, 40)
    assert cnt.tolist() == [[[4, 1]]]
    assert idx[0, 0, 0, :5].tolist() == [39, 31, 2, 0, -1]
    assert idx[0, 0, 1, :2].tolist() == [32, -1]
    assert (idx[0, 0, 1, 1:] == -1).all()


@pytest.mark.parametrize("B,Hkv,M,N,seed", [(1, 1, 3, 1, 0), (2, 2, 5, 31, 1), (1, 3, 4, 32, 2),
                                             (2, 1, 2, 33, 3), (1, 2, 3, 100, 4), (1, 1, 1, 0, 5)])
def test_random_masks_round_trip_through_packbits(B, Hkv, M, N, seed):
    rng = np.random.default_rng(seed)
    W = -(-N // 32)
    mask = rng.random((B, Hkv, M, N)) < 0.4
    padded = np.concatenate([mask, rng.random((B, Hkv, M, 32 * W - N)) < 0.7], axis=-1)
    words = np.packbits(padded, axis=-1, bitorder="little").view("<u4").reshape(B, Hkv, M, W)
    np.testing.assert_array_equal(oracle.bitmask_to_mask(words, N), mask)
    # int32 storage of the same bit patterns decodes the same way
    np.testing.assert_array_equal(oracle.bitmask_to_mask(words.view(np.int32), N), mask)
    cnt, idx = oracle.bitmask_to_index(words, N)
    c2, i2 = oracle.mask_to_index(mask)
    np.testing.assert_array_equal(cnt, c2)
    np.testing.assert_array_equal(idx, i2)


def test_q_heads_read_their_kv_group():
    rng = np.random.default_rng(7)
    B, Hkv, H, M, N = 2, 2, 6, 3, 45
    words = rng.integers(0, 2**32, (B, Hkv, M, 2), dtype=np.uint64).astype(np.uint32)
    mask = oracle.bitmask_to_mask(words, N, H)
    assert mask.shape == (B, H, M, N)
    for h in range(H):
        np.testing.assert_array_equal(mask[:, h], oracle.bitmask_to_mask(words, N)[:, h // 3])
    assert not np.array_equal(mask[:, 0], mask[:, 3])  # the two groups differ on this draw


def test_bad_shapes_are_rejected():
    with pytest.raises(ValueError):
        oracle.bitmask_to_mask(np.zeros((1, 1, 1, 2), np.uint32), 30)
    with pytest.raises(ValueError):
        oracle.bitmask_to_mask(np.zeros((1, 2, 1, 1), np.uint32), 30, H=3)
