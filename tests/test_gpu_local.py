"""GPU: the local (sliding-window) mask_mod and the block classifier
bsa_block_sparsity, against the fp64 oracle on seeded inputs.

The classifier must match oracle.block_sparsity bit for bit; forwards over
the lists it produces must match oracle.blocksparse_attention (which the CPU
pins tie to torch SDPA with the band mask) to the usual tolerances.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_bsa_amd as bsa
import oracle
from bsa_testlib import as_oracle, check_o_lse, to_dev

pytestmark = pytest.mark.gpu

NONE, CAUSAL, KVV, LOCAL = bsa.MASK_NONE, bsa.MASK_CAUSAL, bsa.MASK_KV_VALID_COUNT, bsa.MASK_LOCAL


@pytest.mark.parametrize("mm,Sq,Sk,bq,bk,window", [
    (NONE, 300, 200, 64, 48, None),
    (CAUSAL, 1000, 1000, 128, 128, None),
    (CAUSAL, 333, 517, 64, 112, None),
    (LOCAL, 1000, 1000, 128, 128, (256, 0)),
    (LOCAL, 777, 901, 64, 96, (100, 37)),
    (LOCAL, 130, 4097, 32, 64, (-1, 300)),
    (LOCAL, 4097, 130, 256, 64, (17, -1)),
    (LOCAL, 500, 500, 128, 80, (0, 0)),
    (LOCAL, 500, 500, 128, 80, (-1, -1)),
    (KVV, 100, 330, 50, 64, None),
    (LOCAL, 1, 1, 64, 64, (0, 0)),
])
def test_block_sparsity_matches_oracle_bit_exact(mm, Sq, Sk, bq, bk, window):
    kvv = None
    if mm == KVV:
        rng = np.random.default_rng(Sq + Sk)
        kvv = rng.integers(0, bk + 1, -(-Sk // bk)).astype(np.int32)
    full, part = bsa.bsa_block_sparsity(
        mm, Sq, Sk, bq, bk, window=window,
        kv_valid=None if kvv is None else torch.from_numpy(kvv).cuda())
    torch.cuda.synchronize()
    f_ref, p_ref = oracle.block_sparsity(mm, Sq, Sk, bq, bk, window=window, kv_valid=kvv)
    np.testing.assert_array_equal(full.cpu().numpy(), f_ref)
    np.testing.assert_array_equal(part.cpu().numpy(), p_ref)


def _lists(full, part, B, H):
    """[M,N] class masks -> device lists broadcast over B and H."""
    M, N = full.shape
    fl = bsa.bsa_mask_to_index(full.reshape(1, 1, M, N).contiguous())
    ml = bsa.bsa_mask_to_index(part.reshape(1, 1, M, N).contiguous())
    return (ml if bool(part.any()) else None), (fl if bool(full.any()) else None)


def _run_local(seed, B, Sq, Sk, H, Hkv, D, bq, bk, window, dtype=torch.bfloat16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, H, D), dtype=np.float32)
    k = rng.standard_normal((B, Sk, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, Sk, Hkv, D), dtype=np.float32)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    full, part = bsa.bsa_block_sparsity(LOCAL, Sq, Sk, bq, bk, window=window)
    ml, fl = _lists(full, part, B, H)
    scale = 1 / math.sqrt(D)
    o, lse = bsa.bsa_fwd(qd, kd, vd, ml, fl, bq, bk, LOCAL, None, scale, window=window,
                         validate=True)
    torch.cuda.synchronize()
    M, N = full.shape
    fb = np.broadcast_to(full.cpu().numpy().astype(bool), (B, H, M, N))
    pb = np.broadcast_to(part.cpu().numpy().astype(bool), (B, H, M, N))
    # fp32 inputs are rounded to bf16 at load: the oracle takes those values
    r = lambda t: as_oracle(t.to(torch.bfloat16))
    O, L = oracle.blocksparse_attention(r(qd), r(kd), r(vd), fb, pb, bq, bk, LOCAL, scale,
                                        window=window)
    return o, lse, O, L


@pytest.mark.parametrize("case", [
    dict(Sq=600, Sk=600, D=128, bq=128, bk=128, window=(200, 0)),
    dict(Sq=600, Sk=600, D=64, bq=64, bk=64, window=(100, 100)),
    dict(Sq=333, Sk=517, D=128, bq=64, bk=112, window=(-1, 50)),
    dict(Sq=700, Sk=700, D=128, bq=256, bk=128, window=(300, 0)),  # 256-row blocks, 128-row tiles
    dict(Sq=500, Sk=450, D=96, bq=128, bk=80, window=(64, 64)),
    dict(Sq=400, Sk=400, D=192, bq=128, bk=64, window=(129, 0)),
    dict(Sq=300, Sk=300, D=256, bq=64, bk=64, window=(31, 31)),
    dict(Sq=256, Sk=256, D=128, bq=32, bk=64, window=(0, 0)),
])
def test_local_forward_over_classified_lists(case):
    seed = zlib.crc32(repr(sorted(case.items())).encode())
    o, lse, O, L = _run_local(seed, B=2, H=4, Hkv=2, **case)
    check_o_lse(o, lse, O, L, f"local {case}")


def test_local_fp32_inputs():
    o, lse, O, L = _run_local(5, B=1, Sq=300, Sk=300, H=2, Hkv=2, D=64, bq=64, bk=64,
                              window=(70, 10), dtype=torch.float32)
    check_o_lse(o, lse, O, L, "local fp32")


def test_local_rows_without_keys():
    # window (0, 0): only the diagonal; rows >= Sk see nothing -> O = 0, LSE = -inf
    o, lse, O, L = _run_local(6, B=1, Sq=300, Sk=200, H=2, Hkv=1, D=64, bq=64, bk=64,
                              window=(0, 0))
    check_o_lse(o, lse, O, L, "local diagonal only")
    assert torch.isneginf(lse[:, :, 200:]).all() and (o[:, 200:] == 0).all()


def test_local_minus1_0_is_causal_bit_for_bit():
    rng = np.random.default_rng(8)
    B, S, H, D, bq, bk = 1, 512, 2, 128, 128, 128
    q, k, v = (to_dev(rng.standard_normal((B, S, H, D), dtype=np.float32)) for _ in range(3))
    full, part = bsa.bsa_block_sparsity(CAUSAL, S, S, bq, bk)
    ml, fl = _lists(full, part, B, H)
    a = bsa.bsa_fwd(q, k, v, ml, fl, bq, bk, CAUSAL, None, 0.1)
    b = bsa.bsa_fwd(q, k, v, ml, fl, bq, bk, LOCAL, None, 0.1, window=(-1, 0))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_local_varlen_sequence_local_ids():
    rng = np.random.default_rng(9)
    seqlens = [130, 1, 400, 64, 257]
    H, Hkv, D, bq, bk, window = 2, 1, 64, 64, 64, (90, 20)
    T = sum(seqlens)
    q = rng.standard_normal((T, H, D), dtype=np.float32)
    k = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    fulls, parts = [], []
    for s in seqlens:
        f, p = oracle.block_sparsity(LOCAL, s, s, bq, bk, window=window)
        fulls.append(np.broadcast_to(f.astype(bool), (H,) + f.shape).copy())
        parts.append(np.broadcast_to(p.astype(bool), (H,) + p.shape).copy())
    cu, off, tm, tn = bsa.bsa_varlen_offsets(seqlens, seqlens, bq, bk)
    dev = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    cu_q = dev([0] + list(np.cumsum(seqlens)))
    ml = tuple(torch.from_numpy(a).cuda() for a in
               oracle.pack_varlen_lists(parts, seqlens, seqlens, bq, bk))
    fl = tuple(torch.from_numpy(a).cuda() for a in
               oracle.pack_varlen_lists(fulls, seqlens, seqlens, bq, bk))
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    o, lse = bsa.bsa_varlen_fwd(qd, kd, vd, cu_q, cu_q, dev(cu), dev(off), tm, tn, ml, fl, bq, bk,
                                LOCAL, 0.125, window=window, validate=True)
    torch.cuda.synchronize()
    O, L = oracle.varlen_blocksparse_attention(as_oracle(qd), as_oracle(kd), as_oracle(vd),
                                               seqlens, seqlens, fulls, parts, bq, bk, LOCAL,
                                               0.125, window=window)
    check_o_lse(o, lse, O, L, "local varlen")


def test_local_needs_a_window():
    q = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        bsa.bsa_fwd(q, q, q, None, None, 64, 64, LOCAL, None, 1.0)
    with pytest.raises(ValueError):
        bsa.bsa_block_sparsity(LOCAL, 64, 64, 64, 64)
