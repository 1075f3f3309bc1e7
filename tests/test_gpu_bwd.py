"""GPU: the backward (bsa_bwd) against oracle.blocksparse_attention_bwd on
the same bf16 inputs.  The forward's O and LSE come from bsa_fwd.

Tolerance: P and dS enter their MFMA products rounded to bf16 (relative
error up to 2^-9 each), O enters rowsum(dO * O) as stored (bf16), and the
gradients are stored in bf16.  Each gradient must be within 2 % of its
largest magnitude of the float64 gradient, element by element."""
import math
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_bsa_amd as bsa
import oracle
from bsa_testlib import as_oracle, to_dev

pytestmark = pytest.mark.gpu

NONE, CAUSAL, KVV, LOCAL = bsa.MASK_NONE, bsa.MASK_CAUSAL, bsa.MASK_KV_VALID_COUNT, bsa.MASK_LOCAL
REL_TOL = 2e-2


def _lists(m):
    return bsa.bsa_mask_to_index(torch.from_numpy(np.ascontiguousarray(m, np.uint8)).cuda())


@pytest.mark.parametrize("case", [
    dict(mm=NONE, Sq=256, Sk=256, D=64, bq=64, bk=64),
    dict(mm=CAUSAL, Sq=384, Sk=384, D=128, bq=128, bk=128),
    dict(mm=CAUSAL, Sq=300, Sk=300, D=64, bq=64, bk=64),
    dict(mm=LOCAL, Sq=333, Sk=333, D=128, bq=64, bk=128, window=(100, 20)),
    dict(mm=KVV, Sq=200, Sk=450, D=64, bq=128, bk=48),
    dict(mm=NONE, Sq=130, Sk=517, D=128, bq=64, bk=112),
    dict(mm=CAUSAL, Sq=300, Sk=300, D=96, bq=128, bk=64),
    dict(mm=LOCAL, Sq=260, Sk=260, D=192, bq=64, bk=128, window=(70, 0)),
    dict(mm=CAUSAL, Sq=256, Sk=256, D=256, bq=128, bk=128),
    dict(mm=KVV, Sq=150, Sk=200, D=256, bq=64, bk=64),
])
def test_bwd_matches_oracle(case):
    seed = zlib.crc32(repr(sorted(case.items())).encode())
    rng = np.random.default_rng(seed)
    mm, Sq, Sk, D, bq, bk = case["mm"], case["Sq"], case["Sk"], case["D"], case["bq"], case["bk"]
    window = case.get("window")
    B, H, Hkv = 2, 4, 2
    M, N = -(-Sq // bq), -(-Sk // bk)
    q, k, v = (to_dev(rng.standard_normal(s, dtype=np.float32))
               for s in ((B, Sq, H, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D)))
    do = to_dev(rng.standard_normal((B, Sq, H, D), dtype=np.float32))
    kvv = None
    if mm in (CAUSAL, LOCAL):
        f_c, p_c = oracle.block_sparsity(mm, Sq, Sk, bq, bk, window=window)
        keep_blk = rng.random((B, H, M, N)) < 0.7
        full = f_c.astype(bool)[None, None] & keep_blk
        part = np.broadcast_to(p_c.astype(bool), (B, H, M, N)).copy()
    else:
        sel = rng.random((B, H, M, N)) < 0.4
        split = rng.random((B, H, M, N)) < 0.5
        full, part = sel & split, sel & ~split
        if mm == NONE:
            full, part = sel, np.zeros_like(sel)
        else:
            kvv = rng.integers(0, bk + 1, N).astype(np.int32)
    full[0, 0, 0] = False  # a Q block with nothing listed
    part[0, 0, 0] = False
    ml = _lists(part) if part.any() else None
    fl = _lists(full) if full.any() else None
    kvv_d = None if kvv is None else torch.from_numpy(kvv).cuda()
    scale = 1 / math.sqrt(D)
    o, lse = bsa.bsa_fwd(q, k, v, ml, fl, bq, bk, mm, kvv_d, scale, window=window)
    dq, dk, dv = bsa.bsa_bwd(q, k, v, o, lse, do, ml, fl, bq, bk, mm, kvv_d, scale, window=window)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.blocksparse_attention_bwd(as_oracle(q), as_oracle(k), as_oracle(v), full,
                                                  part, bq, bk, mm, scale, as_oracle(do),
                                                  kv_valid=kvv, window=window)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gg = as_oracle(g)
        assert np.isfinite(gg).all(), f"{name}: NaN/inf"
        err = float(np.abs(gg - r).max())
        ref = float(np.abs(r).max())
        assert err <= REL_TOL * max(ref, 1e-6), f"{name} {case}: err {err:.3e} vs max {ref:.3e}"
    assert (dq[0, :bq, 0] == 0).all()  # the Q block with nothing listed


def test_bwd_rejects_unsupported():
    q = torch.zeros((1, 64, 1, 80), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    fl = _lists(np.ones((1, 1, 1, 1), bool))
    with pytest.raises(bsa.BsaError):
        bsa.bsa_bwd(q, q, q, q, lse, q, None, fl, 64, 64)


def test_bwd_full_size_sweep_sampled_heads():
    # The d128 sweep workload at full size (B2 H16 S4096, 128x128 blocks, 25 %
    # with causal diagonals), the backward the bench times; heads are
    # independent here (H = Hkv), so the oracle runs on two sampled (b, h)
    # slices over the whole sequence and their dQ, dK, dV are compared in full.
    import workloads
    w = workloads.sparse_sweep(128, 128, 128)
    q, k, v = (to_dev(x) for x in (w.q, w.k, w.v))
    do = to_dev(np.random.default_rng(77).standard_normal(w.q.shape, dtype=np.float32))
    ml, fl = _lists(w.part), _lists(w.full)
    o, lse = bsa.bsa_fwd(q, k, v, ml, fl, 128, 128, CAUSAL, None, w.scale)
    dq, dk, dv = bsa.bsa_bwd(q, k, v, o, lse, do, ml, fl, 128, 128, CAUSAL, None, w.scale)
    torch.cuda.synchronize()
    for (b, h) in ((0, 3), (1, 11)):
        sl = lambda t: as_oracle(t[b:b + 1, :, h:h + 1])
        rq, rk, rv = oracle.blocksparse_attention_bwd(
            sl(q), sl(k), sl(v), w.full[b:b + 1, h:h + 1], w.part[b:b + 1, h:h + 1], 128, 128,
            CAUSAL, w.scale, sl(do))
        for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            gg = sl(g)
            err = float(np.abs(gg - r).max())
            ref = float(np.abs(r).max())
            print(f"full-size sweep bwd (b={b}, h={h}) {name}: max err {err:.3e}, "
                  f"max |grad| {ref:.3e}, ratio {err / ref:.2e}")
            assert err <= REL_TOL * ref, f"{name} (b={b}, h={h}): err {err:.3e} vs max {ref:.3e}"
