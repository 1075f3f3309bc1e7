"""GPU: the backward (bsa_bwd) against oracle.blocksparse_attention_bwd on
the same bf16 inputs.  The forward's O and LSE come from bsa_fwd.

Tolerance: P and dS enter their MFMA products rounded to bf16 (relative
error up to 2^-9 each), O enters rowsum(dO * O) as stored (bf16), and the
gradients are stored in bf16.  Each gradient must be within 1 % of its
largest magnitude of the float64 gradient, element by element (the cases
here, full-size ones included, reach at most 0.46 %)."""
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
REL_TOL = 1e-2


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
        print(f"bwd {case} {name}: max err {err:.3e}, max |grad| {ref:.3e}, "
              f"ratio {err / max(ref, 1e-6):.2e}")
        assert err <= REL_TOL * max(ref, 1e-6), f"{name} {case}: err {err:.3e} vs max {ref:.3e}"
    assert (dq[0, :bq, 0] == 0).all()  # the Q block with nothing listed


def test_bwd_rejects_unsupported():
    q = torch.zeros((1, 64, 1, 80), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    fl = _lists(np.ones((1, 1, 1, 1), bool))
    with pytest.raises(bsa.BsaError):
        bsa.bsa_bwd(q, q, q, q, lse, q, None, fl, 64, 64)
    # valid counts shorter than the KV-block count, strided, or missing
    q = torch.zeros((1, 128, 1, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 128), dtype=torch.float32, device="cuda")
    ml = _lists(np.ones((1, 1, 2, 2), bool))
    for kvv in (torch.zeros(1, dtype=torch.int32, device="cuda"),
                torch.zeros(4, dtype=torch.int32, device="cuda")[::2]):
        with pytest.raises(ValueError):
            bsa.bsa_bwd(q, q, q, q, lse, q, ml, None, 64, 64, KVV, kvv)
    with pytest.raises(ValueError):
        bsa.bsa_bwd(q, q, q, q, lse, q, ml, None, 64, 64, KVV, None)


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


def _varlen_setup(rng, mm, sq, sk, H, Hkv, D, bq, bk, window=None):
    """Random per-sequence block masks (CAUSAL / LOCAL: the classifier's
    partial blocks plus 70 % of its full ones; NONE / KVV: 40 % of the
    blocks, split between the lists), the packed device lists, the cu arrays
    of both roles and per-sequence valid counts (KVV)."""
    full, part = [], []
    for a, c in zip(sq, sk):
        M, N = -(-a // bq), -(-c // bk)
        if mm in (CAUSAL, LOCAL):
            f_c, p_c = oracle.block_sparsity(mm, a, c, bq, bk, window=window)
            f = np.broadcast_to(f_c.astype(bool), (H, M, N)) & (rng.random((H, M, N)) < 0.7)
            p = np.broadcast_to(p_c.astype(bool), (H, M, N)).copy()
        else:
            sel = rng.random((H, M, N)) < 0.4
            split = rng.random((H, M, N)) < 0.5 if mm == KVV else np.ones((H, M, N), bool)
            f, p = sel & split, sel & ~split
        full.append(f)
        part.append(p)
    cu, off, tm, tn = bsa.bsa_varlen_offsets(sq, sk, bq, bk)
    cu_kv, off_t, tkv, tn_t = bsa.bsa_varlen_offsets(sk, sq, bk, bq)
    assert off_t == off and tn_t == tn
    dev = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")

    def packed(masks):
        out = np.zeros((H, tn), np.uint8)
        for b, m in enumerate(masks):
            nm, nn = m.shape[1:]
            for i in range(nm):
                out[:, off[b] + i * nn: off[b] + (i + 1) * nn] = m[:, i]
        return torch.from_numpy(out).cuda()
    cu_m, offs = dev(cu), dev(off)
    ml = bsa.bsa_varlen_mask_to_index(packed(part), cu_m, offs, tm, tn) if tn else None
    fl = bsa.bsa_varlen_mask_to_index(packed(full), cu_m, offs, tm, tn) if tn else None
    kvv = None
    if mm == KVV:
        W = max(-(-c // bk) for c in sk) + 2
        kvv = rng.integers(0, bk + 3, size=(len(sk), W)).astype(np.int32)
    meta = dict(cu_q=dev([0] + list(np.cumsum(sq))), cu_k=dev([0] + list(np.cumsum(sk))),
                cu_m=cu_m, cu_kv=dev(cu_kv), offs=offs, tm=tm, tkv=tkv, tn=tn)
    return full, part, ml, fl, kvv, meta


@pytest.mark.parametrize("case", [
    dict(mm=CAUSAL, sq=[300, 0, 129, 517, 64], sk=[300, 0, 129, 517, 64], D=128, bq=64, bk=64),
    dict(mm=KVV, sq=[200, 450, 33], sk=[260, 120, 500], D=64, bq=128, bk=48),
    dict(mm=NONE, sq=[130, 77, 400], sk=[517, 0, 90], D=96, bq=64, bk=112),
    dict(mm=LOCAL, sq=[333, 260], sk=[333, 260], D=256, bq=128, bk=128, window=(70, 10)),
    dict(mm=CAUSAL, sq=[250, 190, 31], sk=[250, 190, 31], D=192, bq=64, bk=64),
    dict(mm=CAUSAL, sq=[384, 128], sk=[384, 128], D=128, bq=128, bk=128),
])
def test_varlen_bwd_matches_oracle(case):
    # packed varlen backward (bsa_varlen_bwd) against the varlen oracle,
    # every token of every sequence; empty sequences and Sq != Sk included
    seed = zlib.crc32(repr(sorted(case.items())).encode())
    rng = np.random.default_rng(seed)
    mm, sq, sk, D, bq, bk = case["mm"], case["sq"], case["sk"], case["D"], case["bq"], case["bk"]
    window = case.get("window")
    H, Hkv = 4, 2
    full, part, ml, fl, kvv, m = _varlen_setup(rng, mm, sq, sk, H, Hkv, D, bq, bk, window)
    q, k, v = (to_dev(rng.standard_normal(s, dtype=np.float32))
               for s in ((sum(sq), H, D), (sum(sk), Hkv, D), (sum(sk), Hkv, D)))
    do = to_dev(rng.standard_normal((sum(sq), H, D), dtype=np.float32))
    kvv_d = None if kvv is None else torch.from_numpy(kvv).cuda()
    scale = 1 / math.sqrt(D)
    print(f"varlen bwd case {case}", flush=True)
    o, lse = bsa.bsa_varlen_fwd(q, k, v, m["cu_q"], m["cu_k"], m["cu_m"], m["offs"], m["tm"],
                                m["tn"], ml, fl, bq, bk, mm, scale, window=window, kv_valid=kvv_d,
                                max_seqlen_k=max(sk))
    dq, dk, dv = bsa.bsa_varlen_bwd(q, k, v, o, lse, do, m["cu_q"], m["cu_k"], m["cu_m"],
                                    m["cu_kv"], m["offs"], m["tm"], m["tkv"], m["tn"], ml, fl,
                                    bq, bk, mm, kvv_d, scale, window=window)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.varlen_blocksparse_attention_bwd(
        as_oracle(q), as_oracle(k), as_oracle(v), sq, sk, full, part, bq, bk, mm, scale,
        as_oracle(do), kv_valid=None if kvv is None else list(kvv), window=window)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gg = as_oracle(g)
        assert np.isfinite(gg).all(), f"{name}: NaN/inf"
        err = float(np.abs(gg - r).max())
        ref = float(np.abs(r).max())
        print(f"  {name}: max err {err:.3e}, max |grad| {ref:.3e}")
        assert err <= REL_TOL * max(ref, 1e-6), f"{name} {case}: err {err:.3e} vs max {ref:.3e}"


@pytest.mark.parametrize("sq,sk,bq,bk", [([300, 0, 129, 517], [250, 100, 1, 0], 64, 48),
                                         ([1000, 64, 333], [1000, 64, 333], 128, 128)])
def test_varlen_kv_major_lists_bit_exact(sq, sk, bq, bk):
    rng = np.random.default_rng(len(sq) * 7 + bq)
    H = 3
    full, part, ml, fl, _, m = _varlen_setup(rng, NONE, sq, sk, H, H, 64, bq, bk)
    cnt_t, idx_t = bsa.bsa_varlen_kv_major_lists(fl, m["cu_m"], m["cu_kv"], m["offs"], m["tm"],
                                                 m["tkv"])
    torch.cuda.synchronize()
    rc, ri = oracle.varlen_kv_major_lists(full, sq, sk, bq, bk)
    np.testing.assert_array_equal(cnt_t.cpu().numpy(), rc)
    np.testing.assert_array_equal(idx_t.cpu().numpy(), ri)


def test_varlen_bwd_rejects_short_valid_counts():
    # per-sequence valid counts must cover ceil(max_seqlen_k / block_kv) blocks
    rng = np.random.default_rng(3)
    sq, sk, H, D, bq, bk = [100, 60], [200, 90], 2, 64, 64, 64
    full, part, ml, fl, kvv, m = _varlen_setup(rng, KVV, sq, sk, H, H, D, bq, bk)
    q = torch.zeros((sum(sq), H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((sum(sk), H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((H, sum(sq)), dtype=torch.float32, device="cuda")
    short = torch.from_numpy(kvv[:, :2].copy()).cuda()  # 4 blocks needed (200 keys)
    with pytest.raises(ValueError):
        bsa.bsa_varlen_bwd(q, k, k, q, lse, q, m["cu_q"], m["cu_k"], m["cu_m"], m["cu_kv"],
                           m["offs"], m["tm"], m["tkv"], m["tn"], ml, fl, bq, bk, KVV, short)


# ------------------------------------------ fp32 tensors (bsa_bwd_f32)
@pytest.mark.parametrize("case", [
    dict(mm=CAUSAL, Sq=300, Sk=300, D=128, bq=128, bk=64),
    dict(mm=KVV, Sq=200, Sk=450, D=64, bq=64, bk=48),
    dict(mm=LOCAL, Sq=260, Sk=260, D=192, bq=64, bk=128, window=(70, 0)),
])
def test_bwd_fp32_tensors(case):
    # fp32 q, k, v, o, dout: the gradients are those of the bf16 path on the
    # same tensors rounded to bf16, widened to fp32 (bit for bit), and within
    # the 1 % bound of the float64 oracle on the rounded inputs.
    seed = zlib.crc32(repr(sorted(case.items())).encode())
    rng = np.random.default_rng(seed)
    mm, Sq, Sk, D, bq, bk = case["mm"], case["Sq"], case["Sk"], case["D"], case["bq"], case["bk"]
    window = case.get("window")
    B, H, Hkv = 2, 4, 2
    M, N = -(-Sq // bq), -(-Sk // bk)
    q, k, v, do = (torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).cuda()
                   for s in ((B, Sq, H, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, H, D)))
    kvv = None
    if mm in (CAUSAL, LOCAL):
        f_c, p_c = oracle.block_sparsity(mm, Sq, Sk, bq, bk, window=window)
        full = f_c.astype(bool)[None, None] & (rng.random((B, H, M, N)) < 0.7)
        part = np.broadcast_to(p_c.astype(bool), (B, H, M, N)).copy()
    else:
        sel = rng.random((B, H, M, N)) < 0.5
        split = rng.random((B, H, M, N)) < 0.5
        full, part = sel & split, sel & ~split
        kvv = rng.integers(0, bk + 1, N).astype(np.int32)
    ml = _lists(part) if part.any() else None
    fl = _lists(full) if full.any() else None
    kvv_d = None if kvv is None else torch.from_numpy(kvv).cuda()
    scale = 1 / math.sqrt(D)
    o, lse = bsa.bsa_fwd(q, k, v, ml, fl, bq, bk, mm, kvv_d, scale, window=window)
    assert o.dtype == torch.float32
    dq, dk, dv = bsa.bsa_bwd(q, k, v, o, lse, do, ml, fl, bq, bk, mm, kvv_d, scale, window=window)
    assert dq.dtype == dk.dtype == dv.dtype == torch.float32
    r16 = [t.to(torch.bfloat16) for t in (q, k, v, o, do)]
    g16 = bsa.bsa_bwd(*r16[:4], lse, r16[4], ml, fl, bq, bk, mm, kvv_d, scale, window=window)
    torch.cuda.synchronize()
    for name, g, h in zip(("dq", "dk", "dv"), (dq, dk, dv), g16):
        assert torch.equal(g, h.float()), f"{name}: fp32 path differs from the bf16 path"
    rq, rk, rv = oracle.blocksparse_attention_bwd(as_oracle(r16[0]), as_oracle(r16[1]),
                                                  as_oracle(r16[2]), full, part, bq, bk, mm,
                                                  scale, as_oracle(r16[4]), kv_valid=kvv,
                                                  window=window)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gg = g.double().cpu().numpy()
        err, ref = float(np.abs(gg - r).max()), float(np.abs(r).max())
        print(f"bwd fp32 {case} {name}: ratio {err / max(ref, 1e-6):.2e}")
        assert err <= REL_TOL * max(ref, 1e-6), f"{name} {case}: err {err:.3e} vs max {ref:.3e}"


def test_bwd_fp32_rejects_noalloc_and_mixed_dtypes():
    q = torch.zeros((1, 64, 1, 64), dtype=torch.float32, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    fl = _lists(np.ones((1, 1, 1, 1), bool))
    with pytest.raises(ValueError):
        bsa.bsa_bwd(q, q, q, q, lse, q, None, fl, 64, 64, noalloc=True)
    with pytest.raises(ValueError):
        bsa.bsa_bwd(q, q, q, q, lse, q.to(torch.bfloat16), None, fl, 64, 64)
