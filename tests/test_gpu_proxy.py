"""GPU: the proxy-compensated route (bsa_fwd with proxy=(k_mean, v_sum))
against oracle.proxy_attention on the same bf16 inputs and summaries."""
import math
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_bsa_amd as bsa
import oracle
from bsa_testlib import as_oracle, check_o_lse, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, B, Sq, Sk, H, Hkv, D, bq, bk, density, listed_rows=None):
    rng = np.random.default_rng(seed)
    q, k, v = (to_dev(rng.standard_normal(s, dtype=np.float32))
               for s in ((B, Sq, H, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D)))
    M, N = -(-Sq // bq), -(-Sk // bk)
    sel = rng.random((B, H, M, N)) < density
    if listed_rows is not None:
        for (b, h, i), val in listed_rows.items():
            sel[b, h, i] = val
    split = rng.random((B, H, M, N)) < 0.5
    full, part = sel & split, sel & ~split
    kbar, vsum = oracle.block_summaries(as_oracle(k), as_oracle(v), bk)
    ks, vs = (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda() for x in (kbar, vsum))
    return q, k, v, full, part, ks, vs


def _lists(m):
    return bsa.bsa_mask_to_index(torch.from_numpy(np.ascontiguousarray(m, np.uint8)).cuda())


def _run(q, k, v, full, part, ks, vs, bq, bk, q_blocks=None):
    D = q.shape[-1]
    scale = 1 / math.sqrt(D)
    o, lse = bsa.bsa_fwd(q, k, v, _lists(part) if part.any() else None,
                         _lists(full) if full.any() else None, bq, bk, bsa.MASK_NONE, None,
                         scale, validate=True, proxy=(ks, vs))
    torch.cuda.synchronize()
    O, L = oracle.proxy_attention(as_oracle(q), as_oracle(k), as_oracle(v), full, part,
                                  as_oracle(ks), as_oracle(vs), bq, bk, scale, q_blocks=q_blocks)
    return o, lse, O, L


@pytest.mark.parametrize("case", [
    dict(Sq=300, Sk=700, D=128, bq=128, bk=128, density=0.3),
    dict(Sq=256, Sk=1000, D=64, bq=64, bk=64, density=0.4),
    dict(Sq=200, Sk=4033, D=128, bq=64, bk=16, density=0.1),     # 253 blocks: 4 chunks, tail of 1
    dict(Sq=256, Sk=5000, D=96, bq=32, bk=48, density=0.2),
    dict(Sq=130, Sk=900, D=192, bq=128, bk=64, density=0.25),
    dict(Sq=100, Sk=777, D=256, bq=64, bk=64, density=0.25),
    dict(Sq=512, Sk=16000, D=128, bq=256, bk=16, density=0.05),  # 1000 blocks, 256-row Q blocks
])
def test_proxy_matches_oracle(case):
    seed = zlib.crc32(repr(sorted(case.items())).encode())
    B, H, Hkv = 2, 4, 2
    listed = {(0, 0, 0): True, (0, 1, 0): False}  # one row all listed, one with no listed block
    q, k, v, full, part, ks, vs = _case(seed, B, H=H, Hkv=Hkv, listed_rows=listed, **case)
    o, lse, O, L = _run(q, k, v, full, part, ks, vs, case["bq"], case["bk"])
    check_o_lse(o, lse, O, L, f"proxy {case}")


@pytest.mark.parametrize("bq,bk", [(128, 128), (64, 64)])
def test_all_listed_rows_equal_the_plain_forward_bit_for_bit(bq, bk):
    """Summaries of listed blocks never enter, and exact blocks take the
    plain kernel's arithmetic."""
    q, k, v, full, part, ks, vs = _case(11, 1, 256, 640, 2, 1, 128, bq, bk, 1.0)
    a = bsa.bsa_fwd(q, k, v, _lists(part), _lists(full), bq, bk, bsa.MASK_NONE, None, 0.1,
                    proxy=(torch.randn_like(ks), torch.randn_like(vs)))
    b = bsa.bsa_fwd(q, k, v, _lists(part), _lists(full), bq, bk, bsa.MASK_NONE, None, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("D,bq,bk", [(128, 128, 64), (64, 64, 48)])
def test_summaries_in_another_layout(D, bq, bk):
    """Summaries whose row stride differs from K's and V's take the
    register-staged kernel; both layouts match the oracle."""
    q, k, v, full, part, ks, vs = _case(13, 2, 300, 900, 4, 2, D, bq, bk, 0.3)
    ks2 = ks.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)  # [B,N,Hkv,D], row stride D
    vs2 = vs.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert ks2.stride(1) != k.stride(1)
    o, lse, O, L = _run(q, k, v, full, part, ks2, vs2, bq, bk)
    check_o_lse(o, lse, O, L, f"proxy, summaries [B,Hkv,N,D] d{D}")
    o1, l1, _, _ = _run(q, k, v, full, part, ks, vs, bq, bk)
    check_o_lse(o1, l1, O, L, f"proxy, summaries [B,N,Hkv,D] d{D}")


def test_pages_workload_sampled():
    """B1 Sq=Sk=32760 H12 d128, 64x64 blocks, 84 of 512 blocks listed per row
    (the proxy workload of the PrimTS page), sampled Q blocks against the oracle."""
    B, S, H, D, bq, bk, per_row = 1, 32760, 12, 128, 64, 64, 84
    rng = np.random.default_rng(1007)
    q, k, v = (to_dev(rng.standard_normal((B, S, H, D), dtype=np.float32)) for _ in range(3))
    M = N = -(-S // 64)
    sel = np.zeros((B, H, M, N), bool)
    for h in range(H):
        for i in range(M):
            sel[0, h, i, rng.choice(N, per_row, replace=False)] = True
    full, part = sel, np.zeros_like(sel)
    kk = k.float().cpu().numpy().astype(np.float64)
    vv = v.float().cpu().numpy().astype(np.float64)
    kbar, vsum = oracle.block_summaries(kk, vv, bk)
    ks, vs = (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda() for x in (kbar, vsum))
    blocks = [(0, int(h), int(i)) for h, i in zip(rng.integers(0, H, 12), rng.integers(0, M, 12))]
    blocks.append((0, 0, M - 1))  # the ragged last Q block
    o, lse, O, L = _run(q, k, v, full, part, ks, vs, bq, bk, q_blocks=blocks)
    rows = np.concatenate([np.arange(i * bq, min((i + 1) * bq, S)) for _, _, i in blocks])
    heads = np.concatenate([np.full(min((i + 1) * bq, S) - i * bq, h) for _, h, i in blocks])
    zero = np.zeros_like(rows)
    check_o_lse(o, lse, O, L, "proxy pages workload (sampled)",
                sel=((zero, rows, heads), (zero, heads, rows)))


def test_proxy_rejects_what_it_does_not_cover():
    q, k, v, full, part, ks, vs = _case(12, 1, 128, 256, 2, 2, 64, 64, 64, 0.5)
    with pytest.raises(bsa.BsaError):
        bsa.bsa_fwd(q, k, v, None, _lists(full), 64, 64, bsa.MASK_CAUSAL, None, 0.1,
                    proxy=(ks, vs))
    with pytest.raises(bsa.BsaError):
        bsa.bsa_fwd(q.float(), k.float(), v.float(), None, _lists(full), 64, 64, bsa.MASK_NONE,
                    None, 0.1, proxy=(ks.float(), vs.float()))
    with pytest.raises(ValueError):
        bsa.bsa_fwd(q, k, v, None, _lists(full), 64, 64, bsa.MASK_NONE, None, 0.1,
                    proxy=(ks[:, :-1], vs))


# ------------------------------------------ backward (bsa_bwd_proxy)
BWD_REL_TOL = 1e-2  # of each gradient's largest magnitude, as for bsa_bwd


@pytest.mark.parametrize("case", [
    dict(Sq=300, Sk=300, D=64, bq=64, bk=64, density=0.3),
    dict(Sq=200, Sk=333, D=128, bq=128, bk=48, density=0.4),  # short last block (45 tokens)
    dict(Sq=150, Sk=410, D=96, bq=64, bk=80, density=0.25),
    dict(Sq=128, Sk=257, D=256, bq=64, bk=64, density=0.3),   # a last block of one token
    # full last blocks (no chunk of its own), 128-key blocks (two sub-tiles per chunk)
    dict(Sq=256, Sk=512, D=128, bq=128, bk=128, density=0.3),
    # 100 full 80-key blocks: the second chunk's positions 80.. straddle two 64-bit words
    dict(Sq=192, Sk=8000, D=64, bq=64, bk=80, density=0.1),
    # 16 full 16-key blocks fill their chunk exactly; the 5-token last one starts the next
    dict(Sq=128, Sk=261, D=128, bq=64, bk=16, density=0.3),
])
def test_proxy_backward_matches_oracle(case):
    # dq, dk, dv and both summaries' gradients against the float64 oracle on
    # the same bf16 inputs, with the forward's O and LSE
    seed = zlib.crc32(repr(sorted(case.items())).encode())
    B, H, Hkv = 2, 4, 2
    D, bq, bk = case["D"], case["bq"], case["bk"]
    q, k, v, full, part, ks, vs = _case(seed, B, case["Sq"], case["Sk"], H, Hkv, D, bq, bk,
                                        case["density"])
    full[0, 0, 0] = part[0, 0, 0] = False  # a row of proxies only
    full[1, 3, 1] = True                    # a row of exact blocks only
    part[1, 3, 1] = False
    scale = 1 / math.sqrt(D)
    ml = _lists(part) if part.any() else None
    fl = _lists(full) if full.any() else None
    o, lse = bsa.bsa_fwd(q, k, v, ml, fl, bq, bk, bsa.MASK_NONE, None, scale, proxy=(ks, vs))
    do = to_dev(np.random.default_rng(seed + 1).standard_normal(q.shape, dtype=np.float32))
    grads = bsa.bsa_bwd(q, k, v, o, lse, do, ml, fl, bq, bk, bsa.MASK_NONE, None, scale,
                        proxy=(ks, vs))
    torch.cuda.synchronize()
    refs = oracle.proxy_attention_bwd(as_oracle(q), as_oracle(k), as_oracle(v), full, part,
                                      as_oracle(ks), as_oracle(vs), bq, bk, scale, as_oracle(do))
    for name, g, r in zip(("dq", "dk", "dv", "dk_mean", "dv_sum"), grads, refs):
        gg = as_oracle(g)
        assert np.isfinite(gg).all(), f"{name}: NaN/inf"
        err, ref = float(np.abs(gg - r).max()), float(np.abs(r).max())
        print(f"proxy bwd {case} {name}: ratio {err / max(ref, 1e-6):.2e}")
        assert err <= BWD_REL_TOL * max(ref, 1e-6), f"{name} {case}: err {err:.3e} vs {ref:.3e}"


def test_proxy_backward_all_listed_is_the_plain_backward():
    # every block listed: no proxy term, so the gradients are bsa_bwd's and
    # the summaries' are zero
    B, H, Hkv, D, bq, bk, Sq, Sk = 1, 2, 1, 64, 64, 64, 192, 200
    q, k, v, full, part, ks, vs = _case(5, B, Sq, Sk, H, Hkv, D, bq, bk, 1.0)
    scale = 1 / math.sqrt(D)
    ml = _lists(part) if part.any() else None
    fl = _lists(full) if full.any() else None
    o, lse = bsa.bsa_fwd(q, k, v, ml, fl, bq, bk, bsa.MASK_NONE, None, scale, proxy=(ks, vs))
    do = to_dev(np.random.default_rng(6).standard_normal(q.shape, dtype=np.float32))
    dq, dk, dv, dks, dvs = bsa.bsa_bwd(q, k, v, o, lse, do, ml, fl, bq, bk, bsa.MASK_NONE, None,
                                       scale, proxy=(ks, vs))
    rq, rk, rv = bsa.bsa_bwd(q, k, v, o, lse, do, ml, fl, bq, bk, bsa.MASK_NONE, None, scale)
    torch.cuda.synchronize()
    assert not dks.any() and not dvs.any()
    for g, r in ((dq, rq), (dk, rk), (dv, rv)):
        gg, rr = as_oracle(g), as_oracle(r)
        assert float(np.abs(gg - rr).max()) <= 1e-2 * float(np.abs(rr).max())


def test_proxy_backward_rejects_what_it_does_not_cover():
    q = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    s = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
    fl = _lists(np.ones((1, 1, 1, 1), bool))
    with pytest.raises(ValueError):   # element masks are not part of the route
        bsa.bsa_bwd(q, q, q, q, lse, q, fl, None, 64, 64, bsa.MASK_CAUSAL, proxy=(s, s))
    with pytest.raises(ValueError):   # summaries of the wrong shape
        bsa.bsa_bwd(q, q, q, q, lse, q, None, fl, 64, 64, proxy=(s[:, :, :, :32], s))
