"""GQA head packing: block lists given per KV head (shared by that KV head's Q
heads), against the oracle run with the lists repeated over the Q heads.
Where the 256-row kernel serves the shape, one workgroup packs G = 256/tile
heads; elsewhere the lists are read through the KV head unpacked.  Every row
is compared (parity criteria: tests/bsa_testlib.py)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_bsa_amd as bsa
import oracle
import workloads
from bsa_testlib import as_oracle, check_o_lse, lists_on_device, to_dev

pytestmark = pytest.mark.gpu


def _run(w, hrep, dtype=torch.bfloat16, mask_mod=None, window=None, kvv=None, lists=None):
    q, k, v = (to_dev(x, dtype) for x in (w.q, w.k, w.v))
    ml, fl = lists if lists is not None else (lists_on_device(w.part), lists_on_device(w.full))
    mm = w.mask_mod if mask_mod is None else mask_mod
    o, lse = bsa.bsa_fwd(q, k, v, ml, fl, w.block_q, w.block_kv, mm,
                         None if kvv is None else torch.from_numpy(kvv).cuda(), w.scale,
                         window=window, kv_head_lists=lists is None, validate=True)
    torch.cuda.synchronize()
    rep = lambda m: np.repeat(m, hrep, axis=1)
    qo, ko, vo = (as_oracle(t.to(torch.bfloat16)) for t in (q, k, v))
    O, L = oracle.blocksparse_attention(qo, ko, vo, rep(w.full), rep(w.part), w.block_q,
                                        w.block_kv, mm, w.scale, kvv, window=window)
    return o, lse, O, L


@pytest.mark.parametrize("D,bq,bk,Hkv,hrep", [
    (128, 128, 128, 2, 2),   # G = 2
    (64, 64, 64, 1, 4),      # G = 4
    (128, 32, 64, 1, 8),     # G = 8
    (128, 112, 112, 2, 2),   # G = 2, 112-row blocks (rows clipped at the block end)
    (96, 128, 64, 1, 4),     # G = 2, two packed groups per KV head
    (128, 64, 128, 2, 8),    # G = 4
    (128, 128, 96, 2, 3),    # 3 heads per KV head: not packed, lists read via the KV head
    (192, 128, 128, 1, 2),   # head_dim 192: the 4-wave kernel, lists via the KV head
])
def test_gqa_packed_heads_match_oracle(D, bq, bk, Hkv, hrep):
    w = workloads.gqa_sweep(D, bq, bk, Hkv, hrep, B=2, S=700, density=0.4,
                            seed=[3, D, bq, bk, Hkv, hrep])
    o, lse, O, L = _run(w, hrep)
    check_o_lse(o, lse, O, L, f"gqa D={D} ({bq},{bk}) Hkv={Hkv} x{hrep}")


def test_gqa_other_kernels_and_masks():
    # fp32 inputs (register-staged kernel), the local mask_mod and the valid
    # count with per-KV-head lists
    w = workloads.gqa_sweep(64, 64, 64, 1, 4, B=1, S=300, density=0.5, seed=8)
    o, lse, O, L = _run(w, 4, dtype=torch.float32)
    check_o_lse(o, lse, O, L, "gqa fp32")
    o, lse, O, L = _run(w, 4, mask_mod=bsa.MASK_LOCAL, window=(100, 0))
    check_o_lse(o, lse, O, L, "gqa local")
    kvv = np.random.default_rng(9).integers(0, 65, w.full.shape[-1]).astype(np.int32)
    o, lse, O, L = _run(w, 4, mask_mod=bsa.MASK_KV_VALID_COUNT, kvv=kvv)
    check_o_lse(o, lse, O, L, "gqa valid count")


def test_lists_broadcast_over_heads_are_packed_alike():
    # one list row for every head (head strides 0): packed without the flag,
    # results equal the flagged per-KV-head call bit for bit
    w = workloads.gqa_sweep(128, 128, 128, 1, 4, B=1, S=900, density=0.3, seed=10)
    ml, fl = lists_on_device(w.part), lists_on_device(w.full)  # [1, 1, M, N]
    o1, l1, O, L = _run(w, 4)
    o2, l2, _, _ = _run(w, 4, lists=(ml, fl))
    check_o_lse(o2, l2, O, L, "broadcast lists")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("bq,hrep", [(128, 2), (64, 4)])
def test_gqa_varlen(bq, hrep):
    Hkv = 2
    w = workloads.varlen_packed(n_seq=4, H=Hkv, D=128, bs=bq, lo=100, hi=1200, seed=20 + bq)
    H = Hkv * hrep
    rng = np.random.default_rng(bq)
    qx = rng.standard_normal((w.q.shape[0], H, 128)).astype(np.float32)
    cu, off, tm, tn = bsa.bsa_varlen_offsets(w.seqlens_q, w.seqlens_k, bq, bq)
    dv = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    cu_q = dv([0] + list(np.cumsum(w.seqlens_q)))
    cu_k = dv([0] + list(np.cumsum(w.seqlens_k)))

    def packed(masks):
        out = np.zeros((Hkv, tn), np.uint8)
        for b, m in enumerate(masks):
            nm, nn = m.shape[1:]
            for i in range(nm):
                out[:, off[b] + i * nn: off[b] + (i + 1) * nn] = m[:, i]
        return torch.from_numpy(out).cuda()

    cu_m, offs = dv(cu), dv(off)
    ml = bsa.bsa_varlen_mask_to_index(packed(w.part), cu_m, offs, tm, tn)
    fl = bsa.bsa_varlen_mask_to_index(packed(w.full), cu_m, offs, tm, tn)
    q, k, v = to_dev(qx), to_dev(w.k), to_dev(w.v)
    o, lse = bsa.bsa_varlen_fwd(q, k, v, cu_q, cu_k, cu_m, offs, tm, tn, ml, fl, bq, bq,
                                w.mask_mod, w.scale, kv_head_lists=True, validate=True)
    torch.cuda.synchronize()
    rep = lambda ms: [np.repeat(m, hrep, axis=0) for m in ms]
    O, L = oracle.varlen_blocksparse_attention(as_oracle(q), as_oracle(k), as_oracle(v),
                                               w.seqlens_q, w.seqlens_k, rep(w.full),
                                               rep(w.part), bq, bq, w.mask_mod, w.scale)
    check_o_lse(o, lse, O, L, f"gqa varlen bq={bq} x{hrep}")
