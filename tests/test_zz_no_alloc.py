"""The allocation-free backward entry point (bsa_bwd_noalloc): same results as
bsa_bwd, whose row-dot workspace the caller passes, on two calls in a row
(the second smaller, so it reads only what it wrote itself into the shared
static array); sizes past the array are rejected before any device work."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_bsa_amd as bsa
import workloads
from bsa_testlib import lists_on_device, to_dev


def _case(D, bq, bk, B, H, S, seed, mask_mod):
    w = workloads.sparse_sweep(D, bq, bk, B=B, H=H, S=S, density=0.4, seed=seed)
    q, k, v = (to_dev(x) for x in (w.q, w.k, w.v))
    ml, fl = lists_on_device(w.part), lists_on_device(w.full)
    o, lse = bsa.bsa_fwd(q, k, v, ml, fl, bq, bk, mask_mod, None, w.scale)
    g = to_dev(np.random.default_rng(seed).standard_normal(o.shape).astype(np.float32))
    return (q, k, v, o, lse, g, ml, fl, bq, bk, mask_mod, None, w.scale)


@pytest.mark.gpu
def test_noalloc_backward_equals_workspace_backward():
    big = _case(128, 128, 64, 2, 4, 700, 41, bsa.MASK_CAUSAL)
    small = _case(64, 64, 48, 1, 2, 230, 42, bsa.MASK_NONE)
    for args in (big, small):  # second call smaller than the first
        ref = bsa.bsa_bwd(*args)
        got = bsa.bsa_bwd(*args, noalloc=True)
        torch.cuda.synchronize()
        for r, x in zip(ref, got):
            assert torch.isfinite(x.float()).all()
            assert torch.equal(r, x)


def test_noalloc_rejects_rows_past_the_static_array():
    # checked on the host before anything touches a device: B*H*Sq past 2**22
    lib = bsa.load_library()
    P = ctypes.c_void_p(256)  # never dereferenced: the size check comes first
    st = (ctypes.c_int64 * 3)(1 << 20, 128, 1 << 27)
    bl = bsa._BlockList()
    bs = bsa._BlockSparse(bl, bl, 128, 128, -1, -1)
    rc = lib.bsa_bwd_noalloc(P, P, P, P, P, P, P, P, P, 1, 1, 1, (1 << 22) + 1, 128, 128,
                             st, st, st, st, ctypes.byref(bs), ctypes.byref(bl),
                             ctypes.byref(bl), 0, None, 0.1, None)
    assert rc == bsa.BSA_ERR_UNSUPPORTED
