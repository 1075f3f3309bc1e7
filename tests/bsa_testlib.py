"""Shared helpers for the GPU parity tests: uploads, metadata through the
library, and the parity criteria.

Tolerances (one reading, stated once):
  * fp32 O:  |O - O_oracle| <= 4e-3
  * bf16 O:  |O - O_oracle| - ulp_bf16(O_oracle)/2 <= 4e-3  (the bf16 output
    rounding alone is half an ulp, 7.8e-3 at |O| in [2,4))
  * LSE:     |LSE - LSE_oracle| <= 1e-3, and -inf exactly where the oracle has -inf
  * metadata and offsets: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_bsa_amd as bsa

O_TOL = 4e-3
LSE_TOL = 1e-3


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def to_dev(x: np.ndarray, dtype=torch.bfloat16, device="cuda") -> torch.Tensor:
    """fp32 numpy -> device tensor in `dtype` (the cast rounds to nearest even on the CPU)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(device)


def as_oracle(t: torch.Tensor) -> np.ndarray:
    """The exact values the kernel reads, as float64 for the oracle."""
    return t.detach().float().cpu().double().numpy()


def lists_on_device(mask: np.ndarray):
    """Dense bool block mask [B,H,M,N] -> (cnt, idx) built by bsa_mask_to_index."""
    m = torch.from_numpy(np.ascontiguousarray(mask.astype(np.uint8))).cuda()
    return bsa.bsa_mask_to_index(m)


def check_o_lse(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, o_ref: np.ndarray, lse_ref: np.ndarray,
                what: str = "", sel=None):
    """Assert the parity criteria; sel restricts to sampled positions (numpy index).
    Returns (raw max |dO|, max |dLSE|)."""
    o = o_gpu.detach().float().cpu().double().numpy()
    lse = lse_gpu.detach().float().cpu().double().numpy()
    if sel is not None:
        o_sel, or_sel = o[sel[0]], o_ref[sel[0]]
        l_sel, lr_sel = lse[sel[1]], lse_ref[sel[1]]
    else:
        o_sel, or_sel, l_sel, lr_sel = o, o_ref, lse, lse_ref
    assert np.isfinite(or_sel).all(), f"{what}: oracle O has NaN/inf (sampling bug)"
    assert np.isfinite(o_sel).all(), f"{what}: kernel O has NaN/inf"
    err = np.abs(o_sel - or_sel)
    if o_gpu.dtype == torch.bfloat16:
        excess = err - 0.5 * bf16_ulp(or_sel)
    else:
        excess = err
    worst = float(excess.max()) if excess.size else 0.0
    assert worst <= O_TOL, (f"{what}: O error {worst:.3e} over tolerance "
                            f"(raw max {float(err.max()):.3e})")
    ninf_ref = np.isneginf(lr_sel)
    assert (np.isneginf(l_sel) == ninf_ref).all(), f"{what}: LSE -inf pattern differs"
    fin = ~ninf_ref
    lerr = float(np.abs(l_sel[fin] - lr_sel[fin]).max()) if fin.any() else 0.0
    assert lerr <= LSE_TOL, f"{what}: LSE error {lerr:.3e}"
    return float(err.max()) if err.size else 0.0, lerr


def check_o_lse_fp32_normaliser(o_gpu, lse_gpu, o_ref, lse_ref, vmax: float, what: str = ""):
    """The bound of the 256-row kernel, which divides O by the sum of the fp32
    P while the PV product takes P rounded to bf16 (relative error <= 2^-8
    per weight): on rows dominated by a few keys these errors do not average
    out, and |O - O_oracle| <= 2^-8 * max|v| + half a bf16 ulp of O (1e-4
    slack for the fp32 arithmetic).  The LSE keeps its 1e-3.  Returns the
    raw max |dO|."""
    o = o_gpu.detach().float().cpu().double().numpy()
    lse = lse_gpu.detach().float().cpu().double().numpy()
    assert np.isfinite(o).all() and np.isfinite(o_ref).all(), what
    err = np.abs(o - o_ref)
    bound = 2.0 ** -8 * vmax + 0.5 * bf16_ulp(np.maximum(np.abs(o), np.abs(o_ref))) + 1e-4
    assert (err <= bound).all(), f"{what}: O error over 2^-8 max|v| by {float((err - bound).max()):.3e}"
    ninf = np.isneginf(lse_ref)
    assert (np.isneginf(lse) == ninf).all(), f"{what}: LSE -inf pattern differs"
    lerr = float(np.abs(lse[~ninf] - lse_ref[~ninf]).max()) if (~ninf).any() else 0.0
    assert lerr <= LSE_TOL, f"{what}: LSE error {lerr:.3e}"
    return float(err.max())


def run_batched(w, dtype=torch.bfloat16, lists=None, validate=False, q_view=None):
    """Upload a BatchedWorkload, build its lists on the GPU and run bsa_fwd.
    Returns (O, LSE, (q, k, v) device tensors)."""
    q, k, v = (to_dev(x, dtype) for x in (w.q, w.k, w.v))
    if lists is None:
        mlist = lists_on_device(w.part) if w.part.any() else None
        flist = lists_on_device(w.full) if w.full.any() else None
    else:
        mlist, flist = lists
    kvv = None if w.kv_valid is None else torch.from_numpy(np.asarray(w.kv_valid, np.int32)).cuda()
    o, lse = bsa.bsa_fwd(q, k, v, mlist, flist, w.block_q, w.block_kv, w.mask_mod, kvv,
                         w.scale, validate=validate)
    return o, lse, (q, k, v)


def sample_q_blocks(B, H, M, n, seed):
    rng = np.random.default_rng(seed)
    picks = {(0, 0, 0), (B - 1, H - 1, M - 1)}
    while len(picks) < min(n, B * H * M):
        picks.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(M))))
    return sorted(picks)


def rows_of(picks, block_q, Sq):
    """numpy fancy indices (for O [B,S,H,D] and LSE [B,H,S]) of the sampled Q blocks."""
    ob, os_, oh, lb, lh, ls = [], [], [], [], [], []
    for (b, h, i) in picks:
        r = np.arange(i * block_q, min((i + 1) * block_q, Sq))
        ob.append(np.full(r.size, b)); os_.append(r); oh.append(np.full(r.size, h))
        lb.append(np.full(r.size, b)); lh.append(np.full(r.size, h)); ls.append(r)
    o_sel = (np.concatenate(ob), np.concatenate(os_), np.concatenate(oh))
    l_sel = (np.concatenate(lb), np.concatenate(lh), np.concatenate(ls))
    return o_sel, l_sel
