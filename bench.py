"""Benchmark: effective TFLOP/s of the block-sparse attention forward on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload video|sweep128]

One step is the whole hot path over one synthetic batch already resident in
HBM: split the cube-level KV selection into 128-token tiles
(bsa_expand_kv_blocks), build the mask and full block lists
(bsa_mask_to_index, twice) and run the forward (bsa_fwd).

Default workload: video sparse attention, B=1, H=24, 30x48x52 latent grid in
4x8x8 = 256-token cubes (74880 tokens, 86016 padded rows), head_dim 128,
bf16, each Q cube attending to its top 40 of 336 KV cubes (11.9% density),
KV cubes run as 128-token tiles with per-tile valid-token counts.

FLOPs per step count the computed blocks: 4 * head_dim * sum over listed
(Q block, KV tile) pairs of (Q rows) x (KV tile keys), every listed 128-token
tile at its full 128 keys and every 256-row Q cube at 256 rows (KV tiles
with no valid token are never listed).  The count over valid keys only, 1.2 %
lower, is printed beside it.

Prints one JSON line.  `--gpus N` with N > 1 exits: this build runs on one GPU.

`--table` instead times the forward alone on every workload of the set (tiny
fp32, causal blocks, the 25 head_dim x block-size sweep runs, varlen packed,
video) and prints a markdown table: GPU milliseconds (median of 20 launches,
HIP events), effective TFLOP/s and % of the bf16 peak, and the oracle's rate
on a sample of Q blocks of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (computed blocks) bf16 block-sparse attn fwd; % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_SCLK_MHZ = 2400.0     # the clock that peak is quoted at
# sources of the forward kernel the video workload launches (256-row workgroups)
FWD_KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_attention_bsa_amd", "csrc", f)
                   for f in ("bsa_fwd_pp.hip", "bsa_fwd_common.h")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "bsa_fwd_pp_kernel_video_hbm_traffic.md")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=["video", "sweep128", "varlen", "bwd_sweep128"],
                    default="video")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-time budget of the oracle sample on the host (0 = skip)")
    ap.add_argument("--print-kernel-hash", action="store_true",
                    help="print the source hash the HBM-traffic summary is keyed on and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--table", action="store_true",
                    help="time the forward on every workload and print a markdown table")
    return ap.parse_args()


def _kernel_hash() -> str:
    h = hashlib.sha256()
    for path in FWD_KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _from_profile(key):
    """A per-launch figure from the committed counter summary of the forward
    kernel, or None if it is missing or was taken on another revision."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    b = re.search(re.escape(key) + r":\s*([0-9.eE+]+)", text)
    if not h or not b or h.group(1) != _kernel_hash():
        return None
    return float(b.group(1))


def _video_inputs(torch, np, workloads):
    w = workloads.video()
    dev = torch.device("cuda")
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
    cube_mask = torch.from_numpy(w.cube_mask.astype(np.uint8)).to(dev)
    cube_valid = torch.from_numpy(w.cube_valid).to(dev)
    # computed blocks: listed (cube, tile) pairs x 256 Q rows x 128 keys; a tile
    # with no valid token is not listed
    f = w.cube_elems // w.kv_tile
    tile_valid = np.clip(w.cube_valid[:, None] - np.arange(f)[None, :] * w.kv_tile, 0,
                         w.kv_tile)  # [cubes, f]
    full_tiles = (tile_valid > 0).sum(1).astype(np.float64) * w.kv_tile
    flops = 4.0 * q.shape[-1] * w.cube_elems * float(
        (w.cube_mask[0].astype(np.float64) @ full_tiles).sum())
    # the finer count: valid keys of each listed tile only
    keys_per_row = (w.cube_mask[0].astype(np.float64) @ tile_valid.sum(1).astype(np.float64))
    flops_valid_keys = 4.0 * q.shape[-1] * w.cube_elems * float(keys_per_row.sum())
    density = float(w.cube_mask.mean())
    cfg = {"workload": "video_sparse_attention", "B": 1, "H": q.shape[2], "tokens": int(
        w.cube_valid.sum()), "padded_seq": q.shape[1], "head_dim": q.shape[3], "cube": list(w.cube),
        "grid": list(w.grid), "block_q": w.cube_elems, "kv_tile": w.kv_tile,
        "kv_cubes_per_q_cube": int(w.cube_mask[0, 0, 0].sum()), "block_density": round(density, 4),
        "mask_mod": "kv_valid_count", "layout": "BSHD"}
    state = dict(q=q, k=k, v=v, cube_mask=cube_mask, cube_valid=cube_valid, f=f, w=w,
                 flops_valid_keys=flops_valid_keys)
    return state, flops, cfg


def _video_step(bsa, st, events=None):
    full, part, kvv = bsa.bsa_expand_kv_blocks(st["cube_mask"], st["cube_valid"], st["f"],
                                               st["w"].kv_tile)
    ml = bsa.bsa_mask_to_index(part)
    fl = bsa.bsa_mask_to_index(full)
    if events is not None:
        events[0].record()
    o, lse = bsa.bsa_fwd(st["q"], st["k"], st["v"], ml, fl, st["w"].cube_elems, st["w"].kv_tile,
                         bsa.MASK_KV_VALID_COUNT, kvv, st["w"].scale, out=st.get("o"),
                         lse=st.get("lse"))
    if events is not None:
        events[1].record()
    st["o"], st["lse"] = o, lse


def _sweep_inputs(torch, np, workloads):
    w = workloads.sparse_sweep(128, 128, 128)
    dev = torch.device("cuda")
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
    sel = (w.full | w.part).astype(np.float64)
    flops = 4.0 * 128 * 128 * 128 * float(sel.sum())
    cfg = {"workload": "blocksparse_sweep_d128", "B": 2, "H": 16, "seq": 4096, "head_dim": 128,
           "block_q": 128, "block_kv": 128, "block_density": round(float(sel.mean()), 4),
           "mask_mod": "causal_diagonal", "layout": "BSHD"}
    st = dict(q=q, k=k, v=v, w=w, part=torch.from_numpy(w.part.astype(np.uint8)).to(dev),
              full=torch.from_numpy(w.full.astype(np.uint8)).to(dev))
    return st, flops, cfg


def _sweep_step(bsa, st, events=None):
    ml = bsa.bsa_mask_to_index(st["part"])
    fl = bsa.bsa_mask_to_index(st["full"])
    if events is not None:
        events[0].record()
    o, lse = bsa.bsa_fwd(st["q"], st["k"], st["v"], ml, fl, 128, 128, bsa.MASK_CAUSAL, None,
                         st["w"].scale, out=st.get("o"), lse=st.get("lse"))
    if events is not None:
        events[1].record()
    st["o"], st["lse"] = o, lse


def _bwd_inputs(torch, np, workloads):
    # the d128 sweep's forward outputs and an upstream gradient, once
    import block_sparse_attention_bsa_amd as bsa
    st, flops, cfg = _sweep_inputs(torch, np, workloads)
    _sweep_step(bsa, st)
    st["do"] = torch.randn(st["q"].shape, generator=torch.Generator().manual_seed(77)).to(
        torch.bfloat16).to("cuda")
    st["ml"] = bsa.bsa_mask_to_index(st["part"])
    st["fl"] = bsa.bsa_mask_to_index(st["full"])
    cfg = dict(cfg, workload="blocksparse_sweep_d128_backward",
               flops="10*d per listed (row, key) cell: S, dP, dV, dK, dQ")
    return st, 2.5 * flops, cfg


def _bwd_step(bsa, st, events=None):
    # timed: the KV-major lists, the row dots, dQ and dK/dV
    if events is not None:
        events[0].record()
    bsa.bsa_bwd(st["q"], st["k"], st["v"], st["o"], st["lse"], st["do"], st["ml"], st["fl"],
                128, 128, bsa.MASK_CAUSAL, None, st["w"].scale)
    if events is not None:
        events[1].record()


def _varlen_inputs(torch, np, workloads):
    w = workloads.varlen_packed()
    dev = torch.device("cuda")
    H, bq, bk, D = w.q.shape[1], w.block_q, w.block_kv, w.q.shape[-1]
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
    flops = sum(_pairs_flops(fu[None], pa[None], bq, bk, sq, sk, D)
                for fu, pa, sq, sk in zip(w.full, w.part, w.seqlens_q, w.seqlens_k))
    M = sum(-(-s // bq) for s in w.seqlens_q)
    dens = sum(float((fu | pa).sum()) for fu, pa in zip(w.full, w.part)) / sum(
        fu.size for fu in w.full)
    cfg = {"workload": "varlen_packed", "sequences": len(w.seqlens_q), "tokens": int(
        sum(w.seqlens_q)), "H": H, "head_dim": D, "block_q": bq, "block_kv": bk,
        "total_m_blocks": M, "block_density": round(dens, 4),
        "mask_mod": "causal_diagonal_plus_random_30pct", "layout": "THD"}
    return dict(q=q, k=k, v=v, w=w), flops, cfg


def _varlen_step(bsa, st, events=None):
    import numpy as np
    import torch
    w = st["w"]
    bq, bk, H = w.block_q, w.block_kv, w.q.shape[1]
    if "cu" not in st:  # host bookkeeping and the packed masks, once (inputs of the step)
        cu, off, tm, tn = bsa.bsa_varlen_offsets(w.seqlens_q, w.seqlens_k, bq, bk)
        dv = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
        st["cu_q"] = dv([0] + list(np.cumsum(w.seqlens_q)))
        st["cu_k"] = dv([0] + list(np.cumsum(w.seqlens_k)))
        st["cu"], st["off"], st["tm"], st["tn"] = dv(cu), dv(off), tm, tn

        def packed(masks):
            out = np.zeros((H, tn), np.uint8)
            for b, m in enumerate(masks):
                nm, nn = m.shape[1:]
                for i in range(nm):
                    out[:, off[b] + i * nn: off[b] + (i + 1) * nn] = m[:, i]
            return torch.from_numpy(out).cuda()
        st["pm"], st["pf"] = packed(w.part), packed(w.full)
    ml = bsa.bsa_varlen_mask_to_index(st["pm"], st["cu"], st["off"], st["tm"], st["tn"])
    fl = bsa.bsa_varlen_mask_to_index(st["pf"], st["cu"], st["off"], st["tm"], st["tn"])
    if events is not None:
        events[0].record()
    o, lse = bsa.bsa_varlen_fwd(st["q"], st["k"], st["v"], st["cu_q"], st["cu_k"], st["cu"],
                                st["off"], st["tm"], st["tn"], ml, fl, bq, bk, w.mask_mod, w.scale,
                                out=st.get("o"), lse=st.get("lse"))
    if events is not None:
        events[1].record()
    st["o"], st["lse"] = o, lse


class _MaxErr:
    """Largest |GPU - oracle| over the Q blocks the oracle computed: raw for O
    and LSE, and for a bf16 O also beyond half a bf16 ulp of the oracle's value
    (the rounding of the stored output), the quantity the 4e-3 bound is on."""

    def __init__(self):
        self.n, self.o, self.o_excess, self.lse = 0, 0.0, 0.0, 0.0

    def note(self, o_gpu, lse_gpu, o_ref, lse_ref):
        import numpy as np
        self.n += 1
        err = np.abs(o_gpu.double().cpu().numpy() - o_ref)
        if o_gpu.dtype.itemsize == 2:
            a = np.abs(o_ref)
            ulp = 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)
            err_x = err - 0.5 * np.where(a > 0, ulp, 0.0)
        else:
            err_x = err
        self.o = max(self.o, float(err.max()))
        self.o_excess = max(self.o_excess, float(err_x.max()))
        self.lse = max(self.lse, float(np.abs(lse_gpu.double().cpu().numpy() - lse_ref).max()))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    """Threads numpy's BLAS runs the oracle's products on (set before numpy
    is imported: OMP_NUM_THREADS if the host sets it, else the CPUs this
    process may run on)."""
    try:
        from threadpoolctl import threadpool_info
        return max([int(i.get("num_threads", 1)) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return 1


def _cpu_baseline(np, st, workload, budget_s, gpu_out=None, err=None):
    """The oracle, as it stands, on a bounded sample of the same workload.
    With gpu_out=(O, LSE) and err, the GPU's rows of each sampled block are
    compared with the oracle's (outside the timed part)."""
    import oracle
    threads = _blas_threads()
    w = st["w"]
    f64 = lambda t: t.float().cpu().double().numpy()
    q, k, v = f64(st["q"]), f64(st["k"]), f64(st["v"])
    rng = np.random.default_rng(0)
    if workload == "video":
        full, part, kv = oracle.expand_kv_blocks(w.cube_mask, w.cube_valid, st["f"], w.kv_tile)
        B, H, M = 1, q.shape[2], len(w.cube_valid)
        bq, bk, mm, kvv = w.cube_elems, w.kv_tile, oracle.MASK_KV_VALID_COUNT, kv
        # the GPU's count: every listed tile at its full size
        row_keys = lambda b, h, i: float((full[b, h, i].sum() + part[b, h, i].sum()) * bk)
    else:
        full, part = w.full, w.part
        B, H, M = full.shape[:3]
        bq, bk, mm, kvv = w.block_q, w.block_kv, w.mask_mod, None
        row_keys = lambda b, h, i: float((full[b, h, i] | part[b, h, i]).sum() * bk)
    D = q.shape[-1]
    flops, n, dt, Sq = 0.0, 0, 0.0, q.shape[1]
    while dt < budget_s:
        b, h, i = int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(M))
        t0 = time.perf_counter()
        O, L = oracle.blocksparse_attention(q, k, v, full, part, bq, bk, mm, w.scale, kvv,
                                            q_blocks=[(b, h, i)])
        dt += time.perf_counter() - t0
        flops += 4.0 * D * bq * row_keys(b, h, i)
        n += 1
        if gpu_out is not None:
            r = slice(i * bq, min((i + 1) * bq, Sq))
            err.note(gpu_out[0][b, r, h], gpu_out[1][b, h, r], O[b, r, h], L[b, h, r])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n} random Q blocks ({bq} rows each) of the same workload, fp64 numpy, "
                      f"{dt:.1f} s wall"}


def _pairs_flops(full, part, bq, bk, Sq, Sk, D):
    """4*D*sum over listed (Q block, KV block) pairs of the clipped block area."""
    import numpy as np
    M, N = full.shape[-2:]
    mext = np.minimum(bq, Sq - np.arange(M) * bq).astype(np.float64)
    next_ = np.minimum(bk, Sk - np.arange(N) * bk).astype(np.float64)
    sel = (full | part).astype(np.float64)
    return 4.0 * D * float((sel * mext[:, None] * next_[None, :]).sum())


def _time_launches(torch, fn, n=20, warm=3, flush=None):
    """Median of n launches, each between its own pair of HIP events.  With
    flush (a device buffer), the buffer is overwritten before every launch,
    outside the events, so no input is left in L2 or the MALL ("cold")."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        if flush is not None:
            flush.fill_(i & 0xFF)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return ms[len(ms) // 2]


def _oracle_rate(fn_blocks, flops_of, budget_s, check):
    """TFLOP/s of the oracle over random Q blocks for about budget_s seconds.
    fn_blocks() -> (pick, (O, LSE)); check(pick, O, LSE) runs untimed."""
    dt, fl = 0.0, 0.0
    while dt < budget_s:
        t0 = time.perf_counter()
        pick, (O, L) = fn_blocks()
        dt += time.perf_counter() - t0
        fl += flops_of(pick)
        check(pick, O, L)
    return fl / dt / 1e12


def table(torch, np, bsa, workloads, oracle_s):
    import oracle
    f64 = lambda t: t.float().cpu().double().numpy()
    dev = torch.device("cuda")
    print("| Workload | GPU ms | GFLOP | TFLOP/s | % bf16 peak | Oracle TFLOP/s (CPU) "
          "| Oracle blocks | max abs err O | O err beyond bf16 rounding | max abs err LSE |")
    print("|---|---|---|---|---|---|---|---|---|---|", flush=True)

    def emit(name, ms, fl, cpu, err):
        tf = fl / (ms * 1e-3) / 1e12
        c = "" if cpu is None else f"{cpu:.4f}"
        e = (" | | | " if err.n == 0 else
             f"{err.n} | {err.o:.2e} | {err.o_excess:.2e} | {err.lse:.2e}")
        print(f"| {name} | {ms:.4f} | {fl / 1e9:.2f} | {tf:.1f} "
              f"| {100 * tf / PEAK_BF16_TFLOPS:.1f} | {c} | {e} |", flush=True)

    def batched(name, w, dtype=torch.bfloat16, oracle_budget=oracle_s):
        q, k, v = (torch.from_numpy(x).to(dtype).to(dev) for x in (w.q, w.k, w.v))
        lists = [bsa.bsa_mask_to_index(torch.from_numpy(m.astype(np.uint8)).to(dev))
                 if m.any() else None for m in (w.part, w.full)]
        kvv = None if w.kv_valid is None else torch.from_numpy(
            np.asarray(w.kv_valid, np.int32)).to(dev)
        o, lse = bsa.bsa_fwd(q, k, v, lists[0], lists[1], w.block_q, w.block_kv, w.mask_mod,
                             kvv, w.scale)
        ms = _time_launches(torch, lambda: bsa.bsa_fwd(q, k, v, lists[0], lists[1], w.block_q,
                                                       w.block_kv, w.mask_mod, kvv, w.scale,
                                                       out=o, lse=lse))
        B, Sq, H, D = w.q.shape
        Sk = w.k.shape[1]
        fl = _pairs_flops(w.full, w.part, w.block_q, w.block_kv, Sq, Sk, D)
        cpu, err = None, _MaxErr()
        if oracle_budget > 0:
            qo, ko, vo = (f64(t.to(torch.bfloat16)) for t in (q, k, v))
            rng = np.random.default_rng(0)
            M = w.full.shape[2]

            def one():
                pick = (int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(M)))
                return pick, oracle.blocksparse_attention(
                    qo, ko, vo, w.full, w.part, w.block_q, w.block_kv, w.mask_mod, w.scale,
                    w.kv_valid, q_blocks=[pick])

            def check(pick, O, L):
                b, h, i = pick
                r = slice(i * w.block_q, min((i + 1) * w.block_q, Sq))
                err.note(o[b, r, h], lse[b, h, r], O[b, r, h], L[b, h, r])

            def fl_of(pick):
                b, h, i = pick
                return _pairs_flops(w.full[b:b + 1, h:h + 1, i:i + 1],
                                    w.part[b:b + 1, h:h + 1, i:i + 1], w.block_q, w.block_kv,
                                    min(w.block_q, Sq - i * w.block_q), Sk, D)
            cpu = _oracle_rate(one, fl_of, oracle_budget, check)
        emit(name, ms, fl, cpu, err)

    batched("tiny fp32 (B1 H1 S256 d64, 64x64, Bernoulli 0.5)", workloads.tiny(),
            dtype=torch.float32)
    batched("causal blocks (B2 H4 S1024 d128, 128x128)", workloads.causal_blocks())
    for D in workloads.SWEEP_HEAD_DIMS:
        for bq, bk in workloads.SWEEP_BLOCKS:
            w = workloads.sparse_sweep(D, bq, bk)
            batched(f"sweep d{D} ({bq},{bk}) (B2 H16 S4096, 25 %)", w,
                    oracle_budget=oracle_s if (D, bq, bk) == (128, 128, 128) else 0)
    # route packing: KV blocks of 16 and 48 keys beside 64 (d128, 128-row Q blocks)
    for bk in (16, 48, 64):
        w = workloads.sparse_sweep(128, 128, bk)
        batched(f"sweep d128 (128,{bk}) (B2 H16 S4096, 25 %; "
                f"{'packed 64-key items' if bk % 64 else 'one block per item'})", w,
                oracle_budget=oracle_s / 4 if bk == 16 else 0)
    # GQA head packing: H 32 over H_kv 4, lists per KV head (shared by 8 Q heads)
    w = workloads.gqa_sweep(128, 128, 128, Hkv=4, hrep=8, B=2, S=4096)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
    B, S, H, D = w.q.shape
    mk, fk = (bsa.bsa_mask_to_index(torch.from_numpy(m.astype(np.uint8)).to(dev))
              for m in (w.part, w.full))
    rep = lambda m: np.repeat(m, H // w.full.shape[1], axis=1)
    mq, fq = (bsa.bsa_mask_to_index(torch.from_numpy(rep(m).astype(np.uint8)).to(dev))
              for m in (w.part, w.full))
    run_pk = lambda **kw: bsa.bsa_fwd(q, k, v, mk, fk, 128, 128, bsa.MASK_CAUSAL, None, w.scale,
                                      kv_head_lists=True, **kw)
    run_un = lambda **kw: bsa.bsa_fwd(q, k, v, mq, fq, 128, 128, bsa.MASK_CAUSAL, None, w.scale,
                                      **kw)
    o1, l1 = run_pk()
    o2, l2 = run_un()
    ms_pk = _time_launches(torch, lambda: run_pk(out=o1, lse=l1))
    ms_un = _time_launches(torch, lambda: run_un(out=o2, lse=l2))
    fl = _pairs_flops(rep(w.full), rep(w.part), 128, 128, S, S, D)
    err = _MaxErr()
    if oracle_s > 0:
        qo, ko, vo = (f64(t) for t in (q, k, v))
        rng = np.random.default_rng(0)
        for _ in range(4):
            b, h, i = int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(S // 128))
            O, L = oracle.blocksparse_attention(qo, ko, vo, rep(w.full), rep(w.part), 128, 128,
                                                bsa.MASK_CAUSAL, w.scale, q_blocks=[(b, h, i)])
            r = slice(i * 128, (i + 1) * 128)
            err.note(o1[b, r, h], l1[b, h, r], O[b, r, h], L[b, h, r])
    tag = f"B{B} H{H} over H_kv {w.full.shape[1]}, S{S} d{D}, 128x128, 25 %"
    emit(f"GQA, lists per KV head, 2 Q heads packed per 256-row workgroup ({tag})", ms_pk, fl,
         None, err)
    emit(f"GQA, the same lists per Q head, unpacked ({tag})", ms_un, fl, None, _MaxErr())
    # backward on the d128 sweep workload: row dots, dQ and dK/dV kernels
    w = workloads.sparse_sweep(128, 128, 128)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
    ml_b = bsa.bsa_mask_to_index(torch.from_numpy(w.part.astype(np.uint8)).to(dev))
    fl_b = bsa.bsa_mask_to_index(torch.from_numpy(w.full.astype(np.uint8)).to(dev))
    o, lse = bsa.bsa_fwd(q, k, v, ml_b, fl_b, 128, 128, bsa.MASK_CAUSAL, None, w.scale)
    g = torch.randn_like(o)
    run_b = lambda: bsa.bsa_bwd(q, k, v, o, lse, g, ml_b, fl_b, 128, 128, bsa.MASK_CAUSAL, None,
                                w.scale)
    run_b()
    ms = _time_launches(torch, run_b)
    B, S, H, D = w.q.shape
    # five products (S, dP, dV, dK, dQ) of 2*D flops per listed (row, key) cell
    fl = 2.5 * _pairs_flops(w.full, w.part, 128, 128, S, S, D)
    emit(f"backward, sweep d{D} (128,128) (B{B} H{H} S{S}, 25 %; includes building the KV-major "
         f"lists; 10*d flops per listed cell)", ms, fl, None, _MaxErr())
    # sliding window: lists from the GPU classifier of the local mask_mod
    w = workloads.sliding_window()
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
    B, S, H, D = w.q.shape
    full_c, part_c = bsa.bsa_block_sparsity(bsa.MASK_LOCAL, S, S, w.block_q, w.block_kv,
                                            window=w.window, device=dev)
    M, N = full_c.shape
    fl_w = bsa.bsa_mask_to_index(full_c.reshape(1, 1, M, N).contiguous())
    ml_w = bsa.bsa_mask_to_index(part_c.reshape(1, 1, M, N).contiguous())
    run_w = lambda **kw: bsa.bsa_fwd(q, k, v, ml_w, fl_w, w.block_q, w.block_kv, bsa.MASK_LOCAL,
                                     None, w.scale, window=w.window, **kw)
    o, lse = run_w()
    ms = _time_launches(torch, lambda: run_w(out=o, lse=lse))
    fc, pc = full_c.cpu().numpy().astype(bool), part_c.cpu().numpy().astype(bool)
    fl = _pairs_flops(np.broadcast_to(fc, (B, H, M, N)), np.broadcast_to(pc, (B, H, M, N)),
                      w.block_q, w.block_kv, S, S, D)
    cpu, err = None, _MaxErr()
    if oracle_s > 0:
        qo, ko, vo = (f64(t) for t in (q, k, v))
        of, op_ = oracle.block_sparsity(oracle.MASK_LOCAL, S, S, w.block_q, w.block_kv,
                                        window=w.window)
        ofb = np.broadcast_to(of.astype(bool), (B, H, M, N))
        opb = np.broadcast_to(op_.astype(bool), (B, H, M, N))
        rng = np.random.default_rng(0)

        def one():
            pick = (int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(M)))
            return pick, oracle.blocksparse_attention(qo, ko, vo, ofb, opb, w.block_q, w.block_kv,
                                                      oracle.MASK_LOCAL, w.scale,
                                                      q_blocks=[pick], window=w.window)

        def check(pick, O, L):
            b, h, i = pick
            r = slice(i * w.block_q, min((i + 1) * w.block_q, S))
            err.note(o[b, r, h], lse[b, h, r], O[b, r, h], L[b, h, r])

        def fl_of(pick):
            b, h, i = pick
            return _pairs_flops(ofb[b:b + 1, h:h + 1, i:i + 1], opb[b:b + 1, h:h + 1, i:i + 1],
                                w.block_q, w.block_kv, min(w.block_q, S - i * w.block_q), S, D)
        cpu = _oracle_rate(one, fl_of, oracle_s, check)
    emit(f"sliding window (B{B} H{H} S{S} d{D}, window {w.window[0]} back, 128x128, "
         f"{100 * fl / (4.0 * D * B * H * S * S):.1f} %)", ms, fl, cpu, err)
    # proxy-compensated routes: the page's proxy workload, exact-only and with proxies
    w = workloads.proxy_routes()
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
    B, S, H, D = w.q.shape
    bk = w.block_kv
    M, N = w.full.shape[2:]
    fl_p = bsa.bsa_mask_to_index(torch.from_numpy(w.full.astype(np.uint8)).to(dev))
    # summaries (inputs, built outside the timed region): mean K and summed V per block
    pad = N * bk - S
    kp_ = torch.nn.functional.pad(k.float(), (0, 0, 0, 0, 0, pad)).reshape(B, N, bk, H, D)
    vp_ = torch.nn.functional.pad(v.float(), (0, 0, 0, 0, 0, pad)).reshape(B, N, bk, H, D)
    cnt = torch.clamp(S - torch.arange(N, device=dev) * bk, max=bk).float().reshape(1, N, 1, 1)
    ks = (kp_.sum(2) / cnt).to(torch.bfloat16).contiguous()
    vs = vp_.sum(2).to(torch.bfloat16).contiguous()
    run_e = lambda **kw: bsa.bsa_fwd(q, k, v, None, fl_p, w.block_q, bk, bsa.MASK_NONE, None,
                                     w.scale, **kw)
    run_p = lambda **kw: bsa.bsa_fwd(q, k, v, None, fl_p, w.block_q, bk, bsa.MASK_NONE, None,
                                     w.scale, proxy=(ks, vs), **kw)
    oe, le = run_e()
    op, lp = run_p()
    ms_e = _time_launches(torch, lambda: run_e(out=oe, lse=le))
    ms_p = _time_launches(torch, lambda: run_p(out=op, lse=lp))
    fl = _pairs_flops(w.full, w.part, w.block_q, bk, S, S, D)
    cpu, err = None, _MaxErr()
    if oracle_s > 0:
        qo, ko, vo, kso, vso = (f64(t) for t in (q, k, v, ks, vs))
        rng = np.random.default_rng(0)

        def one():
            pick = (int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(M)))
            return pick, oracle.proxy_attention(qo, ko, vo, w.full, w.part, kso, vso, w.block_q,
                                                bk, w.scale, q_blocks=[pick])

        def check(pick, O, L):
            b, h, i = pick
            r = slice(i * w.block_q, min((i + 1) * w.block_q, S))
            err.note(op[b, r, h], lp[b, h, r], O[b, r, h], L[b, h, r])

        def fl_of(pick):
            b, h, i = pick
            return _pairs_flops(w.full[b:b + 1, h:h + 1, i:i + 1], w.part[b:b + 1, h:h + 1, i:i + 1],
                                w.block_q, bk, min(w.block_q, S - i * w.block_q), S, D)
        cpu = _oracle_rate(one, fl_of, oracle_s, check)
    tag = f"B{B} S{S} H{H} d{D}, 64x64, 84 of {N} blocks per row"
    emit(f"proxy workload, exact blocks only ({tag})", ms_e, fl, None, _MaxErr())
    emit(f"proxy-compensated ({tag}; TFLOP/s over exact-block FLOPs; "
         f"+{100 * (ms_p / ms_e - 1):.1f} % time over exact only)", ms_p, fl, cpu, err)
    # their backward: the exact-only one, and the route's (keys, then one summary key per block)
    g = torch.randn_like(op)
    run_be = lambda: bsa.bsa_bwd(q, k, v, oe, le, g, None, fl_p, w.block_q, bk, bsa.MASK_NONE,
                                 None, w.scale)
    run_bp = lambda: bsa.bsa_bwd(q, k, v, op, lp, g, None, fl_p, w.block_q, bk, bsa.MASK_NONE,
                                 None, w.scale, proxy=(ks, vs))
    run_be()
    run_bp()
    ms_be = _time_launches(torch, run_be, n=5)
    ms_bp = _time_launches(torch, run_bp, n=5)
    emit(f"backward, proxy workload, exact blocks only ({tag}; 10*d flops per listed cell)",
         ms_be, 2.5 * fl, None, _MaxErr())
    emit(f"backward, proxy-compensated ({tag}; over the exact blocks' 10*d flops; one summary "
         f"key per omitted block: {ms_bp / ms_be:.2f}x the exact-only time)", ms_bp,
         2.5 * fl, None, _MaxErr())
    # varlen packed
    w = workloads.varlen_packed()
    H, bq, bk = w.q.shape[1], w.block_q, w.block_kv
    cu, off, tm, tn = bsa.bsa_varlen_offsets(w.seqlens_q, w.seqlens_k, bq, bk)
    dv = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    cu_q, cu_k = dv([0] + list(np.cumsum(w.seqlens_q))), dv([0] + list(np.cumsum(w.seqlens_k)))
    cu_m, offs = dv(cu), dv(off)

    def packed(masks):
        out = np.zeros((H, tn), np.uint8)
        for b, m in enumerate(masks):
            nm, nn = m.shape[1:]
            for i in range(nm):
                out[:, off[b] + i * nn: off[b] + (i + 1) * nn] = m[:, i]
        return torch.from_numpy(out).to(dev)

    ml = bsa.bsa_varlen_mask_to_index(packed(w.part), cu_m, offs, tm, tn)
    fl_ = bsa.bsa_varlen_mask_to_index(packed(w.full), cu_m, offs, tm, tn)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
    o, lse = bsa.bsa_varlen_fwd(q, k, v, cu_q, cu_k, cu_m, offs, tm, tn, ml, fl_, bq, bk,
                                w.mask_mod, w.scale)
    ms = _time_launches(torch, lambda: bsa.bsa_varlen_fwd(q, k, v, cu_q, cu_k, cu_m, offs, tm, tn,
                                                          ml, fl_, bq, bk, w.mask_mod, w.scale,
                                                          out=o, lse=lse))
    D = w.q.shape[-1]
    fl = sum(_pairs_flops(fu[None], pa[None], bq, bk, sq, sk, D)
             for fu, pa, sq, sk in zip(w.full, w.part, w.seqlens_q, w.seqlens_k))
    cpu, err = None, _MaxErr()
    if oracle_s > 0:
        qo, ko, vo = (f64(t) for t in (q, k, v))
        rng = np.random.default_rng(0)
        cq = np.concatenate([[0], np.cumsum(w.seqlens_q)])

        def one():
            b = int(rng.integers(len(w.seqlens_q)))
            i = int(rng.integers(-(-w.seqlens_q[b] // bq)))
            h = int(rng.integers(H))
            return (b, h, i), oracle.varlen_blocksparse_attention(
                qo, ko, vo, w.seqlens_q, w.seqlens_k, w.full, w.part, bq, bk, w.mask_mod,
                w.scale, q_blocks=[(b, h, i)])

        def check(pick, O, L):
            b, h, i = pick
            r = slice(int(cq[b]) + i * bq, int(cq[b]) + min((i + 1) * bq, w.seqlens_q[b]))
            err.note(o[r, h], lse[h, r], O[r, h], L[h, r])

        def fl_of(pick):
            b, h, i = pick
            sq, sk = w.seqlens_q[b], w.seqlens_k[b]
            return _pairs_flops(w.full[b][None, h:h + 1, i:i + 1], w.part[b][None, h:h + 1, i:i + 1],
                                bq, bk, min(bq, sq - i * bq), sk, D)
        cpu = _oracle_rate(one, fl_of, oracle_s, check)
    emit(f"varlen packed (8 seqs, {sum(w.seqlens_q)} tokens, H16 d128, 128x128)", ms, fl, cpu,
         err)
    # backward of the same packed batch (KV-block prefix from the offsets with roles swapped)
    cu_kv, _, tkv, _ = bsa.bsa_varlen_offsets(w.seqlens_k, w.seqlens_q, bk, bq)
    g = torch.randn_like(o)
    run_vb = lambda: bsa.bsa_varlen_bwd(q, k, v, o, lse, g, cu_q, cu_k, cu_m, dv(cu_kv), offs,
                                        tm, tkv, tn, ml, fl_, bq, bk, w.mask_mod,
                                        softmax_scale=w.scale)
    run_vb()
    ms = _time_launches(torch, run_vb)
    emit(f"backward, varlen packed (8 seqs, {sum(w.seqlens_q)} tokens, H16 d128, 128x128; "
         f"includes building the KV-major lists; 10*d flops per listed cell)", ms, 2.5 * fl,
         None, _MaxErr())
    # video (forward only; the step's metadata kernels add < 1 %)
    st, flops, _ = _video_inputs(torch, np, workloads)
    wv = st["w"]
    full, part, kvv = bsa.bsa_expand_kv_blocks(st["cube_mask"], st["cube_valid"], st["f"],
                                               wv.kv_tile)
    mlv, flv = bsa.bsa_mask_to_index(part), bsa.bsa_mask_to_index(full)
    o, lse = bsa.bsa_fwd(st["q"], st["k"], st["v"], mlv, flv, wv.cube_elems, wv.kv_tile,
                         bsa.MASK_KV_VALID_COUNT, kvv, wv.scale)
    ms = _time_launches(torch, lambda: bsa.bsa_fwd(st["q"], st["k"], st["v"], mlv, flv,
                                                   wv.cube_elems, wv.kv_tile,
                                                   bsa.MASK_KV_VALID_COUNT, kvv, wv.scale,
                                                   out=o, lse=lse))
    # cold: a 1 GiB buffer (four times the 256 MB MALL) written before each launch
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ms_cold = _time_launches(torch, lambda: bsa.bsa_fwd(st["q"], st["k"], st["v"], mlv, flv,
                                                        wv.cube_elems, wv.kv_tile,
                                                        bsa.MASK_KV_VALID_COUNT, kvv, wv.scale,
                                                        out=o, lse=lse), n=10, flush=flush)
    del flush
    err = _MaxErr()
    cpu = (_cpu_baseline(np, st, "video", oracle_s, gpu_out=(o, lse), err=err)["value"]
           if oracle_s > 0 else None)
    emit("video (B1 H24 86016 rows d128, 256x128, 11.9 %)", ms, flops, cpu, err)
    emit("video, cold (1 GiB written before each launch)", ms_cold, flops, None, _MaxErr())


def _set_blas_threads():
    # before numpy is imported: the host's OMP_NUM_THREADS if it sets one,
    # else every CPU this process may run on
    n = os.environ.get("OMP_NUM_THREADS") or str(len(os.sched_getaffinity(0)))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, n)


def main():
    args = _parse()
    _set_blas_threads()
    if args.print_kernel_hash:
        print(_kernel_hash())
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this block-sparse forward runs on one GPU "
              "per process; sharding batch and heads across GPUs needs no change to the "
              "kernels.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_attention_bsa_amd as bsa
    import workloads

    bsa.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.table:
        table(torch, np, bsa, workloads, args.cpu_seconds / 3.0)
        return
    if args.calibrate_copy:
        n = 1 << 30
        x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "launches": 3}))
        return
    make, step = {"video": (_video_inputs, _video_step), "sweep128": (_sweep_inputs, _sweep_step),
                  "varlen": (_varlen_inputs, _varlen_step),
                  "bwd_sweep128": (_bwd_inputs, _bwd_step)}[args.workload]
    st, flops, cfg = make(torch, np, workloads)
    for _ in range(args.warmup):
        step(bsa, st)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(bsa, st, evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    fwd_ms = [a.elapsed_time(b) for a, b in evs]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (fwd_avg * 1e-3) / 1e12
    video = args.workload == "video"
    traffic = _from_profile("hbm_bytes_per_launch") if video else None
    # GPU-active cycles per launch (per XCD) from the committed counter run of
    # this kernel revision: the cycle count does not move with the clock, so
    # over the live kernel time it gives the shader clock of this run
    cycles = _from_profile("active_cycles_per_launch_per_xcd") if video else None
    # head_dim 128; 256-row workgroups for 256-token Q cubes, 128 rows otherwise
    kernel_name = "bsa_fwd_pp_kernel<128> (256-row workgroup, 8 waves)" \
        if args.workload == "video" else "bsa_fwd_kernel<128,4> (128-row workgroup)"
    metric = METRIC
    if args.workload == "bwd_sweep128":
        kernel_name = "backward: KV-major lists, bwd_rowdot, bwd_dq_kernel<128,4>, bwd_dkdv_kernel<128,4>"
        metric = "effective TFLOP/s bf16 block-sparse attn bwd (10*d flops per listed cell)"
    if args.workload in ("varlen", "bwd_sweep128"):
        args.cpu_seconds = 0  # the oracle leg samples the video and sweep workloads only
    out = {
        "metric": metric, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded top-k block selection)",
        "config": cfg,
        "pct_of_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": kernel_name,
                     "kernel_ms": round(fwd_avg, 4), "flops_per_launch": flops,
                     # achieved against the peak scaled to the clock of this run
                     "measured_sclk_mhz": None, "frac_at_measured_clock": None},
    }
    if cycles:
        sclk = cycles / (fwd_avg * 1e-3) / 1e6
        out["roofline"]["measured_sclk_mhz"] = round(sclk, 1)
        out["roofline"]["frac_at_measured_clock"] = round(
            achieved / (PEAK_BF16_TFLOPS * sclk / PEAK_SCLK_MHZ), 4)
    if video:
        out["flops_valid_keys_per_launch"] = st["flops_valid_keys"]
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = _cpu_baseline(np, st, args.workload, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
