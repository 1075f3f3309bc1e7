"""Host-side logic of bench.py (no GPU): the one-GPU contract, the FLOP count
of listed block pairs, and profile figures that are only used while the
kernel they were measured on is unchanged."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("seed,bq,bk,Sq,Sk,D", [(0, 64, 64, 256, 256, 64),
                                                (1, 128, 112, 300, 500, 128),
                                                (2, 64, 128, 1, 129, 96)])
def test_pair_flops_brute_force(seed, bq, bk, Sq, Sk, D):
    """4*D times the number of (row, key) cells inside listed blocks, counted
    cell by cell: rows past Sq and keys past Sk are not in any block."""
    rng = np.random.default_rng(seed)
    M, N = -(-Sq // bq), -(-Sk // bk)
    full = rng.random((1, 1, M, N)) < 0.4
    part = (rng.random((1, 1, M, N)) < 0.3) & ~full
    cells = 0
    for r in range(Sq):
        for c in range(Sk):
            i, j = r // bq, c // bk
            cells += int(full[0, 0, i, j] or part[0, 0, i, j])
    assert bench._pairs_flops(full, part, bq, bk, Sq, Sk, D) == 4.0 * D * cells


def test_profile_figures_follow_the_kernel_hash(tmp_path, monkeypatch):
    h = bench._kernel_hash()
    good = tmp_path / "good.md"
    good.write_text(f"kernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 1.25e9\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(good))
    assert bench._from_profile("hbm_bytes_per_launch") == 1.25e9
    assert bench._from_profile("active_cycles_per_launch_per_xcd") is None
    stale = tmp_path / "stale.md"
    other = "0" * 16 if h != "0" * 16 else "1" * 16
    stale.write_text(f"kernel_source_sha256_16: {other}\nhbm_bytes_per_launch: 1.25e9\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(stale))
    assert bench._from_profile("hbm_bytes_per_launch") is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench._from_profile("hbm_bytes_per_launch") is None

