"""The forward kernels issue their K/V DMA (global_load_lds / buffer_load
... lds) from inline assembly, which the compiler's hazard checks do not see
into.  A vector-memory instruction needs five wait states after a VALU
instruction writes an SGPR it reads (on this chip family a base address or
buffer descriptor restored from a spill with v_readlane); with fewer it can
read a stale address.  This compiles the forward and backward DMA kernels' sources for gfx950
with the library's flags and checks every DMA in the assembly: no VALU write
of its base SGPRs within the five wait states before it (an s_nop N counts
N + 1).  CPU only; needs hipcc."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_bsa_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


def _asm(src, out):
    cmd = [HIPCC, "-O3", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read().splitlines()


def _sgprs(op):
    m = re.match(r"s\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", op)
    return {int(m.group(1))} if m else set()


def _hazards(lines):
    """(DMA sites, [(kernel, line) with a VALU-written base SGPR too close])."""
    kern, bad, sites = None, [], 0
    for i, line in enumerate(lines):
        if re.match(r"^_Z\w+:", line):
            kern = line.split(":")[0]
        m = re.search(r"(global_load_lds_dwordx4|buffer_load_dwordx4)\s+v\d+,\s*(s\[\d+:\d+\])",
                      line)
        if not m or (m.group(1) == "buffer_load_dwordx4" and " lds" not in line):
            continue
        sites += 1
        regs, waits, j = _sgprs(m.group(2)), 0, i - 1
        while j >= 0 and waits < 5:
            t = lines[j].strip()
            j -= 1
            if not t or t[0] in ";./" or t.startswith(";;"):
                continue
            n = re.match(r"s_nop\s+(\d+)", t)
            if n:
                waits += int(n.group(1)) + 1
                continue
            parts = t.split()
            if t.startswith("v_") and len(parts) > 1 and _sgprs(parts[1].rstrip(",")) & regs:
                bad.append((kern, i + 1))
                break
            waits += 1
    return sites, bad


def test_scanner_finds_a_planted_hazard():
    planted = ["_Zk:", "\tv_readlane_b32 s9, v255, 1", "\ts_nop 0",
               "\tglobal_load_lds_dwordx4 v100, s[8:9]", "_Zj:", "\tv_readlane_b32 s9, v255, 1",
               "\ts_nop 4", "\tglobal_load_lds_dwordx4 v100, s[8:9]"]
    sites, bad = _hazards(planted)
    assert sites == 2 and bad == [("_Zk", 4)]


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_dma_base_sgprs_are_stable(tmp_path):
    srcs = ["bsa_fwd.hip", "bsa_fwd_pp.hip", "bsa_bwd.hip"]
    with ThreadPoolExecutor(3) as ex:
        asms = list(ex.map(lambda s: _asm(s, str(tmp_path / (s + ".s"))), srcs))
    for src, lines in zip(srcs, asms):
        sites, bad = _hazards(lines)
        assert sites > 0, src
        assert not bad, f"{src}: {len(bad)} of {sites} DMAs too close to a VALU SGPR write: {bad[:3]}"
