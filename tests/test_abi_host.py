"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function include/bsa.h declares, and its pure-host bookkeeping matches
the oracle bit-exactly."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import block_sparse_attention_bsa_amd as bsa
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "bsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:bsa_status|const char\*)\s+(bsa_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert names == sorted(["bsa_fwd", "bsa_varlen_fwd", "bsa_mask_to_index",
                            "bsa_varlen_mask_to_index", "bsa_varlen_offsets",
                            "bsa_expand_kv_blocks", "bsa_block_sparsity", "bsa_bitmask_to_index",
                            "bsa_kv_major_lists", "bsa_bwd", "bsa_bwd_noalloc", "bsa_bwd_f32",
                            "bsa_bwd_proxy", "bsa_bwd_proxy_work_size",
                            "bsa_varlen_bwd", "bsa_varlen_kv_major_lists", "bsa_status_str"])
    lib = bsa.load_library()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", bsa.library_path()], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\sT\s+(bsa_\w+)", out))
    assert set(names) <= exported


def test_status_strings():
    assert bsa.bsa_status_str(0) == "ok"
    assert "misaligned" in bsa.bsa_status_str(3)
    assert bsa.bsa_status_str(99) == "unknown status"


@pytest.mark.parametrize("seed", range(6))
def test_varlen_offsets_match_oracle(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(0, 12))
    sq = [int(x) for x in rng.integers(0, 20000, B)]
    sk = [int(x) for x in rng.integers(0, 20000, B)]
    bq, bk = int(rng.choice([32, 64, 128, 256])), int(rng.choice([16, 48, 64, 112, 128]))
    assert bsa.bsa_varlen_offsets(sq, sk, bq, bk) == tuple(oracle.varlen_offsets(sq, sk, bq, bk))


def test_varlen_offsets_errors():
    with pytest.raises(ValueError):
        bsa.bsa_varlen_offsets([5, -1], [5, 5], 64, 64)
    with pytest.raises(ValueError):
        bsa.bsa_varlen_offsets([5], [5], 0, 64)
    with pytest.raises(ValueError):  # int32 overflow of the packed slot count
        bsa.bsa_varlen_offsets([2 ** 30], [2 ** 30], 32, 32)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(bsa, "_lib", None)
    monkeypatch.setattr(bsa, "_LIB_PATH", "/nonexistent/libbsa.so")
    with pytest.raises(RuntimeError):
        bsa.load_library()


def test_product_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "block_sparse_attention_bsa_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


def test_varlen_backward_argument_errors_on_the_host():
    # Rejected before any device work: negative sizes, H not a multiple of
    # H_kv, a negative kv_valid row stride; an empty pack is a no-op.
    lib = bsa.load_library()
    z = [None] * 9
    i64 = (ctypes.c_int64 * 2)(8, 8)
    bs = bsa._BlockSparse(bsa._BlockList(), bsa._BlockList(), 64, 64, -1, -1)
    lt = bsa._BlockList()

    def call(B, H, Hkv, tm, tkv, ld):
        return lib.bsa_varlen_bwd(*z, B, H, Hkv, 128, None, None, None, None, None, tm, tkv, 0,
                                  i64, i64, i64, i64, ctypes.byref(bs), ctypes.byref(lt),
                                  ctypes.byref(lt), 0, None, ld, 0.1, None, None)
    assert call(-1, 2, 2, 1, 1, 0) == 1
    assert call(1, 3, 2, 1, 1, 0) == 1
    assert call(1, 2, 2, 1, 1, -1) == 1
    assert call(1, 2, 2, -1, 1, 0) == 1
    assert call(0, 2, 2, 0, 0, 0) == 0
    assert lib.bsa_varlen_kv_major_lists(None, None, -1, 1, None, None, None, 0, 0, 0, None, None,
                                         None, None) == 1
    assert lib.bsa_varlen_kv_major_lists(None, None, 2, 1, None, None, None, 0, 0, 0, None, None,
                                         None, None) == 0


def test_fp32_backward_argument_errors_on_the_host():
    # Rejected before any device work: negative sizes, H not a multiple of
    # H_kv, an unsupported head_dim, strides that break 16-byte rows; an
    # empty problem is a no-op.
    lib = bsa.load_library()
    z = [None] * 9
    good = (ctypes.c_int64 * 3)(1024, 64, 64)
    odd = (ctypes.c_int64 * 3)(1024, 66, 66)
    bs = bsa._BlockSparse(bsa._BlockList(), bsa._BlockList(), 64, 64, -1, -1)
    lt = bsa._BlockList()
    buf = ctypes.create_string_buffer(64 + 16)
    p16 = (ctypes.addressof(buf) + 15) // 16 * 16  # host memory, never dereferenced

    def call(B, H, Hkv, Sq, Sk, D, st=good, ptrs=None):
        return lib.bsa_bwd_f32(*(ptrs or z), B, H, Hkv, Sq, Sk, D, st, st, st, st,
                               ctypes.byref(bs), ctypes.byref(lt), ctypes.byref(lt), 0, None,
                               0.1, ptrs[0] if ptrs else None, None)
    assert call(-1, 2, 2, 8, 8, 64) == 1
    assert call(1, 3, 2, 8, 8, 64) == 1
    assert call(1, 2, 2, 8, 8, 80) == 2
    assert call(0, 2, 2, 8, 8, 64) == 0
    assert call(1, 2, 2, 8, 8, 64) == 1  # missing pointers
    assert call(1, 2, 2, 8, 8, 64, odd, [p16] * 9) == 3
    # a list with counts but no ids: rejected by the bf16 backward's checks,
    # which run before the fp32 tensors are staged (nothing is launched)
    bad = bsa._BlockList()
    bad.cnt = p16
    bs.mask = bad
    assert call(1, 2, 2, 8, 8, 64, good, [p16] * 9) == 1


def test_proxy_backward_argument_errors_on_the_host():
    # Rejected before any device work: bad sizes, no summaries, an
    # unsupported head_dim, misaligned strides; the workspace size query.
    lib = bsa.load_library()
    z = [None] * 11
    st = (ctypes.c_int64 * 3)(1024, 64, 64)
    bs = bsa._BlockSparse(bsa._BlockList(), bsa._BlockList(), 64, 64, -1, -1)

    def call(B, H, Hkv, D, ptrs=None):
        return lib.bsa_bwd_proxy(*(ptrs or z), B, H, Hkv, 8, 8, D, st, st, st, st,
                                 ctypes.byref(bs), 0.1, None, None)
    assert call(-1, 2, 2, 64) == 1
    assert call(1, 3, 2, 64) == 1
    assert call(1, 2, 2, 64) == 1  # no summaries
    buf = ctypes.create_string_buffer(64 + 16)
    p16 = (ctypes.addressof(buf) + 15) // 16 * 16  # host memory, never dereferenced
    bs.proxy_k = bs.proxy_v = p16
    assert call(1, 2, 2, 80) == 2
    assert call(1, 2, 2, 64) == 1  # missing tensors
    nbytes = ctypes.c_int64()
    assert lib.bsa_bwd_proxy_work_size(2, 4, 2, 300, 333, 128, 128, 48, ctypes.byref(nbytes)) == 0
    # Sk 333 = 6 full 48-key blocks and one of 45: the six summaries in one
    # chunk, the partial block's in a chunk of its own, so 7 + 2 KV blocks
    NX, M = 9, 3
    xb = 2 * NX * 48 * 2 * 128 * 2  # B * NX*bk * Hkv * D * 2 bytes, K and V
    assert nbytes.value >= 2 * xb + 2 * 4 * M * NX * 4
    assert lib.bsa_bwd_proxy_work_size(2, 4, 2, 300, 333, 128, 0, 48, ctypes.byref(nbytes)) == 1
