"""Block-sparse attention forward on AMD Instinct MI355X (gfx950).

Thin ctypes binding over libbsa.so (include/bsa.h).  The functions here only
marshal torch tensors into pointers, sizes and strides and raise on a bad
status; every step of the computation runs in the HIP kernels.  PyTorch
supplies device memory and the current stream.  If libbsa.so has not been
built, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "MASK_NONE", "MASK_CAUSAL", "MASK_KV_VALID_COUNT", "MASK_LOCAL", "BsaError",
    "bsa_fwd", "bsa_varlen_fwd", "bsa_mask_to_index", "bsa_bitmask_to_index", "bsa_kv_major_lists",
    "bsa_bwd", "bsa_bwd_noalloc", "bsa_varlen_bwd", "bsa_varlen_kv_major_lists",
    "bsa_varlen_mask_to_index",
    "bsa_varlen_offsets", "bsa_expand_kv_blocks", "bsa_block_sparsity", "bsa_status_str",
    "library_path", "load_library",
]

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KV_VALID_COUNT = 2
MASK_LOCAL = 3
FLAG_VALIDATE = 1
FLAG_KV_HEAD_LISTS = 2

BSA_OK = 0
BSA_ERR_INVALID_ARGUMENT = 1
BSA_ERR_UNSUPPORTED = 2
BSA_ERR_MISALIGNED = 3
BSA_ERR_METADATA = 4
BSA_ERR_HIP = 5

_DTYPES = {torch.bfloat16: 0, torch.float32: 1}

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsa.so")
_lib = None


class BsaError(RuntimeError):
    """A libbsa call returned a non-zero status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class BsaValueError(BsaError, ValueError):
    """Invalid, unsupported or misaligned arguments, or bad metadata."""


class _BlockList(ctypes.Structure):
    _fields_ = [("cnt", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("cnt_stride", ctypes.c_int64 * 3), ("idx_stride", ctypes.c_int64 * 4)]


class _BlockSparse(ctypes.Structure):
    _fields_ = [("mask", _BlockList), ("full", _BlockList),
                ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32),
                ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
                ("proxy_k", ctypes.c_void_p), ("proxy_v", ctypes.c_void_p),
                ("proxy_k_str", ctypes.c_int64 * 3), ("proxy_v_str", ctypes.c_int64 * 3)]


def _window(mask_mod: int, window) -> Tuple[int, int]:
    if mask_mod != MASK_LOCAL:
        return -1, -1
    if window is None or len(window) != 2:
        raise ValueError("MASK_LOCAL needs window=(left, right) (a negative bound is unbounded)")
    return int(window[0]), int(window[1])


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libbsa.so (once).  Raises RuntimeError if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_attention_bsa_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)
    F32, U32 = ctypes.c_float, ctypes.c_uint32
    BS = ctypes.POINTER(_BlockSparse)
    lib.bsa_fwd.argtypes = [P, P, P, P, P, ctypes.c_int, I32, I32, I32, I32, I32, I32,
                            I64P, I64P, I64P, I64P, BS, ctypes.c_int, P, F32, U32, P]
    lib.bsa_varlen_fwd.argtypes = [P, P, P, P, P, ctypes.c_int, I32, I32, I32, I32,
                                   P, P, P, P, I32, I32, I32, I64P, I64P, I64P, I64P, BS,
                                   ctypes.c_int, P, ctypes.c_int64, F32, U32, P]
    lib.bsa_mask_to_index.argtypes = [P, I32, I32, I32, I32, P, P, P]
    lib.bsa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                            P, P, P, P, P, P, P, ctypes.c_int, P, ctypes.c_float, P, P]
    lib.bsa_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                    P, P, P, P, P, P, P, ctypes.c_int, P, ctypes.c_float, P]
    lib.bsa_bwd_f32.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                P, P, P, P, P, P, P, ctypes.c_int, P, ctypes.c_float, P, P]
    lib.bsa_bwd_proxy_work_size.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, P]
    lib.bsa_bwd_proxy.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                  P, P, P, P, P, ctypes.c_float, P, P]
    lib.bsa_kv_major_lists.argtypes = [P, P, I32, I32, I32, I32, P, P, P, P]
    lib.bsa_varlen_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32,
                                   P, P, P, P, P, I32, I32, I32, P, P, P, P, P, P, P,
                                   ctypes.c_int, P, ctypes.c_int64, ctypes.c_float, P, P]
    lib.bsa_varlen_kv_major_lists.argtypes = [P, P, I32, I32, P, P, P, I32, I32, I32, P, P, P, P]
    lib.bsa_bitmask_to_index.argtypes = [P, I32, I32, I32, I32, I32, P, P, P]
    lib.bsa_varlen_mask_to_index.argtypes = [P, I32, I32, P, P, I32, I32, P, P, P]
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.bsa_varlen_offsets.argtypes = [I32P, I32P, I32, I32, I32, I32P, I32P, I32P, I32P]
    lib.bsa_expand_kv_blocks.argtypes = [P, P, I32, I32, I32, I32, P, P, P, P]
    lib.bsa_block_sparsity.argtypes = [ctypes.c_int, I32, I32, P, I32, I32, I32, I32, P, P, P]
    lib.bsa_status_str.argtypes = [ctypes.c_int]
    lib.bsa_status_str.restype = ctypes.c_char_p
    for fn in ("bsa_fwd", "bsa_varlen_fwd", "bsa_mask_to_index", "bsa_varlen_mask_to_index",
               "bsa_bwd", "bsa_bwd_noalloc", "bsa_bwd_f32", "bsa_bwd_proxy",
               "bsa_bwd_proxy_work_size", "bsa_kv_major_lists",
               "bsa_bitmask_to_index",
               "bsa_varlen_bwd", "bsa_varlen_kv_major_lists",
               "bsa_varlen_offsets", "bsa_expand_kv_blocks", "bsa_block_sparsity"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def bsa_status_str(status: int) -> str:
    return load_library().bsa_status_str(status).decode()


def _check(fn: str, status: int):
    if status != BSA_OK:
        msg = bsa_status_str(status)
        if status in (BSA_ERR_INVALID_ARGUMENT, BSA_ERR_UNSUPPORTED, BSA_ERR_MISALIGNED,
                      BSA_ERR_METADATA):
            raise BsaValueError(fn, status, msg)
        raise BsaError(fn, status, msg)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _i64(vals: Sequence[int]):
    return (ctypes.c_int64 * len(vals))(*[int(x) for x in vals])


def _dev(name: str, t: torch.Tensor, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _block_list(lst, batched: bool, shape) -> _BlockList:
    """shape: batched (B, H, M, N); varlen (H, total_m, total_n)."""
    L = _BlockList()
    if lst is None:
        return L
    cnt, idx = lst
    _dev("cnt", cnt, torch.int32)
    _dev("idx", idx, torch.int32)
    L.cnt, L.idx = cnt.data_ptr(), idx.data_ptr()
    if batched:
        B, H, M, N = shape
        if cnt.dim() != 3 or idx.dim() != 4:
            raise ValueError("batched block lists must be cnt [B,H,M] and idx [B,H,M,N]")
        if cnt.shape[0] not in (1, B) or cnt.shape[1] not in (1, H) or cnt.shape[2] != M or \
                idx.shape[0] not in (1, B) or idx.shape[1] not in (1, H) or idx.shape[2] != M or \
                idx.shape[3] < N:
            raise ValueError(f"block lists must be cnt [B|1,H|1,{M}] and idx [B|1,H|1,{M},>={N}]"
                             f"; got {tuple(cnt.shape)} and {tuple(idx.shape)}")
        cs, is_ = cnt.stride(), idx.stride()
        L.cnt_stride[:] = [cs[0] if cnt.shape[0] > 1 else 0, cs[1] if cnt.shape[1] > 1 else 0, cs[2]]
        L.idx_stride[:] = [is_[0] if idx.shape[0] > 1 else 0, is_[1] if idx.shape[1] > 1 else 0,
                           is_[2], is_[3]]
    else:
        H, tm, tn = shape
        if cnt.dim() != 2 or idx.dim() != 2:
            raise ValueError("varlen block lists must be cnt [H,total_m] and idx [H,total_n]")
        if cnt.shape[0] not in (1, H) or cnt.shape[1] != tm or idx.shape[0] not in (1, H) or \
                idx.shape[1] != tn:
            raise ValueError(f"varlen block lists must be cnt [H,{tm}] and idx [H,{tn}]")
        L.cnt_stride[:] = [0, cnt.stride(0) if cnt.shape[0] > 1 else 0, cnt.stride(1)]
        L.idx_stride[:] = [0, idx.stride(0) if idx.shape[0] > 1 else 0, 0, idx.stride(1)]
    return L


def bsa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            mask_list: Optional[Tuple[torch.Tensor, torch.Tensor]],
            full_list: Optional[Tuple[torch.Tensor, torch.Tensor]],
            block_q: int, block_kv: int, mask_mod: int = MASK_NONE,
            kv_valid: Optional[torch.Tensor] = None, softmax_scale: Optional[float] = None,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            validate: bool = False, window: Optional[Tuple[int, int]] = None,
            proxy: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
            kv_head_lists: bool = False):
    """Batched block-sparse attention forward.

    q [B,Sq,H,D], k/v [B,Sk,Hkv,D] (bf16 or fp32, head_dim contiguous, any
    other strides, e.g. BSHD or a BHSD tensor permuted to this view).
    mask_list / full_list: (cnt int32 [B|1,H|1,M], idx int32 [B|1,H|1,M,N])
    with M = ceil(Sq/block_q), N = ceil(Sk/block_kv); a size-1 batch or head
    dimension broadcasts.  kv_head_lists=True: the lists' head dimension is
    the KV head (Hkv|1), shared by that KV head's Q heads, which the forward
    then packs into one workgroup.  window=(left, right): the bounds of MASK_LOCAL.
    proxy=(k_mean, v_sum): bf16 [B,N,Hkv,D] block summaries for the
    proxy-compensated route (MASK_NONE only): every block a row does not list
    enters its softmax once, weighted by the block's token count.
    Returns (O [B,Sq,H,D], LSE float32 [B,H,Sq]).
    """
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev(n, t)
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{n} must be 4-D with a contiguous last dimension")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bfloat16 or float32")
    B, Sq, H, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B,Sk,Hkv,D] matching q")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _dev("out", out, q.dtype)
    _dev("lse", lse, torch.float32)
    if tuple(out.shape) != (B, Sq, H, D) or out.stride(-1) != 1:
        raise ValueError("out must be [B,Sq,H,D] with a contiguous last dimension")
    if tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,Sq] tensor")
    if block_q <= 0 or block_kv <= 0:
        raise ValueError("block sizes must be positive")
    M, N = -(-Sq // block_q), -(-Sk // block_kv)
    if kv_valid is not None:
        _dev("kv_valid", kv_valid, torch.int32)
        if not kv_valid.is_contiguous() or kv_valid.numel() < N:
            raise ValueError(f"kv_valid must be a contiguous int32 tensor with {N} entries")
    Hl = Hkv if kv_head_lists else H
    bs = _BlockSparse(_block_list(mask_list, True, (B, Hl, M, N)),
                      _block_list(full_list, True, (B, Hl, M, N)), int(block_q), int(block_kv),
                      *_window(mask_mod, window))
    if proxy is not None:
        for n, t in zip(("proxy k_mean", "proxy v_sum"), proxy):
            _dev(n, t, q.dtype)
            if tuple(t.shape) != (B, N, Hkv, D) or t.stride(-1) != 1:
                raise ValueError(f"{n} must be [B,N,Hkv,D]={(B, N, Hkv, D)} with a contiguous "
                                 "last dimension")
        bs.proxy_k, bs.proxy_v = proxy[0].data_ptr(), proxy[1].data_ptr()
        bs.proxy_k_str = (ctypes.c_int64 * 3)(*proxy[0].stride()[:3])
        bs.proxy_v_str = (ctypes.c_int64 * 3)(*proxy[1].stride()[:3])
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    st = lib.bsa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _DTYPES[q.dtype],
                     B, H, Hkv, Sq, Sk, D,
                     _i64([q.stride(0), q.stride(1), q.stride(2)]),
                     _i64([k.stride(0), k.stride(1), k.stride(2)]),
                     _i64([v.stride(0), v.stride(1), v.stride(2)]),
                     _i64([out.stride(0), out.stride(1), out.stride(2)]),
                     ctypes.byref(bs), int(mask_mod), _ptr(kv_valid), scale,
                     (FLAG_VALIDATE if validate else 0) |
                     (FLAG_KV_HEAD_LISTS if kv_head_lists else 0), _stream(q))
    _check("bsa_fwd", st)
    return out, lse


def bsa_varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                   cu_total_m_blocks: torch.Tensor, block_idx_offsets: torch.Tensor,
                   total_m_blocks: int, total_n_blocks: int,
                   mask_list: Optional[Tuple[torch.Tensor, torch.Tensor]],
                   full_list: Optional[Tuple[torch.Tensor, torch.Tensor]],
                   block_q: int, block_kv: int, mask_mod: int = MASK_NONE,
                   softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, validate: bool = False,
                   window: Optional[Tuple[int, int]] = None,
                   kv_valid: Optional[torch.Tensor] = None,
                   max_seqlen_k: Optional[int] = None, kv_head_lists: bool = False):
    """Packed varlen forward.  q [Tq,H,D], k/v [Tk,Hkv,D]; lists (cnt int32
    [H,total_m_blocks], idx int32 [H,total_n_blocks]); cu arrays int32 [B+1]
    on the device; the two totals are host ints.  kv_valid (MASK_KV_VALID_COUNT):
    int32 [B, W] (row b: the valid-token counts of sequence b's KV blocks,
    sequence-local ids) or [W] shared by every sequence, W >=
    ceil(max_seqlen_k / block_kv); max_seqlen_k is read from cu_seqlens_k (a
    device->host copy) when not given.  kv_head_lists=True: lists [Hkv, ...],
    shared by each KV head's Q heads (packed).  Returns (O [Tq,H,D], LSE
    float32 [H,Tq])."""
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev(n, t)
        if t.dim() != 3 or t.stride(-1) != 1:
            raise ValueError(f"{n} must be 3-D [tokens,heads,D] with a contiguous last dimension")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bfloat16 or float32")
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k),
                 ("cu_total_m_blocks", cu_total_m_blocks), ("block_idx_offsets", block_idx_offsets)):
        _dev(n, t, torch.int32)
        if t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous 1-D int32 tensor")
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1 or cu_total_m_blocks.numel() != B + 1 or \
            block_idx_offsets.numel() != B + 1:
        raise ValueError("cu arrays must all have B+1 entries")
    Tq, H, D = q.shape
    Tk, Hkv, Dk = k.shape
    if Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [Tk,Hkv,D] matching q")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
    _dev("out", out, q.dtype)
    _dev("lse", lse, torch.float32)
    if tuple(out.shape) != (Tq, H, D) or out.stride(-1) != 1:
        raise ValueError("out must be [Tq,H,D] with a contiguous last dimension")
    if tuple(lse.shape) != (H, Tq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [H,Tq] tensor")
    if int(total_m_blocks) < 0 or int(total_n_blocks) < 0:
        raise ValueError("totals must be non-negative")
    shp = (Hkv if kv_head_lists else H, int(total_m_blocks), int(total_n_blocks))
    bs = _BlockSparse(_block_list(mask_list, False, shp), _block_list(full_list, False, shp),
                      int(block_q), int(block_kv), *_window(mask_mod, window))
    kvv_ld = 0
    if kv_valid is not None:
        _dev("kv_valid", kv_valid, torch.int32)
        if kv_valid.dim() not in (1, 2) or kv_valid.stride(-1) != 1 or \
                (kv_valid.dim() == 2 and kv_valid.shape[0] != B):
            raise ValueError("kv_valid must be int32 [B, W] or [W] with a contiguous last dimension")
        if max_seqlen_k is None:
            max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item()) if B else 0
        need = -(-int(max_seqlen_k) // block_kv) if block_kv > 0 else 0
        if kv_valid.shape[-1] < need:
            raise ValueError(f"kv_valid rows need {need} entries (ceil(max_seqlen_k / block_kv))")
        kvv_ld = kv_valid.stride(0) if kv_valid.dim() == 2 else 0
    elif mask_mod == MASK_KV_VALID_COUNT and mask_list is not None:
        raise ValueError("MASK_KV_VALID_COUNT needs kv_valid")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    st = lib.bsa_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _DTYPES[q.dtype],
                            B, H, Hkv, D, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                            _ptr(cu_total_m_blocks), _ptr(block_idx_offsets),
                            int(total_m_blocks), int(total_n_blocks), Tq,
                            _i64([q.stride(0), q.stride(1)]), _i64([k.stride(0), k.stride(1)]),
                            _i64([v.stride(0), v.stride(1)]), _i64([out.stride(0), out.stride(1)]),
                            ctypes.byref(bs), int(mask_mod), _ptr(kv_valid), int(kvv_ld), scale,
                            (FLAG_VALIDATE if validate else 0) |
                            (FLAG_KV_HEAD_LISTS if kv_head_lists else 0), _stream(q))
    _check("bsa_varlen_fwd", st)
    return out, lse


def bsa_mask_to_index(mask: torch.Tensor, cnt: Optional[torch.Tensor] = None,
                      idx: Optional[torch.Tensor] = None):
    """uint8 block mask [B,H,M,N] (contiguous, device) -> (cnt int32 [B,H,M],
    idx int32 [B,H,M,N]): selected ids in descending order, then -1."""
    lib = load_library()
    _dev("mask", mask, torch.uint8)
    if mask.dim() != 4 or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous uint8 [B,H,M,N] tensor")
    B, H, M, N = mask.shape
    if cnt is None:
        cnt = torch.empty((B, H, M), dtype=torch.int32, device=mask.device)
    if idx is None:
        idx = torch.empty((B, H, M, N), dtype=torch.int32, device=mask.device)
    if not cnt.is_contiguous() or not idx.is_contiguous() or tuple(idx.shape) != (B, H, M, N) \
            or tuple(cnt.shape) != (B, H, M):
        raise ValueError("cnt/idx must be contiguous [B,H,M] / [B,H,M,N] int32 tensors")
    st = lib.bsa_mask_to_index(_ptr(mask), B, H, M, N, _ptr(cnt), _ptr(idx), _stream(mask))
    _check("bsa_mask_to_index", st)
    return cnt, idx


def bsa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
            lse: torch.Tensor, dout: torch.Tensor,
            mask_list: Optional[Tuple[torch.Tensor, torch.Tensor]],
            full_list: Optional[Tuple[torch.Tensor, torch.Tensor]],
            block_q: int, block_kv: int, mask_mod: int = MASK_NONE,
            kv_valid: Optional[torch.Tensor] = None, softmax_scale: Optional[float] = None,
            window: Optional[Tuple[int, int]] = None, noalloc: bool = False,
            proxy: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Backward of bsa_fwd (head_dim 64/96/128/192/256): returns (dq, dk, dv),
    and with proxy=(k_mean, v_sum) (the forward's summaries, bf16, MASK_NONE)
    (dq, dk, dv, dk_mean, dv_sum) through bsa_bwd_proxy.
    bf16 tensors call bsa_bwd; fp32 tensors (all five) call bsa_bwd_f32, which
    rounds them to bf16 in its workspace and returns fp32 gradients.  o and
    lse are the forward's outputs, dout the gradient of o; the lists, block
    sizes, mask_mod, kv_valid, scale and window are the forward's.  The
    KV-major lists are built here with bsa_kv_major_lists.  noalloc=True calls
    bsa_bwd_noalloc (bf16 only; the row dots in the library's static
    per-device array, B*H*Sq <= 2**22) instead of passing a workspace."""
    lib = load_library()
    f32 = q.dtype == torch.float32
    if f32 and noalloc:
        raise ValueError("noalloc is bf16 only")
    if proxy is not None and (f32 or noalloc or mask_mod != MASK_NONE):
        raise ValueError("the proxy route's backward is bf16, MASK_NONE, with a workspace")
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev(n, t, torch.float32 if f32 else torch.bfloat16)
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{n} must be 4-D with a contiguous last dimension")
    _dev("lse", lse, torch.float32)
    B, Sq, H, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape) or o.shape != q.shape \
            or dout.shape != q.shape or tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous():
        raise ValueError("shapes: q/o/dout [B,Sq,H,D], k/v [B,Sk,Hkv,D], lse [B,H,Sq]")
    if dout.stride() != o.stride():
        o, dout = o.contiguous(), dout.contiguous()
    M, N = -(-Sq // block_q), -(-Sk // block_kv)

    def full_shape(lst):
        if lst is None:
            return None
        cnt, idx = lst
        return (cnt.expand(B, H, M).contiguous(), idx.expand(B, H, M, N).contiguous())
    ml, fl = full_shape(mask_list), full_shape(full_list)
    bs = _BlockSparse(_block_list(ml, True, (B, H, M, N)), _block_list(fl, True, (B, H, M, N)),
                      int(block_q), int(block_kv), *_window(mask_mod, window))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("q, k and v must be dense (their gradients take their strides)")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if proxy is not None:
        for n, t in zip(("proxy k_mean", "proxy v_sum"), proxy):
            _dev(n, t, torch.bfloat16)
            if tuple(t.shape) != (B, N, Hkv, D) or t.stride(-1) != 1:
                raise ValueError(f"{n} must be [B,N,Hkv,D]={(B, N, Hkv, D)} with a contiguous "
                                 "last dimension")
        bs.proxy_k, bs.proxy_v = proxy[0].data_ptr(), proxy[1].data_ptr()
        bs.proxy_k_str = (ctypes.c_int64 * 3)(*proxy[0].stride()[:3])
        bs.proxy_v_str = (ctypes.c_int64 * 3)(*proxy[1].stride()[:3])
        dks, dvs = torch.empty_like(proxy[0]), torch.empty_like(proxy[1])
        if dks.stride() != proxy[0].stride() or dvs.stride() != proxy[1].stride():
            raise ValueError("the summaries must be dense (their gradients take their strides)")
        nbytes = ctypes.c_int64()
        _check("bsa_bwd_proxy_work_size",
               lib.bsa_bwd_proxy_work_size(B, H, Hkv, Sq, Sk, D, int(block_q), int(block_kv),
                                           ctypes.byref(nbytes)))
        pwork = torch.empty(max(nbytes.value, 16), dtype=torch.uint8, device=q.device)
        st = lib.bsa_bwd_proxy(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(dks), _ptr(dvs), B, H, Hkv, Sq, Sk, D,
                               _i64([q.stride(0), q.stride(1), q.stride(2)]),
                               _i64([k.stride(0), k.stride(1), k.stride(2)]),
                               _i64([v.stride(0), v.stride(1), v.stride(2)]),
                               _i64([o.stride(0), o.stride(1), o.stride(2)]),
                               ctypes.byref(bs), scale, _ptr(pwork), _stream(q))
        _check("bsa_bwd_proxy", st)
        return dq, dk, dv, dks, dvs
    mt = bsa_kv_major_lists(ml) if ml is not None else None
    ft = bsa_kv_major_lists(fl) if fl is not None else None
    lt_m = _block_list(mt, True, (B, H, N, M))
    lt_f = _block_list(ft, True, (B, H, N, M))
    # row dots, then the dK/dV start order (fp32: then the bf16 copies)
    nwork = B * H * Sq + B * Hkv * N
    if f32:
        nwork = -(-nwork // 4) * 4 + 2 * (B * Sq * H * D + B * Sk * Hkv * D)
    work = None if noalloc else torch.empty(max(nwork, 1), dtype=torch.float32, device=q.device)
    if kv_valid is not None:
        _dev("kv_valid", kv_valid, torch.int32)
        if not kv_valid.is_contiguous() or kv_valid.numel() < N:
            raise ValueError(f"kv_valid must be a contiguous int32 tensor with {N} entries")
    elif mask_mod == MASK_KV_VALID_COUNT and mask_list is not None:
        raise ValueError("MASK_KV_VALID_COUNT needs kv_valid")
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), B, H, Hkv, Sq, Sk, D, _i64([q.stride(0), q.stride(1), q.stride(2)]),
            _i64([k.stride(0), k.stride(1), k.stride(2)]),
            _i64([v.stride(0), v.stride(1), v.stride(2)]),
            _i64([o.stride(0), o.stride(1), o.stride(2)]),
            ctypes.byref(bs), ctypes.byref(lt_m), ctypes.byref(lt_f), int(mask_mod),
            _ptr(kv_valid), scale]
    if noalloc:
        st = lib.bsa_bwd_noalloc(*args, _stream(q))
        _check("bsa_bwd_noalloc", st)
    elif f32:
        st = lib.bsa_bwd_f32(*args, _ptr(work), _stream(q))
        _check("bsa_bwd_f32", st)
    else:
        st = lib.bsa_bwd(*args, _ptr(work), _stream(q))
        _check("bsa_bwd", st)
    return dq, dk, dv


def bsa_varlen_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                   lse: torch.Tensor, dout: torch.Tensor,
                   cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                   cu_total_m_blocks: torch.Tensor, cu_total_kv_blocks: torch.Tensor,
                   block_idx_offsets: torch.Tensor, total_m_blocks: int, total_kv_blocks: int,
                   total_n_blocks: int,
                   mask_list: Optional[Tuple[torch.Tensor, torch.Tensor]],
                   full_list: Optional[Tuple[torch.Tensor, torch.Tensor]],
                   block_q: int, block_kv: int, mask_mod: int = MASK_NONE,
                   kv_valid: Optional[torch.Tensor] = None,
                   softmax_scale: Optional[float] = None,
                   window: Optional[Tuple[int, int]] = None,
                   max_seqlen_k: Optional[int] = None):
    """Backward of bsa_varlen_fwd (bf16): returns (dq [Tq,H,D], dk, dv [Tk,Hkv,D]).
    o and lse [H,Tq] are the forward's outputs, dout the gradient of o; the cu
    arrays, totals, lists (cnt [H,total_m_blocks], idx [H,total_n_blocks]),
    block sizes, mask_mod, kv_valid ([B, W] or [W]), scale and window are the
    forward's.  cu_total_kv_blocks (int32 [B+1] on the device) and
    total_kv_blocks count the KV blocks per sequence (bsa_varlen_offsets with
    the Q and KV roles swapped gives them).  The KV-major lists are built here
    with bsa_varlen_kv_major_lists."""
    lib = load_library()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev(n, t, torch.bfloat16)
        if t.dim() != 3 or t.stride(-1) != 1:
            raise ValueError(f"{n} must be 3-D [tokens,heads,D] with a contiguous last dimension")
    _dev("lse", lse, torch.float32)
    cus = (cu_seqlens_q, cu_seqlens_k, cu_total_m_blocks, cu_total_kv_blocks, block_idx_offsets)
    for n, t in zip(("cu_seqlens_q", "cu_seqlens_k", "cu_total_m_blocks", "cu_total_kv_blocks",
                     "block_idx_offsets"), cus):
        _dev(n, t, torch.int32)
        if t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous 1-D int32 tensor")
    B = cu_seqlens_q.numel() - 1
    if any(t.numel() != B + 1 for t in cus):
        raise ValueError("cu arrays must all have B+1 entries")
    Tq, H, D = q.shape
    Tk, Hkv, Dk = k.shape
    if Dk != D or tuple(v.shape) != tuple(k.shape) or o.shape != q.shape \
            or dout.shape != q.shape or tuple(lse.shape) != (H, Tq) or not lse.is_contiguous():
        raise ValueError("shapes: q/o/dout [Tq,H,D], k/v [Tk,Hkv,D], lse [H,Tq]")
    if dout.stride() != o.stride():
        o, dout = o.contiguous(), dout.contiguous()
    tm, tkv, tn = int(total_m_blocks), int(total_kv_blocks), int(total_n_blocks)

    def transposed(lst):
        if lst is None:
            return None
        cnt, idx = (x.expand(H, x.shape[1]).contiguous() for x in lst)
        return (cnt, idx), bsa_varlen_kv_major_lists((cnt, idx), cu_total_m_blocks,
                                                     cu_total_kv_blocks, block_idx_offsets,
                                                     tm, tkv)
    mp, fp = transposed(mask_list), transposed(full_list)
    ml, mt = mp if mp is not None else (None, None)
    fl, ft = fp if fp is not None else (None, None)
    bs = _BlockSparse(_block_list(ml, False, (H, tm, tn)), _block_list(fl, False, (H, tm, tn)),
                      int(block_q), int(block_kv), *_window(mask_mod, window))
    lt_m = _block_list(mt, False, (H, tkv, tn))
    lt_f = _block_list(ft, False, (H, tkv, tn))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("q, k and v must be dense (their gradients take their strides)")
    # row dots, then the dK/dV start order
    work = torch.empty(max(H * Tq + Hkv * tkv, 1), dtype=torch.float32, device=q.device)
    kvv_ld = 0
    if kv_valid is not None:
        _dev("kv_valid", kv_valid, torch.int32)
        if kv_valid.dim() not in (1, 2) or kv_valid.stride(-1) != 1 or \
                (kv_valid.dim() == 2 and kv_valid.shape[0] != B):
            raise ValueError("kv_valid must be int32 [B, W] or [W] with a contiguous last dimension")
        if max_seqlen_k is None:
            max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item()) if B else 0
        need = -(-int(max_seqlen_k) // block_kv) if block_kv > 0 else 0
        if kv_valid.shape[-1] < need:
            raise ValueError(f"kv_valid rows need {need} entries (ceil(max_seqlen_k / block_kv))")
        kvv_ld = kv_valid.stride(0) if kv_valid.dim() == 2 else 0
    elif mask_mod == MASK_KV_VALID_COUNT and mask_list is not None:
        raise ValueError("MASK_KV_VALID_COUNT needs kv_valid")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    st = lib.bsa_varlen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                            _ptr(dk), _ptr(dv), B, H, Hkv, D, *(_ptr(t) for t in cus[:4]),
                            _ptr(block_idx_offsets), tm, tkv, Tq,
                            _i64([q.stride(0), q.stride(1)]), _i64([k.stride(0), k.stride(1)]),
                            _i64([v.stride(0), v.stride(1)]), _i64([o.stride(0), o.stride(1)]),
                            ctypes.byref(bs), ctypes.byref(lt_m), ctypes.byref(lt_f),
                            int(mask_mod), _ptr(kv_valid), int(kvv_ld), scale, _ptr(work),
                            _stream(q))
    _check("bsa_varlen_bwd", st)
    return dq, dk, dv


def bsa_varlen_kv_major_lists(lists: Tuple[torch.Tensor, torch.Tensor],
                              cu_total_m_blocks: torch.Tensor, cu_total_kv_blocks: torch.Tensor,
                              block_idx_offsets: torch.Tensor, total_m_blocks: int,
                              total_kv_blocks: int):
    """Packed varlen lists (cnt int32 [H,total_m_blocks], idx int32
    [H,total_n_blocks], contiguous) -> KV-major lists (cnt_t int32
    [H,total_kv_blocks], idx_t int32 [H,total_n_blocks]; row (b, j) at
    block_idx_offsets[b] + j*num_m(b)): per KV block of each sequence, its
    Q blocks that list it, descending, then -1."""
    lib = load_library()
    cnt, idx = lists
    _dev("cnt", cnt, torch.int32)
    _dev("idx", idx, torch.int32)
    if cnt.dim() != 2 or idx.dim() != 2 or cnt.shape[0] != idx.shape[0] or \
            cnt.shape[1] != total_m_blocks or not cnt.is_contiguous() or not idx.is_contiguous():
        raise ValueError("lists must be contiguous int32 [H,total_m_blocks] / [H,total_n_blocks]")
    for n, t in (("cu_total_m_blocks", cu_total_m_blocks), ("cu_total_kv_blocks", cu_total_kv_blocks),
                 ("block_idx_offsets", block_idx_offsets)):
        _dev(n, t, torch.int32)
    H, tn = idx.shape
    B = cu_total_m_blocks.numel() - 1
    work = torch.empty((H, tn), dtype=torch.uint8, device=idx.device)
    cnt_t = torch.empty((H, int(total_kv_blocks)), dtype=torch.int32, device=idx.device)
    idx_t = torch.empty((H, tn), dtype=torch.int32, device=idx.device)
    st = lib.bsa_varlen_kv_major_lists(_ptr(cnt), _ptr(idx), H, B, _ptr(cu_total_m_blocks),
                                       _ptr(cu_total_kv_blocks), _ptr(block_idx_offsets),
                                       int(total_m_blocks), int(total_kv_blocks), tn, _ptr(work),
                                       _ptr(cnt_t), _ptr(idx_t), _stream(idx))
    _check("bsa_varlen_kv_major_lists", st)
    return cnt_t, idx_t


def bsa_kv_major_lists(lists: Tuple[torch.Tensor, torch.Tensor]):
    """Block lists (cnt int32 [B,H,M], idx int32 [B,H,M,N], contiguous, as
    bsa_mask_to_index writes them) -> KV-major lists (cnt_t int32 [B,H,N],
    idx_t int32 [B,H,N,M]): per KV block, the Q blocks that list it, in
    descending order, then -1."""
    lib = load_library()
    cnt, idx = lists
    _dev("cnt", cnt, torch.int32)
    _dev("idx", idx, torch.int32)
    if idx.dim() != 4 or cnt.shape != idx.shape[:3] or not cnt.is_contiguous() \
            or not idx.is_contiguous():
        raise ValueError("lists must be contiguous int32 [B,H,M] / [B,H,M,N] tensors")
    B, H, M, N = idx.shape
    work = torch.empty((B, H, N, M), dtype=torch.uint8, device=idx.device)
    cnt_t = torch.empty((B, H, N), dtype=torch.int32, device=idx.device)
    idx_t = torch.empty((B, H, N, M), dtype=torch.int32, device=idx.device)
    st = lib.bsa_kv_major_lists(_ptr(cnt), _ptr(idx), B, H, M, N, _ptr(work), _ptr(cnt_t),
                                _ptr(idx_t), _stream(idx))
    _check("bsa_kv_major_lists", st)
    return cnt_t, idx_t


def bsa_bitmask_to_index(words: torch.Tensor, N: int, H: Optional[int] = None,
                         cnt: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None):
    """Packed UInt32 block bitmap [B,Hkv,M,ceil(N/32)] (int32 or uint32,
    contiguous, device; bit j of word w selects KV block 32*w+j, padding bits
    past N ignored) -> (cnt int32 [B,H,M], idx int32 [B,H,M,N]) in the format
    of bsa_mask_to_index.  Q head h reads KV head h // (H // Hkv); H defaults
    to Hkv."""
    lib = load_library()
    if not isinstance(words, torch.Tensor) or words.dtype not in (torch.int32, torch.uint32) \
            or not words.is_cuda or words.dim() != 4 or not words.is_contiguous():
        raise ValueError("words must be a contiguous int32/uint32 [B,Hkv,M,W] device tensor")
    B, Hkv, M, W = words.shape
    H = Hkv if H is None else int(H)
    if N < 0 or W != (N + 31) // 32:
        raise ValueError(f"{W} words per row for N={N} blocks (need {(N + 31) // 32})")
    if Hkv == 0 or H % Hkv:
        raise ValueError(f"H={H} must be a positive multiple of Hkv={Hkv}")
    if cnt is None:
        cnt = torch.empty((B, H, M), dtype=torch.int32, device=words.device)
    if idx is None:
        idx = torch.empty((B, H, M, N), dtype=torch.int32, device=words.device)
    if not cnt.is_contiguous() or not idx.is_contiguous() or tuple(idx.shape) != (B, H, M, N) \
            or tuple(cnt.shape) != (B, H, M):
        raise ValueError("cnt/idx must be contiguous [B,H,M] / [B,H,M,N] int32 tensors")
    st = lib.bsa_bitmask_to_index(_ptr(words), B, Hkv, H, M, N, _ptr(cnt), _ptr(idx),
                                  _stream(words))
    _check("bsa_bitmask_to_index", st)
    return cnt, idx


def bsa_varlen_mask_to_index(mask: torch.Tensor, cu_total_m_blocks: torch.Tensor,
                             block_idx_offsets: torch.Tensor, total_m_blocks: int,
                             total_n_blocks: int):
    """Packed uint8 mask [H,total_n_blocks] -> (cnt [H,total_m_blocks],
    idx [H,total_n_blocks]) int32, same conversion per packed row."""
    lib = load_library()
    _dev("mask", mask, torch.uint8)
    if mask.dim() != 2 or not mask.is_contiguous() or mask.shape[1] != total_n_blocks:
        raise ValueError("mask must be a contiguous uint8 [H,total_n_blocks] tensor")
    H = mask.shape[0]
    B = cu_total_m_blocks.numel() - 1
    cnt = torch.empty((H, total_m_blocks), dtype=torch.int32, device=mask.device)
    idx = torch.empty((H, total_n_blocks), dtype=torch.int32, device=mask.device)
    st = lib.bsa_varlen_mask_to_index(_ptr(mask), H, B, _ptr(cu_total_m_blocks),
                                      _ptr(block_idx_offsets), int(total_m_blocks),
                                      int(total_n_blocks), _ptr(cnt), _ptr(idx), _stream(mask))
    _check("bsa_varlen_mask_to_index", st)
    return cnt, idx


def bsa_varlen_offsets(seqlens_q: Sequence[int], seqlens_k: Sequence[int], block_q: int,
                       block_kv: int):
    """Host-only: (cu_total_m_blocks, block_idx_offsets, total_m_blocks,
    total_n_blocks) as python lists/ints, computed by the library."""
    lib = load_library()
    B = len(seqlens_q)
    if len(seqlens_k) != B:
        raise ValueError("seqlens_q and seqlens_k differ in length")
    A = ctypes.c_int32 * max(B, 1)
    sq, sk = A(*seqlens_q), A(*seqlens_k)
    cu = (ctypes.c_int32 * (B + 1))()
    off = (ctypes.c_int32 * (B + 1))()
    tm, tn = ctypes.c_int32(), ctypes.c_int32()
    st = lib.bsa_varlen_offsets(sq, sk, B, int(block_q), int(block_kv), cu, off,
                                ctypes.byref(tm), ctypes.byref(tn))
    _check("bsa_varlen_offsets", st)
    return list(cu), list(off), tm.value, tn.value


def bsa_expand_kv_blocks(block_mask: torch.Tensor, block_valid: torch.Tensor, factor: int,
                         child: int):
    """Split logical KV blocks into `factor` child tiles of `child` tokens.
    block_mask uint8 [..., NL] (contiguous), block_valid int32 [NL] ->
    (full uint8 [..., NL*factor], part uint8 [..., NL*factor], kv_valid int32 [NL*factor])."""
    lib = load_library()
    _dev("block_mask", block_mask, torch.uint8)
    _dev("block_valid", block_valid, torch.int32)
    if not block_mask.is_contiguous() or not block_valid.is_contiguous():
        raise ValueError("block_mask and block_valid must be contiguous")
    NL = block_mask.shape[-1]
    if block_valid.numel() != NL:
        raise ValueError("block_valid must have one entry per logical KV block")
    R = block_mask.numel() // NL if NL else 0
    shape = tuple(block_mask.shape[:-1]) + (NL * factor,)
    full = torch.empty(shape, dtype=torch.uint8, device=block_mask.device)
    part = torch.empty(shape, dtype=torch.uint8, device=block_mask.device)
    kvv = torch.empty((NL * factor,), dtype=torch.int32, device=block_mask.device)
    st = lib.bsa_expand_kv_blocks(_ptr(block_mask), _ptr(block_valid), R, NL, int(factor),
                                  int(child), _ptr(full), _ptr(part), _ptr(kvv),
                                  _stream(block_mask))
    _check("bsa_expand_kv_blocks", st)
    return full, part, kvv


def bsa_block_sparsity(mask_mod: int, Sq: int, Sk: int, block_q: int, block_kv: int,
                       window: Optional[Tuple[int, int]] = None,
                       kv_valid: Optional[torch.Tensor] = None,
                       device: Optional[torch.device] = None):
    """Classify the (Q block, KV block) grid of an Sq x Sk problem under an
    element mask_mod: returns (full, part) uint8 [ceil(Sq/block_q),
    ceil(Sk/block_kv)] on the device (1 = every / some but not every element
    kept).  bsa_mask_to_index turns them into the full and mask lists."""
    lib = load_library()
    if block_q <= 0 or block_kv <= 0 or Sq < 0 or Sk < 0:
        raise ValueError("sizes must be non-negative and block sizes positive")
    dev = torch.device("cuda") if device is None else torch.device(device)
    if kv_valid is not None:
        _dev("kv_valid", kv_valid, torch.int32)
        dev = kv_valid.device
    M, N = -(-Sq // block_q), -(-Sk // block_kv)
    full = torch.empty((M, N), dtype=torch.uint8, device=dev)
    part = torch.empty((M, N), dtype=torch.uint8, device=dev)
    wl, wr = _window(mask_mod, window)
    with torch.cuda.device(dev):
        st = lib.bsa_block_sparsity(int(mask_mod), wl, wr, _ptr(kv_valid), int(Sq), int(Sk),
                                    int(block_q), int(block_kv), _ptr(full), _ptr(part),
                                    _stream(full))
    _check("bsa_block_sparsity", st)
    return full, part
