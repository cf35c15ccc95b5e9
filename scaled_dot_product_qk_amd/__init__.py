"""Python binding of the gfx950 attention library (argument marshalling only).

Every step of the computation runs in the HIP kernels of libattn_gfx950.so;
this module only fills the C structs of include/attn.h from torch tensors and
calls the C entry points with the same names.  torch provides device memory
and the current stream.  There is no other execution path: if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_gfx950.so")

ATTN_BF16, ATTN_F32 = 0, 1
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_DTYPE",
                4: "ATTN_ERR_LAYOUT", 5: "ATTN_ERR_UNSUPPORTED", 6: "ATTN_ERR_WORKSPACE",
                7: "ATTN_ERR_HIP", 8: "ATTN_ERR_SCRATCH"}
ATTN_DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20  # static workspace of attn_decode_noalloc, per device
EXPORTED = ("attn_fwd", "attn_fwd_masked", "attn_fwd_varlen", "attn_fwd_fp8", "attn_bwd",
            "attn_bwd_workspace_bytes", "attn_decode", "attn_decode_noalloc", "attn_decode_workspace_bytes",
            "attn_validate_fwd",
            "attn_validate_fwd_masked", "attn_validate_fwd_varlen", "attn_validate_fwd_fp8",
            "attn_validate_bwd", "attn_validate_decode", "attn_status_str", "attn_kernel_name",
            "attn_version")
ATTN_MASK_BOOL, ATTN_MASK_ADD_BF16 = 1, 2

_i64 = ctypes.c_int64
_i64x3 = _i64 * 3
_i64x2 = _i64 * 2


class FwdArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("B", _i64), ("Hq", _i64), ("Hkv", _i64), ("Lq", _i64), ("Lk", _i64), ("d", _i64),
                ("q_strides", _i64x3), ("k_strides", _i64x3), ("v_strides", _i64x3),
                ("o_strides", _i64x3),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float)]


class MaskArgs(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("kind", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("strides", _i64x3)]


class FwdVarlenArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("B", _i64), ("Hq", _i64), ("Hkv", _i64), ("total_q", _i64), ("total_k", _i64),
                ("max_seqlen_q", _i64), ("d", _i64),
                ("q_strides", _i64x2), ("k_strides", _i64x2), ("v_strides", _i64x2),
                ("o_strides", _i64x2),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float)]


class FwdFp8Args(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("B", _i64), ("Hq", _i64), ("Hkv", _i64), ("Lq", _i64), ("Lk", _i64), ("d", _i64),
                ("q_strides", _i64x3), ("k_strides", _i64x3), ("v_strides", _i64x3),
                ("o_strides", _i64x3),
                ("q_descale", ctypes.c_float), ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("B", _i64), ("Hq", _i64), ("Hkv", _i64), ("Lq", _i64), ("Lk", _i64), ("d", _i64),
                ("q_strides", _i64x3), ("k_strides", _i64x3), ("v_strides", _i64x3),
                ("o_strides", _i64x3), ("do_strides", _i64x3), ("dq_strides", _i64x3),
                ("dk_strides", _i64x3), ("dv_strides", _i64x3),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("seqlens", ctypes.c_void_p), ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("B", _i64), ("Hq", _i64), ("Hkv", _i64), ("Lmax", _i64), ("d", _i64),
                ("q_strides", _i64x2), ("k_strides", _i64x3), ("v_strides", _i64x3),
                ("o_strides", _i64x2),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (built by scaled_dot_product_qk_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m scaled_dot_product_qk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.attn_fwd.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
        L.attn_fwd.restype = ctypes.c_int
        L.attn_validate_fwd.argtypes = [ctypes.POINTER(FwdArgs)]
        L.attn_validate_fwd.restype = ctypes.c_int
        L.attn_fwd_masked.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(MaskArgs), ctypes.c_void_p]
        L.attn_fwd_masked.restype = ctypes.c_int
        L.attn_validate_fwd_masked.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(MaskArgs)]
        L.attn_validate_fwd_masked.restype = ctypes.c_int
        L.attn_fwd_varlen.argtypes = [ctypes.POINTER(FwdVarlenArgs), ctypes.c_void_p]
        L.attn_fwd_varlen.restype = ctypes.c_int
        L.attn_validate_fwd_varlen.argtypes = [ctypes.POINTER(FwdVarlenArgs)]
        L.attn_validate_fwd_varlen.restype = ctypes.c_int
        L.attn_fwd_fp8.argtypes = [ctypes.POINTER(FwdFp8Args), ctypes.c_void_p]
        L.attn_fwd_fp8.restype = ctypes.c_int
        L.attn_validate_fwd_fp8.argtypes = [ctypes.POINTER(FwdFp8Args)]
        L.attn_validate_fwd_fp8.restype = ctypes.c_int
        L.attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.attn_bwd.restype = ctypes.c_int
        L.attn_validate_bwd.argtypes = [ctypes.POINTER(BwdArgs)]
        L.attn_validate_bwd.restype = ctypes.c_int
        L.attn_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64]
        L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.attn_kernel_name.argtypes = [ctypes.POINTER(FwdArgs)]
        L.attn_kernel_name.restype = ctypes.c_char_p
        L.attn_decode.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
        L.attn_decode.restype = ctypes.c_int
        L.attn_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
        L.attn_decode_noalloc.restype = ctypes.c_int
        L.attn_validate_decode.argtypes = [ctypes.POINTER(DecodeArgs)]
        L.attn_validate_decode.restype = ctypes.c_int
        L.attn_decode_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
        L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
        L.attn_status_str.argtypes = [ctypes.c_int]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_version.argtypes = []
        L.attn_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().attn_status_str(status).decode()


def version() -> str:
    return lib().attn_version().decode()


# ------------------------------------------------------------------ helpers
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    return -1


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def make_fwd_args(q, k, v, o, lse, causal: bool, scale: Optional[float]) -> FwdArgs:
    a = FwdArgs()
    a.q, a.k, a.v, a.o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr()
    a.B, a.Hq, a.Lq, a.d = q.shape
    a.Hkv, a.Lk = k.shape[1], k.shape[2]
    a.q_strides = _i64x3(*q.stride()[:3])
    a.k_strides = _i64x3(*k.stride()[:3])
    a.v_strides = _i64x3(*v.stride()[:3])
    a.o_strides = _i64x3(*o.stride()[:3])
    a.dtype = _dtype_code(q)
    a.causal = 1 if causal else 0
    a.scale = 0.0 if scale is None else float(scale)
    return a


def _check_device(*tensors):
    dev = tensors[0].device
    for t in tensors:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must live on the same GPU device")


def _check_fwd_tensors(q, k, v):
    _check_device(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    for t in (q, k, v):
        if t.numel() and t.stride(3) != 1:
            raise ValueError("head_dim must be the innermost, contiguous dimension")


# ------------------------------------------------------------------ entry points
def attn_fwd(q, k, v, causal: bool = False, scale: Optional[float] = None, out=None, lse=None,
             stream=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """O and LSE of attention over device tensors q [B,Hq,Lq,d], k/v [B,Hkv,Lk,d]."""
    import torch
    _check_fwd_tensors(q, k, v)
    B, Hq, Lq, d = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    _check_device(q, out, lse)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.shape != (B, Hq, Lq):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Lq] tensor")
    if out.shape != q.shape or out.dtype != q.dtype or (out.numel() and out.stride(3) != 1):
        raise ValueError("out must match q's shape and dtype with a contiguous head_dim")
    args = make_fwd_args(q, k, v, out, lse, causal, scale)
    st = lib().attn_fwd(ctypes.byref(args), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return out, lse


def make_mask_args(mask, B: int, Hq: int, Lq: int, Lk: int) -> MaskArgs:
    """mask: bool (True = the pair takes part) or bf16 additive, broadcastable to
    [B, Hq, Lq, Lk] through its batch and head dimensions (4-D, key-contiguous)."""
    import torch
    if mask.dim() != 4 or mask.shape[2] != Lq or mask.shape[3] != Lk or mask.shape[0] not in (1, B) \
            or mask.shape[1] not in (1, Hq):
        raise ValueError(f"mask must be [B|1, Hq|1, Lq, Lk]; got {tuple(mask.shape)}")
    if mask.numel() and mask.stride(3) != 1:
        raise ValueError("the mask's key dimension must be contiguous")
    m = MaskArgs()
    m.data = mask.data_ptr()
    if mask.dtype == torch.bool:
        m.kind = ATTN_MASK_BOOL
    elif mask.dtype == torch.bfloat16:
        m.kind = ATTN_MASK_ADD_BF16
    else:
        raise ValueError("mask must be torch.bool or torch.bfloat16 (additive)")
    sb = 0 if mask.shape[0] == 1 else mask.stride(0)
    sh = 0 if mask.shape[1] == 1 else mask.stride(1)
    m.strides = _i64x3(sb, sh, mask.stride(2))
    return m


def attn_fwd_masked(q, k, v, mask, causal: bool = False, scale: Optional[float] = None, out=None, lse=None,
                    stream=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """attn_fwd with an attention mask (bool: True = take part; bf16: added to
    the scaled scores), broadcastable over batch and heads."""
    import torch
    _check_fwd_tensors(q, k, v)
    _check_device(q, mask)
    B, Hq, Lq, d = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    _check_device(q, out, lse)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.shape != (B, Hq, Lq):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Lq] tensor")
    args = make_fwd_args(q, k, v, out, lse, causal, scale)
    margs = make_mask_args(mask, B, Hq, Lq, k.shape[2])
    st = lib().attn_fwd_masked(ctypes.byref(args), ctypes.byref(margs), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_masked")
    return out, lse


def make_fwd_fp8_args(q8, k8, v8, o, lse, descales, causal: bool, scale: Optional[float]) -> FwdFp8Args:
    a = FwdFp8Args()
    a.q, a.k, a.v, a.o, a.lse = q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr()
    a.B, a.Hq, a.Lq, a.d = q8.shape
    a.Hkv, a.Lk = k8.shape[1], k8.shape[2]
    a.q_strides = _i64x3(*q8.stride()[:3])
    a.k_strides = _i64x3(*k8.stride()[:3])
    a.v_strides = _i64x3(*v8.stride()[:3])
    a.o_strides = _i64x3(*o.stride()[:3])
    a.q_descale, a.k_descale, a.v_descale = (float(x) for x in descales)
    a.causal = 1 if causal else 0
    a.scale = 0.0 if scale is None else float(scale)
    return a


def attn_fwd_fp8(q8, k8, v8, descales, causal: bool = False, scale: Optional[float] = None, out=None,
                 lse=None, stream=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """O (bf16) and LSE of attention over e4m3 codes: q8 [B,Hq,Lq,d], k8/v8
    [B,Hkv,Lk,d] as uint8 (or float8_e4m3fn) device tensors; descales =
    (q_descale, k_descale, v_descale), an element standing for descale *
    value(code)."""
    import torch
    q8, k8, v8 = (t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t for t in (q8, k8, v8))
    _check_fwd_tensors(q8, k8, v8)
    if q8.dtype != torch.uint8:
        raise ValueError("q8, k8, v8 must hold e4m3 codes (torch.uint8 or torch.float8_e4m3fn)")
    B, Hq, Lq, d = q8.shape
    if out is None:
        out = torch.empty((B, Hq, Lq, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q8.device)
    _check_device(q8, out, lse)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.shape != (B, Hq, Lq):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Lq] tensor")
    if out.shape != q8.shape or out.dtype != torch.bfloat16 or (out.numel() and out.stride(3) != 1):
        raise ValueError("out must be bf16 with q's shape and a contiguous head_dim")
    if len(descales) != 3:
        raise ValueError("descales = (q_descale, k_descale, v_descale)")
    args = make_fwd_fp8_args(q8, k8, v8, out, lse, descales, causal, scale)
    st = lib().attn_fwd_fp8(ctypes.byref(args), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_fp8")
    return out, lse


def make_fwd_varlen_args(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, o, lse, causal: bool,
                         scale: Optional[float]) -> FwdVarlenArgs:
    a = FwdVarlenArgs()
    a.q, a.k, a.v, a.o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr()
    a.cu_seqlens_q, a.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
    a.B = cu_seqlens_q.numel() - 1
    a.total_q, a.Hq, a.d = q.shape
    a.total_k, a.Hkv = k.shape[0], k.shape[1]
    a.max_seqlen_q = int(max_seqlen_q)
    a.q_strides = _i64x2(*q.stride()[:2])
    a.k_strides = _i64x2(*k.stride()[:2])
    a.v_strides = _i64x2(*v.stride()[:2])
    a.o_strides = _i64x2(*o.stride()[:2])
    a.dtype = _dtype_code(q)
    a.causal = 1 if causal else 0
    a.scale = 0.0 if scale is None else float(scale)
    return a


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                    scale: Optional[float] = None, out=None, lse=None,
                    stream=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """O [total_q,Hq,d] and LSE [Hq,total_q] of packed variable-length attention:
    q [total_q,Hq,d], k/v [total_k,Hkv,d], int32 device offsets cu_seqlens_q/k
    of B + 1 entries; max_seqlen_q (a host int) bounds every query length."""
    import torch
    _check_device(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError(f"q must be [total_q,Hq,d], k and v [total_k,Hkv,d]; got "
                         f"{tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    for t in (q, k, v):
        if t.numel() and t.stride(2) != 1:
            raise ValueError("head_dim must be the innermost, contiguous dimension")
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous 1-D int32 tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same B + 1 >= 1 entries")
    total_q, Hq, d = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    _check_device(q, out, lse)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.shape != (Hq, total_q):
        raise ValueError("lse must be a contiguous float32 [Hq, total_q] tensor")
    if out.shape != q.shape or out.dtype != q.dtype or (out.numel() and out.stride(2) != 1):
        raise ValueError("out must match q's shape and dtype with a contiguous head_dim")
    args = make_fwd_varlen_args(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, out, lse, causal, scale)
    st = lib().attn_fwd_varlen(ctypes.byref(args), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_varlen")
    return out, lse


def attn_bwd_workspace_bytes(B: int, Hq: int, Lq: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Lq))


def make_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, scale: Optional[float]) -> BwdArgs:
    a = BwdArgs()
    a.q, a.k, a.v, a.o, a.dout = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr()
    a.lse, a.dq, a.dk, a.dv = lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.B, a.Hq, a.Lq, a.d = q.shape
    a.Hkv, a.Lk = k.shape[1], k.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(a, f"{name}_strides", _i64x3(*t.stride()[:3]))
    a.dtype = _dtype_code(q)
    a.causal = 1 if causal else 0
    a.scale = 0.0 if scale is None else float(scale)
    return a


def attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: Optional[float] = None, dq=None, dk=None,
             dv=None, workspace=None, stream=None):
    """dQ, dK, dV of attention for the output gradient dout, recomputing the
    probabilities from lse (as attn_fwd returned it for q, k, v, o)."""
    import torch
    _check_fwd_tensors(q, k, v)
    _check_device(q, o, lse, dout)
    for t in (o, dout):
        if t.shape != q.shape or t.dtype != q.dtype or (t.numel() and t.stride(3) != 1):
            raise ValueError("o and dout must match q's shape and dtype with a contiguous head_dim")
    B, Hq, Lq, d = q.shape
    if lse.shape != (B, Hq, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be the contiguous float32 [B, Hq, Lq] tensor attn_fwd returned")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    _check_device(q, dq, dk, dv)
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype or (t.numel() and t.stride(3) != 1):
            raise ValueError("gradients must match their inputs' shapes and dtypes with a contiguous head_dim")
    need = attn_bwd_workspace_bytes(B, Hq, Lq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_device(q, workspace)
    args = make_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, causal, scale)
    st = lib().attn_bwd(ctypes.byref(args), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                        _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def kernel_name(q, k, v, causal: bool = False, scale: Optional[float] = None) -> str:
    """Name of the kernel attn_fwd launches for these tensors ("none" if invalid)."""
    args = make_fwd_args(q, k, v, q, q, causal, scale)
    return lib().attn_kernel_name(ctypes.byref(args)).decode()


def attn_decode_workspace_bytes(B: int, Hq: int, Lmax: int, d: int) -> int:
    return int(lib().attn_decode_workspace_bytes(B, Hq, Lmax, d))


def make_decode_args(q, k_cache, v_cache, seqlens, o, lse, scale: Optional[float]) -> DecodeArgs:
    a = DecodeArgs()
    a.q, a.k_cache, a.v_cache = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr()
    a.seqlens, a.o, a.lse = seqlens.data_ptr(), o.data_ptr(), lse.data_ptr()
    a.B, a.Hq, a.d = q.shape
    a.Hkv, a.Lmax = k_cache.shape[1], k_cache.shape[2]
    a.q_strides = _i64x2(*q.stride()[:2])
    a.k_strides = _i64x3(*k_cache.stride()[:3])
    a.v_strides = _i64x3(*v_cache.stride()[:3])
    a.o_strides = _i64x2(*o.stride()[:2])
    a.dtype = _dtype_code(q)
    a.scale = 0.0 if scale is None else float(scale)
    return a


def attn_decode(q, k_cache, v_cache, seqlens, scale: Optional[float] = None, workspace=None,
                out=None, lse=None, stream=None):
    """O [B,Hq,d] and LSE [B,Hq] of one query token per sequence against a KV cache.

    q [B,Hq,d]; k_cache/v_cache [B,Hkv,Lmax,d]; seqlens int32 [B] on the device.
    workspace: optional device tensor (any dtype) of at least attn_decode_workspace_bytes bytes.
    """
    import torch
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B,Hq,d] and the caches [B,Hkv,Lmax,d]")
    if seqlens.dtype != torch.int32 or seqlens.numel() != q.shape[0]:
        raise ValueError("seqlens must be int32 [B]")
    for t in (q, k_cache, v_cache):
        if t.numel() and t.stride(-1) != 1:
            raise ValueError("head_dim must be the innermost, contiguous dimension")
    _check_device(q, k_cache, v_cache, seqlens)
    B, Hq, d = q.shape
    Lmax = k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_device(q, out, lse)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.shape != (B, Hq):
        raise ValueError("lse must be a contiguous float32 [B, Hq] tensor")
    if out.shape != q.shape or out.dtype != q.dtype or (out.numel() and out.stride(-1) != 1):
        raise ValueError("out must match q's shape and dtype with a contiguous head_dim")
    need = attn_decode_workspace_bytes(B, Hq, Lmax, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_device(q, workspace)
    args = make_decode_args(q, k_cache, v_cache, seqlens, out, lse, scale)
    st = lib().attn_decode(ctypes.byref(args), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_decode")
    return out, lse


def attn_decode_noalloc(q, k_cache, v_cache, seqlens, out, lse, scale: Optional[float] = None, stream=None):
    """attn_decode with the library's static device workspace: the C entry
    point allocates nothing, and neither does this call, so the caller passes
    the outputs out [B,Hq,d] and lse [B,Hq] (float32, contiguous).  Calls that
    may overlap on one device share that workspace and must be ordered (one
    stream).  Sizes needing more than ATTN_DECODE_NOALLOC_SCRATCH_BYTES of
    workspace raise AttnError (ATTN_ERR_SCRATCH)."""
    import torch
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B,Hq,d] and the caches [B,Hkv,Lmax,d]")
    if seqlens.dtype != torch.int32 or seqlens.numel() != q.shape[0]:
        raise ValueError("seqlens must be int32 [B]")
    for t in (q, k_cache, v_cache):
        if t.numel() and t.stride(-1) != 1:
            raise ValueError("head_dim must be the innermost, contiguous dimension")
    _check_device(q, k_cache, v_cache, seqlens, out, lse)
    B, Hq, _ = q.shape
    if not lse.is_contiguous() or lse.dtype != torch.float32 or lse.shape != (B, Hq):
        raise ValueError("lse must be a contiguous float32 [B, Hq] tensor")
    if out.shape != q.shape or out.dtype != q.dtype or (out.numel() and out.stride(-1) != 1):
        raise ValueError("out must match q's shape and dtype with a contiguous head_dim")
    args = make_decode_args(q, k_cache, v_cache, seqlens, out, lse, scale)
    st = lib().attn_decode_noalloc(ctypes.byref(args), _stream_handle(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_noalloc")
    return out, lse


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
