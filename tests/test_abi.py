"""The C-ABI library on the host: it loads, exports what include/attn.h
declares, and rejects every invalid argument before any device work.

No GPU is needed: the validation functions make no HIP call, and attn_fwd /
attn_decode return their error before touching the device.  The pointers used
here are fake addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import scaled_dot_product_qk_amd as sdpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, DTYPE, LAYOUT, UNSUP, WS, HIP = range(8)
P = 0x7f0000000000  # a 256-byte aligned fake device address


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = sdpa.lib()
    declared = header_functions()
    assert declared, "no declarations parsed"
    assert set(declared) == set(sdpa.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name
    assert sdpa.version().startswith("attn-gfx950")


def test_status_strings():
    for s in range(9):
        assert sdpa.status_str(s) and sdpa.status_str(s) != "unknown status"
    assert sdpa.status_str(99) == "unknown status"


def fwd_args(**kw):
    a = sdpa.FwdArgs()
    B, Hq, Hkv, Lq, Lk, d = kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("Lq", 300), \
        kw.get("Lk", 300), kw.get("d", 64)
    a.q, a.k, a.v, a.o, a.lse = [kw.get(n, P + i * 0x10000000) for i, n in
                                 enumerate(("q", "k", "v", "o", "lse"))]
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.d = B, Hq, Hkv, Lq, Lk, d
    a.q_strides = sdpa._i64x3(*kw.get("qs", (Hq * Lq * d, Lq * d, d)))
    a.k_strides = sdpa._i64x3(*kw.get("ks", (Hkv * Lk * d, Lk * d, d)))
    a.v_strides = sdpa._i64x3(*kw.get("vs", (Hkv * Lk * d, Lk * d, d)))
    a.o_strides = sdpa._i64x3(*kw.get("os", (Hq * Lq * d, Lq * d, d)))
    a.dtype = kw.get("dtype", sdpa.ATTN_BF16)
    a.causal = kw.get("causal", 0)
    a.scale = kw.get("scale", 0.0)
    return a


def vfwd(**kw):
    return sdpa.lib().attn_validate_fwd(ctypes.byref(fwd_args(**kw)))


def run_fwd(**kw):
    # Only reached with invalid arguments: attn_fwd returns before any HIP call.
    return sdpa.lib().attn_fwd(ctypes.byref(fwd_args(**kw)), None)


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("causal", [0, 1])
def test_fwd_valid_configurations(d, dtype, causal):
    assert vfwd(d=d, dtype=dtype, causal=causal) == OK
    name = sdpa.lib().attn_kernel_name(ctypes.byref(fwd_args(d=d, dtype=dtype, causal=causal))).decode()
    assert name == f"attn_fwd_{'bf16' if dtype == 0 else 'f32'}_d{d}" + ("_causal" if causal else "")


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL),
    (dict(dtype=2), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(B=-1), SHAPE), (dict(Lq=-5), SHAPE), (dict(Hkv=0), SHAPE), (dict(Hq=8, Hkv=3), SHAPE),
    (dict(scale=float("nan")), SHAPE),
    (dict(scale=float("inf")), SHAPE),
    (dict(d=96), UNSUP), (dict(d=32), UNSUP), (dict(d=256), UNSUP), (dict(d=0), UNSUP),
    (dict(q=P + 8), LAYOUT), (dict(k=P + 2), LAYOUT), (dict(lse=P + 4), LAYOUT),
    (dict(qs=(8 * 300 * 64, 300 * 64, 68)), LAYOUT),   # token stride not a 16-byte multiple
    (dict(ks=(-1, 300 * 64, 64)), LAYOUT),
    (dict(dtype=1, qs=(8 * 300 * 64, 300 * 64, 66)), LAYOUT),
    (dict(Lq=2 ** 31, Lk=2 ** 31), UNSUP),
    (dict(ks=(8 * 300 * 64, 300 * 64, 2 ** 28)), UNSUP),   # K token stride past the copy limit
    (dict(vs=(8 * 300 * 64, 300 * 64, 2 ** 28)), UNSUP),
])
def test_fwd_rejections(kw, status):
    assert vfwd(**kw) == status
    assert run_fwd(**kw) == status
    assert sdpa.lib().attn_kernel_name(ctypes.byref(fwd_args(**kw))).decode() == "none"


def test_fwd_token_stride_limit_is_bf16_only():
    big = (8 * 300 * 64, 300 * 64, 2 ** 28 - 8)
    assert vfwd(ks=big, vs=big) == OK
    assert vfwd(dtype=1, ks=(8 * 300 * 64, 300 * 64, 2 ** 28), vs=(8 * 300 * 64, 300 * 64, 2 ** 28)) == OK


def test_fwd_empty_inputs_are_valid_noops():
    assert vfwd(B=0) == OK and run_fwd(B=0) == OK
    assert vfwd(Hq=0, Hkv=0) == OK and run_fwd(Hq=0, Hkv=0) == OK
    assert vfwd(Lq=0) == OK and run_fwd(Lq=0) == OK
    # no keys: valid (O = 0, LSE = -inf); k and v may be NULL then
    assert vfwd(Lk=0, k=0, v=0) == OK
    assert vfwd(Lk=0, causal=1, k=0, v=0) == OK


@pytest.mark.parametrize("Lq,Lk", [(300, 200), (200, 300), (1, 4096), (4096, 1)])
def test_fwd_cross_attention_shapes_are_valid(Lq, Lk):
    # Lq != Lk (cross-attention), causal or not; causal is top-left (j <= i)
    for causal in (0, 1):
        assert vfwd(Lq=Lq, Lk=Lk, causal=causal) == OK


def test_fwd_null_struct():
    L = sdpa.lib()
    assert L.attn_validate_fwd(None) == NULL
    assert L.attn_fwd(None, None) == NULL
    assert L.attn_kernel_name(None).decode() == "none"


def dec_args(**kw):
    a = sdpa.DecodeArgs()
    B, Hq, Hkv, Lmax, d = kw.get("B", 4), kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("Lmax", 1000), \
        kw.get("d", 128)
    a.q, a.k_cache, a.v_cache, a.seqlens, a.o, a.lse = [
        kw.get(n, P + i * 0x10000000) for i, n in
        enumerate(("q", "k_cache", "v_cache", "seqlens", "o", "lse"))]
    a.B, a.Hq, a.Hkv, a.Lmax, a.d = B, Hq, Hkv, Lmax, d
    a.q_strides = sdpa._i64x2(*kw.get("qs", (Hq * d, d)))
    a.k_strides = sdpa._i64x3(*kw.get("ks", (Hkv * Lmax * d, Lmax * d, d)))
    a.v_strides = sdpa._i64x3(*kw.get("vs", (Hkv * Lmax * d, Lmax * d, d)))
    a.o_strides = sdpa._i64x2(*kw.get("os", (Hq * d, d)))
    a.dtype = kw.get("dtype", sdpa.ATTN_BF16)
    a.scale = kw.get("scale", 0.0)
    return a


def vdec(**kw):
    return sdpa.lib().attn_validate_decode(ctypes.byref(dec_args(**kw)))


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 8), (4, 4), (40, 1)])
def test_decode_valid(d, Hq, Hkv):
    assert vdec(d=d, Hq=Hq, Hkv=Hkv) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), NULL), (dict(seqlens=0), NULL), (dict(k_cache=0), NULL), (dict(lse=0), NULL),
    (dict(dtype=7), DTYPE), (dict(dtype=1), UNSUP), (dict(d=96), UNSUP), (dict(d=32), UNSUP),
    (dict(Hkv=3), SHAPE), (dict(Hkv=0), SHAPE), (dict(Lmax=-1), SHAPE),
    (dict(scale=float("nan")), SHAPE),
    (dict(q=P + 2), LAYOUT), (dict(seqlens=P + 2), LAYOUT), (dict(ks=(8 * 1000 * 128, 1000 * 128, 130)), LAYOUT),
    (dict(B=64, Lmax=40_000_000), UNSUP), (dict(Lmax=2 ** 31), UNSUP),
])
def test_decode_rejections(kw, status):
    assert vdec(**kw) == status
    ws = sdpa.attn_decode_workspace_bytes(4, 8, 1000, 128)
    assert sdpa.lib().attn_decode(ctypes.byref(dec_args(**kw)), P, ws, None) == status


def test_decode_workspace_rules():
    L = sdpa.lib()
    need = sdpa.attn_decode_workspace_bytes(4, 8, 1000, 128)
    # 1000 slots span at most 3 pieces of >= 512 slots: O partials 4*8*3*128 floats
    # (256-aligned) + LSE partials
    assert need == 4 * 8 * 3 * 128 * 4 + 4 * 8 * 3 * 4
    assert L.attn_decode(ctypes.byref(dec_args()), None, need, None) == WS
    assert L.attn_decode(ctypes.byref(dec_args()), P, need - 1, None) == WS
    assert L.attn_decode(ctypes.byref(dec_args()), P + 16, need, None) == LAYOUT
    assert sdpa.attn_decode_workspace_bytes(-1, 8, 10, 128) == 0
    assert sdpa.attn_decode_workspace_bytes(64, 32, 8192, 128) == 64 * 32 * 17 * 129 * 4
    assert sdpa.attn_decode_workspace_bytes(2, 2, 0, 128) == 0


def test_decode_empty_is_noop():
    L = sdpa.lib()
    assert vdec(B=0) == OK and L.attn_decode(ctypes.byref(dec_args(B=0)), None, 0, None) == OK
    assert vdec(Hq=0, Hkv=0) == OK


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sdpa.attn_fwd(q, q, q)
    with pytest.raises(ValueError):
        sdpa.attn_decode(torch.zeros(1, 2, 64, dtype=torch.bfloat16), q, q,
                         torch.ones(1, dtype=torch.int32))


def test_build_entry_point_exists():
    import importlib
    ge = importlib.import_module("__graft_entry__")
    assert callable(ge.build) and callable(ge.smoke)


def var_args(**kw):
    a = sdpa.FwdVarlenArgs()
    B, Hq, Hkv, tq, tk, mq, d = (kw.get("B", 3), kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("total_q", 500),
                                 kw.get("total_k", 700), kw.get("max_seqlen_q", 300), kw.get("d", 128))
    a.q, a.k, a.v, a.o, a.lse, a.cu_seqlens_q, a.cu_seqlens_k = [
        kw.get(n, P + i * 0x10000000) for i, n in
        enumerate(("q", "k", "v", "o", "lse", "cu_seqlens_q", "cu_seqlens_k"))]
    a.B, a.Hq, a.Hkv, a.total_q, a.total_k, a.max_seqlen_q, a.d = B, Hq, Hkv, tq, tk, mq, d
    a.q_strides = sdpa._i64x2(*kw.get("qs", (Hq * d, d)))
    a.k_strides = sdpa._i64x2(*kw.get("ks", (Hkv * d, d)))
    a.v_strides = sdpa._i64x2(*kw.get("vs", (Hkv * d, d)))
    a.o_strides = sdpa._i64x2(*kw.get("os", (Hq * d, d)))
    a.dtype = kw.get("dtype", sdpa.ATTN_BF16)
    a.causal = kw.get("causal", 0)
    a.scale = kw.get("scale", 0.0)
    return a


def vvar(**kw):
    return sdpa.lib().attn_validate_fwd_varlen(ctypes.byref(var_args(**kw)))


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_varlen_valid(d, causal):
    assert vvar(d=d, causal=causal) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), NULL), (dict(cu_seqlens_q=0), NULL), (dict(cu_seqlens_k=0), NULL), (dict(lse=0), NULL),
    (dict(k=0), NULL), (dict(dtype=1), UNSUP), (dict(dtype=5), DTYPE), (dict(d=96), UNSUP),
    (dict(Hkv=3), SHAPE), (dict(B=-1), SHAPE), (dict(max_seqlen_q=501), SHAPE), (dict(total_k=-1), SHAPE),
    (dict(scale=float("inf")), SHAPE),
    (dict(q=P + 8), LAYOUT), (dict(cu_seqlens_k=P + 2), LAYOUT), (dict(qs=(8 * 128 + 4, 128)), LAYOUT),
    (dict(ks=(2 ** 28, 128)), UNSUP), (dict(total_q=2 ** 31, max_seqlen_q=10), UNSUP),
])
def test_varlen_rejections(kw, status):
    assert vvar(**kw) == status
    assert sdpa.lib().attn_fwd_varlen(ctypes.byref(var_args(**kw)), None) == status


def test_varlen_empty_is_noop():
    L = sdpa.lib()
    for kw in (dict(B=0), dict(Hq=0, Hkv=0), dict(max_seqlen_q=0)):
        assert vvar(**kw) == OK and L.attn_fwd_varlen(ctypes.byref(var_args(**kw)), None) == OK
    # no keys at all: k and v may be NULL (every row gets O = 0, LSE = -inf)
    assert vvar(total_k=0, k=0, v=0) == OK
    assert L.attn_validate_fwd_varlen(None) == NULL


def bwd_args(**kw):
    a = sdpa.BwdArgs()
    B, Hq, Hkv, Lq, Lk, d = (kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("Lq", 300),
                             kw.get("Lk", 300), kw.get("d", 64))
    names = ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv")
    for i, n in enumerate(names):
        setattr(a, n, kw.get(n, P + i * 0x10000000))
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.d = B, Hq, Hkv, Lq, Lk, d
    qs, ks = (Hq * Lq * d, Lq * d, d), (Hkv * Lk * d, Lk * d, d)
    for n, dflt in (("q", qs), ("k", ks), ("v", ks), ("o", qs), ("do", qs), ("dq", qs), ("dk", ks), ("dv", ks)):
        setattr(a, f"{n}_strides", sdpa._i64x3(*kw.get(f"{n}s", dflt)))
    a.dtype = kw.get("dtype", sdpa.ATTN_BF16)
    a.causal = kw.get("causal", 0)
    a.scale = kw.get("scale", 0.0)
    return a


def vbwd(**kw):
    return sdpa.lib().attn_validate_bwd(ctypes.byref(bwd_args(**kw)))


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("Lq,Lk", [(300, 300), (100, 700), (700, 100)])
def test_bwd_valid(d, causal, Lq, Lk):
    assert vbwd(d=d, causal=causal, Lq=Lq, Lk=Lk) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), NULL), (dict(dout=0), NULL), (dict(lse=0), NULL), (dict(dq=0), NULL), (dict(dk=0), NULL),
    (dict(dv=0), NULL), (dict(dtype=1), UNSUP), (dict(dtype=9), DTYPE), (dict(d=96), UNSUP), (dict(d=32), UNSUP),
    (dict(Hkv=3), SHAPE), (dict(Lq=-1), SHAPE), (dict(scale=float("nan")), SHAPE),
    (dict(dq=P + 8), LAYOUT), (dict(lse=P + 2), LAYOUT), (dict(dos=(8 * 300 * 64, 300 * 64, 66)), LAYOUT),
])
def test_bwd_rejections(kw, status):
    assert vbwd(**kw) == status
    ws = sdpa.attn_bwd_workspace_bytes(2, 8, 300)
    assert sdpa.lib().attn_bwd(ctypes.byref(bwd_args(**kw)), P, ws, None) == status


def test_bwd_workspace_rules():
    L = sdpa.lib()
    need = sdpa.attn_bwd_workspace_bytes(2, 8, 300)
    assert need == (2 * 8 * 300 * 8 + 255) // 256 * 256
    assert L.attn_bwd(ctypes.byref(bwd_args()), None, need, None) == WS
    assert L.attn_bwd(ctypes.byref(bwd_args()), P, need - 1, None) == WS
    assert L.attn_bwd(ctypes.byref(bwd_args()), P + 16, need, None) == LAYOUT
    assert sdpa.attn_bwd_workspace_bytes(-1, 8, 3) == 0
    # nothing to do: no call touches the device
    assert L.attn_bwd(ctypes.byref(bwd_args(B=0)), None, 0, None) == OK
    assert L.attn_bwd(ctypes.byref(bwd_args(Lq=0, Lk=0)), None, 0, None) == OK
    assert L.attn_validate_bwd(None) == NULL


def test_bwd_query_token_stride_limit():
    # the backward's copies address up to 31 rows of Q, dO, K and V with 32-bit lane offsets
    big = 1 << 26
    assert vbwd(Lq=300, Lk=300, qs=(8 * big * 300, big * 300, big)) == UNSUP
    assert vbwd(Lq=300, Lk=300, dos=(8 * big * 300, big * 300, big)) == UNSUP
    assert vbwd(Lq=300, Lk=300, ks=(2 * big * 300, big * 300, big)) == UNSUP
    assert vbwd(Lq=300, Lk=300, vs=(2 * big * 300, big * 300, big)) == UNSUP
    assert vbwd(Lq=300, Lk=300, qs=(8 * (big - 8) * 300, (big - 8) * 300, big - 8)) == OK


def mask_args(**kw):
    m = sdpa.MaskArgs()
    m.data = kw.get("data", P + 0x70000000)
    m.kind = kw.get("kind", sdpa.ATTN_MASK_BOOL)
    m.strides = sdpa._i64x3(*kw.get("ms", (0, 0, 320)))
    return m


def vmask(fkw=None, **kw):
    return sdpa.lib().attn_validate_fwd_masked(ctypes.byref(fwd_args(**(fkw or {}))), ctypes.byref(mask_args(**kw)))


@pytest.mark.parametrize("kind", [1, 2])
@pytest.mark.parametrize("d", [64, 80, 128])
def test_masked_valid(kind, d):
    assert vmask(dict(d=d, Lk=320, Lq=300, ks=(2 * 320 * d, 320 * d, d), vs=(2 * 320 * d, 320 * d, d)),
                 kind=kind) == OK


@pytest.mark.parametrize("fkw,kw,status", [
    (None, dict(kind=0), DTYPE), (None, dict(kind=3), DTYPE), (None, dict(data=0), NULL),
    (dict(dtype=1), dict(), UNSUP), (None, dict(data=P + 8), LAYOUT), (None, dict(ms=(0, 0, 303)), LAYOUT),
    (None, dict(ms=(-1, 0, 320)), LAYOUT),
    (None, dict(), UNSUP),                                   # Lk = 300 is not a multiple of 16
    (dict(Lk=320, Lq=320, ks=(2 * 320 * 64, 320 * 64, 64), vs=(2 * 320 * 64, 320 * 64, 64)),
     dict(ms=(0, 0, 2 ** 27)), UNSUP),                       # mask rows too far apart
    (dict(Lk=320, Lq=320, ks=(2 * 320 * 64, 320 * 64, 64), vs=(2 * 320 * 64, 320 * 64, 64)),
     dict(kind=2, ms=(0, 0, 324)), LAYOUT),                  # bf16 rows must start on 16 bytes
])
def test_masked_rejections(fkw, kw, status):
    assert vmask(fkw, **kw) == status
    assert sdpa.lib().attn_fwd_masked(ctypes.byref(fwd_args(**(fkw or {}))), ctypes.byref(mask_args(**kw)),
                                      None) == status


def test_masked_null_mask_struct():
    assert sdpa.lib().attn_validate_fwd_masked(ctypes.byref(fwd_args()), None) == NULL


# ------------------------------------------------------------------ FP8
def fp8_args(**kw):
    a = sdpa.FwdFp8Args()
    B, Hq, Hkv, Lq, Lk, d = kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("Lq", 300), \
        kw.get("Lk", 300), kw.get("d", 128)
    a.q, a.k, a.v, a.o, a.lse = [kw.get(n, P + i * 0x10000000) for i, n in
                                 enumerate(("q", "k", "v", "o", "lse"))]
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.d = B, Hq, Hkv, Lq, Lk, d
    a.q_strides = sdpa._i64x3(*kw.get("qs", (Hq * Lq * d, Lq * d, d)))
    a.k_strides = sdpa._i64x3(*kw.get("ks", (Hkv * Lk * d, Lk * d, d)))
    a.v_strides = sdpa._i64x3(*kw.get("vs", (Hkv * Lk * d, Lk * d, d)))
    a.o_strides = sdpa._i64x3(*kw.get("os", (Hq * Lq * d, Lq * d, d)))
    a.q_descale, a.k_descale, a.v_descale = kw.get("descales", (0.01, 0.02, 0.03))
    a.causal = kw.get("causal", 0)
    a.scale = kw.get("scale", 0.0)
    return a


def vfp8(**kw):
    return sdpa.lib().attn_validate_fwd_fp8(ctypes.byref(fp8_args(**kw)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("Lq,Lk", [(300, 300), (100, 700), (700, 100)])
def test_fp8_valid(d, causal, Lq, Lk):
    assert vfp8(d=d, causal=causal, Lq=Lq, Lk=Lk) == OK
    assert vfp8(d=d, causal=causal, Lq=Lq, Lk=Lk, descales=(-0.5, 2.0, -1.0), scale=-0.1) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(d=80), UNSUP), (dict(d=96), UNSUP), (dict(Hq=6, Hkv=4), SHAPE), (dict(Lq=-1), SHAPE),
    (dict(descales=(float("nan"), 1.0, 1.0)), SHAPE), (dict(descales=(1.0, float("inf"), 1.0)), SHAPE),
    (dict(descales=(1.0, 1.0, float("inf"))), SHAPE), (dict(scale=float("nan")), SHAPE),
    (dict(descales=(3e38, 3e38, 1.0)), SHAPE),                       # score multiplier past the float range
    (dict(q=0), NULL), (dict(lse=0), NULL), (dict(k=0), NULL),
    (dict(q=P + 8), LAYOUT), (dict(o=P + 4), LAYOUT),
    (dict(qs=(300 * 8 * 128, 300 * 128, 136)), LAYOUT),              # token stride not 16 bytes
    (dict(os=(300 * 8 * 128, 300 * 128, 132)), LAYOUT),              # bf16 output stride not 16 bytes
    (dict(ks=(1 << 40, 1 << 30, 1 << 28)), UNSUP),                   # K token stride past 2^28 bytes
])
def test_fp8_rejections(kw, status):
    assert vfp8(**kw) == status
    a = fp8_args(**kw)
    assert sdpa.lib().attn_fwd_fp8(ctypes.byref(a), None) == status


def test_fp8_token_stride_limit_and_bf16_output_stride():
    assert vfp8(ks=(1 << 40, 1 << 30, (1 << 28) - 16), vs=(1 << 40, 1 << 30, (1 << 28) - 16)) == OK
    assert vfp8(os=(300 * 8 * 136, 300 * 136, 136)) == OK           # padded bf16 rows, 16-byte multiple


def test_fp8_empty_inputs_are_valid_noops():
    for kw in (dict(B=0), dict(Hq=0, Hkv=0), dict(Lq=0)):
        a = fp8_args(q=0, k=0, v=0, o=0, lse=0, **kw)
        assert sdpa.lib().attn_validate_fwd_fp8(ctypes.byref(a)) == OK
        assert sdpa.lib().attn_fwd_fp8(ctypes.byref(a), None) == OK
    assert vfp8(Lk=0, k=0, v=0) == OK
    assert sdpa.lib().attn_validate_fwd_fp8(None) == NULL


# ------------------------------------------------------- attn_decode_noalloc
@pytest.mark.parametrize("kw,status", [
    (dict(q=0), NULL), (dict(dtype=1), UNSUP), (dict(d=96), UNSUP), (dict(Hkv=3), SHAPE),
    (dict(q=P + 2), LAYOUT), (dict(B=64, Lmax=40_000_000), UNSUP),
])
def test_decode_noalloc_rejections(kw, status):
    """Argument errors come back before the library touches the device."""
    assert sdpa.lib().attn_decode_noalloc(ctypes.byref(dec_args(**kw)), None) == status


def test_decode_noalloc_scratch_limit():
    """Sizes whose workspace exceeds the static scratch are refused with
    ATTN_ERR_SCRATCH, before any device work; the largest decode cache that
    fits at B=64, Hq=32, d=128 is Lmax=15360 (31 pieces per sequence)."""
    L = sdpa.lib()
    lim = sdpa.ATTN_DECODE_NOALLOC_SCRATCH_BYTES
    assert sdpa.attn_decode_workspace_bytes(64, 32, 15360, 128) <= lim
    assert sdpa.attn_decode_workspace_bytes(64, 32, 15361, 128) > lim
    big = dec_args(B=64, Hq=32, Hkv=8, Lmax=15361, d=128)
    assert L.attn_decode_noalloc(ctypes.byref(big), None) == 8
    assert sdpa.status_str(8) != "unknown status"
    assert L.attn_decode_noalloc(ctypes.byref(dec_args(B=0)), None) == OK
