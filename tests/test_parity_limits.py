"""Parity near the documented size limits: long sequences and large token
strides, where the kernels' 32-bit lane offsets and 64-bit base offsets are
exercised.  Outputs are compared on sampled rows (and keys) that the oracle
computes one by one.
"""
import numpy as np
import pytest
import torch

import scaled_dot_product_qk_amd as sdpa
import workloads as wl
from oracle import sdpa_oracle as orc
from parity_util import bwd_gate, bwd_rounding_bound, check, check_fp8, fp8_sigmas, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    return torch.device("cuda:0")


def _rows(n, rng, extra=64):
    return np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, n // 2, n - 2, n - 1],
                                     rng.choice(n, extra, replace=False)]))


def _strided(t, token_stride, dev):
    """t [B, H, L, d] copied into device memory whose token stride is
    token_stride elements (rows of a much larger buffer)."""
    B, H, L, d = t.shape
    buf = torch.empty(B * H * L * token_stride, dtype=t.dtype, device=dev)
    view = buf.as_strided((B, H, L, d), (H * L * token_stride, L * token_stride, token_stride, 1))
    view.copy_(t.to(dev))
    return view


@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence_prefill(dev, causal):
    """n = 65536 tokens, GQA 2:1, d = 128."""
    n = 65536
    w = wl.FwdWorkload("long", 1, 2, 1, n, n, 128, "bf16", causal, 8001)
    q, k, v = wl.make_fwd_inputs(w)
    o, lse = sdpa.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    rng = np.random.default_rng(8002)
    for h in range(2):
        rows = _rows(n, rng)
        o_ref, lse_ref = orc.attention_forward_rows(q, k, v, 0, h, rows, causal=causal)
        check(o[0, h, rows], o_ref, lse[0, h, rows], lse_ref, "bf16", f"n=65536 causal={causal} head {h}")


def test_long_sequence_fp8(dev):
    n = 32768
    w = wl.FwdWorkload("long8", 1, 2, 1, n, n, 128, "fp8", True, 8003)
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    o, lse = sdpa.attn_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), ds, causal=True)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    rows = _rows(n, np.random.default_rng(8004))
    o_ref, lse_ref, _, p = orc.attention_forward_fp8_rows(q8, k8, v8, *ds, 0, 1, rows, causal=True, return_sp=True)
    so, sl, wa = fp8_sigmas(p, orc.dequantize_e4m3(v8[0, 0], ds[2]))
    check_fp8(o[0, 1, rows], o_ref, lse[0, 1, rows], lse_ref, so, sl, wa, "fp8 n=32768 causal")


def test_long_decode(dev):
    """A 65536-slot cache, lengths at both ends: the longest sequence spans
    several pieces of the balanced split (at least 512 slots each)."""
    w = wl.DecodeWorkload("long_dec", 3, 8, 2, 65536, 128, 1, 65536, "bf16", 8005)
    lens = torch.tensor([65536, 30001, 1], dtype=torch.int32)
    q, kc, vc, lens = wl.make_decode_inputs(w, poison_tail=True, lengths=lens)
    o, lse = sdpa.attn_decode(q.to(dev), kc.to(dev), vc.to(dev), lens.to(dev))
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_decode(q, kc, vc, lens.numpy())
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", "decode Lmax=65536")


@pytest.mark.parametrize("d", [64, 128])
def test_large_token_strides_prefill(dev, d):
    """K and V rows 2^22 elements apart (8 MiB; the copies' per-lane offsets
    span up to 15 rows), Q and O dense."""
    L = 200
    w = wl.FwdWorkload("stride", 1, 2, 2, L, L, d, "bf16", True, 8006 + d)
    q, k, v = wl.make_fwd_inputs(w)
    ks, vs = _strided(k, 1 << 22, dev), _strided(v, 1 << 22, dev)
    o, lse = sdpa.attn_fwd(q.to(dev), ks, vs, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=True)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"K/V token stride 2^22, d={d}")
    del ks, vs


def test_large_token_strides_fp8(dev):
    L = 300
    w = wl.FwdWorkload("stride8", 1, 2, 1, L, L, 64, "fp8", False, 8010)
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    ks, vs = _strided(k8, 1 << 24, dev), _strided(v8, 1 << 24, dev)
    o, lse = sdpa.attn_fwd_fp8(q8.to(dev), ks, vs, ds)
    torch.cuda.synchronize()
    o_ref, lse_ref, _, p = orc.attention_forward_fp8(q8, k8, v8, *ds, return_sp=True)
    vd = orc.dequantize_e4m3(v8, ds[2])
    sig = [fp8_sigmas(p[0, h], vd[0, 0]) for h in range(2)]
    check_fp8(to_np(o), o_ref, to_np(lse), lse_ref, np.stack([s[0] for s in sig])[None],
              np.stack([s[1] for s in sig])[None], np.stack([s[2] for s in sig])[None], "fp8 K/V stride 2^24")
    del ks, vs


def test_large_token_strides_backward(dev):
    """Q, dO, K, V rows 2^24 elements apart (just under the backward's 2^26
    limit for 31-row lane offsets)."""
    L, d = 100, 64
    w = wl.FwdWorkload("stride_bwd", 1, 2, 1, L, L, d, "bf16", True, 8011)
    q, k, v = wl.make_fwd_inputs(w)
    g = torch.Generator().manual_seed(8012)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    st = 1 << 24
    qs, ks, vs, dos = (_strided(x, st, dev) for x in (q, k, v, do))
    o, lse = sdpa.attn_fwd(qs, ks, vs, causal=True)
    dq, dk, dv = sdpa.attn_bwd(qs, ks, vs, o, lse, dos, causal=True)
    torch.cuda.synchronize()
    refs = orc.attention_backward(q, k, v, do, causal=True)
    bounds = bwd_rounding_bound(q, k, v, do, True)
    for name, got, ref, bd in zip(("dq", "dk", "dv"), (dq, dk, dv), refs, bounds):
        worst, mean, finite = bwd_gate(to_np(got), ref, bd)
        print(f"[parity] bwd stride 2^24 {name}: worst_over_gate={worst:.3e} mean_over_gate={mean:.3e}", flush=True)
        assert finite and worst <= 1.0 and mean <= 1.0, (name, worst, mean)
    del qs, ks, vs, dos
