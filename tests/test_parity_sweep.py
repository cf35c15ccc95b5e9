"""Randomised parity sweep: every entry point on seeded random shapes.

Each case draws its sizes from a seeded generator (case index = seed), so a
failure names a reproducible configuration.  Sizes stay small enough for the
float64 oracle (a few hundred rows and keys) but cross tile edges, grouped
heads, cross-attention lengths, scales of both signs and strided layouts at
random.  The gates are the ones the dedicated parity tests use.
"""
import numpy as np
import pytest
import torch

import scaled_dot_product_qk_amd as sdpa
import workloads as wl
from oracle import sdpa_oracle as orc
from parity_util import bwd_gate, bwd_rounding_bound, check, check_fp8, fp8_sigmas, to_np

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    return torch.device("cuda:0")


def _shape(r, d_choices):
    d = int(r.choice(d_choices))
    Hkv = int(r.integers(1, 4))
    group = int(r.choice([1, 2, 4]))
    B = int(r.integers(1, 3))
    Lq = int(r.integers(1, 400))
    Lk = int(r.integers(1, 400)) if r.random() < 0.5 else Lq
    causal = bool(r.random() < 0.5)
    scale = None if r.random() < 0.5 else float(r.choice([-1, 1]) * r.uniform(0.02, 0.3))
    return d, B, Hkv * group, Hkv, Lq, Lk, causal, scale


def _maybe_strided(t, r, dev):
    """Half the time, store [B, L, H, d] and view it as [B, H, L, d]."""
    if r.random() < 0.5:
        return t.transpose(1, 2).contiguous().to(dev).transpose(1, 2)
    return t.to(dev)


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_fwd(dev, case):
    r = np.random.default_rng(5000 + case)
    d, B, Hq, Hkv, Lq, Lk, causal, scale = _shape(r, [64, 80, 128])
    dtype = "f32" if r.random() < 0.25 else "bf16"
    w = wl.FwdWorkload("sweep", B, Hq, Hkv, Lq, Lk, d, dtype, causal, 6000 + case)
    q, k, v = wl.make_fwd_inputs(w, q_mul=float(r.choice([1.0, 3.0])))
    o, lse = sdpa.attn_fwd(_maybe_strided(q, r, dev), _maybe_strided(k, r, dev), _maybe_strided(v, r, dev),
                           causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=causal, scale=scale)
    check(to_np(o), o_ref, to_np(lse), lse_ref, dtype, f"sweep fwd {case}: {w}, scale={scale}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_fwd_fp8(dev, case):
    r = np.random.default_rng(5100 + case)
    d, B, Hq, Hkv, Lq, Lk, causal, scale = _shape(r, [64, 128])
    w = wl.FwdWorkload("sweep8", B, Hq, Hkv, Lq, Lk, d, "fp8", causal, 6100 + case)
    q8, k8, v8, ds = wl.make_fp8_inputs(w, q_mul=float(r.choice([1.0, 3.0])))
    ds = tuple(x * float(r.choice([-1, 1])) * float(r.uniform(0.5, 2.0)) for x in ds)
    o, lse = sdpa.attn_fwd_fp8(_maybe_strided(q8, r, dev), _maybe_strided(k8, r, dev), _maybe_strided(v8, r, dev),
                               ds, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref, _, p = orc.attention_forward_fp8(q8, k8, v8, *ds, causal=causal, scale=scale, return_sp=True)
    vd = orc.dequantize_e4m3(v8, ds[2])
    sig_o, sig_l, wabs = np.zeros_like(o_ref), np.zeros(lse_ref.shape), np.zeros_like(o_ref)
    for b in range(B):
        for h in range(Hq):
            sig_o[b, h], sig_l[b, h], wabs[b, h] = fp8_sigmas(p[b, h], vd[b, h // (Hq // Hkv)])
    check_fp8(to_np(o), o_ref, to_np(lse), lse_ref, sig_o, sig_l, wabs, f"sweep fp8 {case}: {w}, scale={scale}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_varlen(dev, case):
    r = np.random.default_rng(5200 + case)
    d = int(r.choice([64, 80, 128]))
    Hkv = int(r.integers(1, 3)) * (8 if r.random() < 0.3 else 1)
    group = int(r.choice([1, 2, 4]))
    nseq = int(r.integers(1, 6))
    causal = bool(r.random() < 0.5)
    lens_q = r.integers(0, 300, nseq)
    lens_q[0] = max(int(lens_q[0]), 1)  # at least one query row
    lens_k = lens_q if r.random() < 0.5 else r.integers(0, 300, nseq)
    w = wl.VarlenWorkload("sweepv", nseq, Hkv * group, Hkv, 0, 0, d, "bf16", causal, 6200 + case)
    q, k, v, cu_q, cu_k = wl.make_varlen_inputs(w, lens_q=lens_q, lens_k=lens_k)
    max_q = int(lens_q.max())
    o, lse = sdpa.attn_fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev), max_q,
                                  causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_forward_varlen(q, k, v, cu_q.tolist(), cu_k.tolist(), causal=causal)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"sweep varlen {case}: {w.Hq}/{w.Hkv} d{d} "
          f"lens_q={lens_q.tolist()} lens_k={np.asarray(lens_k).tolist()} causal={causal}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_masked(dev, case):
    r = np.random.default_rng(5300 + case)
    d, B, Hq, Hkv, Lq, _, causal, scale = _shape(r, [64, 80, 128])
    kind = "bool" if r.random() < 0.5 else "add"
    Lk = int(r.integers(1, 25)) * 16
    w = wl.FwdWorkload("sweepm", B, Hq, Hkv, Lq, Lk, d, "bf16", causal, 6300 + case)
    q, k, v = wl.make_fwd_inputs(w)
    mshape = (B if r.random() < 0.5 else 1, Hq if r.random() < 0.5 else 1, Lq, Lk)
    m = wl.make_mask(mshape, kind, 6400 + case, keep=float(r.uniform(0.3, 0.95)))
    o, lse = sdpa.attn_fwd_masked(q.to(dev), k.to(dev), v.to(dev), m.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=causal, scale=scale, attn_mask=m)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"sweep masked {case}: {w} {kind} {mshape}")


def _grad_check(name, got, ref, label, bound):
    """The backward's gate (parity_util.bwd_gate) with the allowance for the
    method's own roundings, as in the full comparisons of test_parity_bwd."""
    worst, mean, finite = bwd_gate(got, ref, bound)
    d = np.abs(np.asarray(got, np.float64) - ref)
    print(f"[parity] {label} {name}: max_abs={d.max() if d.size else 0:.3e} mean_abs={d.mean() if d.size else 0:.3e} "
          f"worst_over_gate={worst:.3e} mean_over_gate={mean:.3e}", flush=True)
    assert finite, f"non-finite values in {name}"
    assert worst <= 1.0 and mean <= 1.0, (name, worst, mean)


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_bwd(dev, case):
    r = np.random.default_rng(5400 + case)
    d, B, Hq, Hkv, Lq, Lk, causal, scale = _shape(r, [64, 80, 128])
    Lq, Lk = min(Lq, 260), min(Lk, 260)
    w = wl.FwdWorkload("sweepb", B, Hq, Hkv, Lq, Lk, d, "bf16", causal, 6500 + case)
    q, k, v = wl.make_fwd_inputs(w)
    g = torch.Generator().manual_seed(6600 + case)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = sdpa.attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = sdpa.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward(q, k, v, do, causal=causal, scale=scale)
    bq, bk, bv = bwd_rounding_bound(q, k, v, do, causal, scale=scale)
    label = f"sweep bwd {case}: {w}, scale={scale}"
    _grad_check("dq", to_np(dq), rq, label, bq)
    _grad_check("dk", to_np(dk), rk, label, bk)
    _grad_check("dv", to_np(dv), rv, label, bv)


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_decode(dev, case):
    r = np.random.default_rng(5500 + case)
    d = int(r.choice([64, 80, 128]))
    Hkv = int(r.integers(1, 4))
    group = int(r.choice([1, 2, 4, 8, 20]))
    B = int(r.integers(1, 7))
    Lmax = int(r.integers(1, 2000))
    w = wl.DecodeWorkload("sweepd", B, Hkv * group, Hkv, Lmax, d, 0, Lmax, "bf16", 6700 + case)
    lens = torch.as_tensor(r.integers(0, Lmax + 1, B), dtype=torch.int32)
    q, kc, vc, lens = wl.make_decode_inputs(w, poison_tail=True, lengths=lens)
    scale = None if r.random() < 0.5 else float(r.uniform(0.02, 0.3))
    o, lse = sdpa.attn_decode(q.to(dev), kc.to(dev), vc.to(dev), lens.to(dev), scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_decode(q, kc, vc, lens.numpy(), scale=scale)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"sweep decode {case}: {w} lens={lens.tolist()}")
