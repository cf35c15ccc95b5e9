"""The FP8 parity gate itself, on the CPU: arithmetic that rounds every
probability to e4m3 the way the kernel does passes it, and plausible slips of
an FP8 kernel (keys out of order in the P V product, V's descale dropped, the
score multiplier off, probabilities truncated instead of rounded to
3 mantissa bits) fail it.  No GPU, no HIP path: the "kernel" here is numpy
with torch's float8_e4m3fn rounding, fed the same seeded codes."""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import sdpa_oracle as orc
from parity_util import check_fp8, fp8_sigmas


def _e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _emulated(q, k, v, causal, ref_shift=0.0, slip=None):
    """One head: probabilities against the row max shifted by ref_shift (log2
    units, as a reference max below the true one gives), rounded to e4m3,
    summed after rounding; O rounded to bf16."""
    d = q.shape[1]
    s = (q @ k.T) / math.sqrt(d) * (1.7 if slip == "score_multiplier" else 1.0)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > np.arange(q.shape[0])[:, None], -np.inf, s)
    m = s.max(-1, keepdims=True)
    pe = np.exp2((s - m) / math.log(2) + ref_shift)
    if slip == "truncate_to_2_bits":
        e = np.floor(np.log2(np.maximum(pe, 1e-300)))
        pr = np.where(pe > 0, np.floor(pe / 2.0 ** (e - 2)) * 2.0 ** (e - 2), 0.0)
    else:
        pr = _e4m3(pe)
    vv = v
    if slip == "keys_out_of_order":   # swap the two 32-key blocks of every 64-key half
        idx = np.arange(k.shape[0])
        blk = idx // 32
        idx = np.where(blk ^ 1 < (k.shape[0] + 31) // 32, (blk ^ 1) * 32 + idx % 32, idx)
        idx = np.minimum(idx, k.shape[0] - 1)
        vv = v[idx]
    l = pr.sum(-1)
    o = (pr @ vv) / l[:, None]
    lse = m[:, 0] + np.log(l) - ref_shift * math.log(2)
    return torch.from_numpy(o.astype(np.float32)).to(torch.bfloat16).double().numpy(), lse


def _case(causal, slip=None, shift=0.0, q_mul=1.0):
    w = wl.FwdWorkload("gate", 1, 2, 1, 300, 300, 128, "fp8", causal, 801)
    q8, k8, v8, ds = wl.make_fp8_inputs(w, q_mul=q_mul)
    o_ref, lse_ref, _, p = orc.attention_forward_fp8(q8, k8, v8, *ds, causal=causal, return_sp=True)
    v_true = orc.dequantize_e4m3(v8[0, 0], ds[2])
    q = orc.dequantize_e4m3(q8[0, 0], ds[0])
    k = orc.dequantize_e4m3(k8[0, 0], ds[1])
    v = v_true / ds[2] if slip == "v_descale_dropped" else v_true
    o, lse = _emulated(q, k, v, causal, shift, slip)
    so, sl, wa = fp8_sigmas(p[0, 0], v_true)
    return check_fp8(o, o_ref[0, 0], lse, lse_ref[0, 0], so, sl, wa, f"emulated {slip}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shift,q_mul", [(0.0, 1.0), (5.3, 1.0), (7.9, 4.0)])
def test_rounded_arithmetic_passes(causal, shift, q_mul):
    r = _case(causal, None, shift, q_mul)
    assert r["worst"] < 0.95 and r["mean_ratio"] < 0.8


@pytest.mark.parametrize("slip", ["keys_out_of_order", "v_descale_dropped", "score_multiplier", "truncate_to_2_bits"])
def test_slips_fail(slip):
    with pytest.raises(AssertionError):
        _case(True, slip)
