"""Comparison helpers for the GPU-vs-oracle parity tests.

Gates (per output tensor, element by element against the float64 oracle fed
the very same input values):
  bf16 inputs: max |O - O*| <= 2e-2 and mean |O - O*| <= 1e-3;
               LSE: max |LSE - LSE*| <= 1e-3.
  fp32 inputs: max |O - O*| / max |O*| <= 1e-5 (norm-wise relative error);
               LSE: max |LSE - LSE*| / max |LSE*| <= 1e-5.
Rows that see no key must give O == 0 exactly and LSE == -inf.

FP8 inputs (attn_fwd_fp8) have no fixed tolerance: the kernel rounds every
probability to e4m3 before the P V product, so the gate follows from that
rounding.  In units of its row maximum a probability p is rounded with an
error of at most half a step: 2^-4 p in the normal range, 2^-10 below 2^-6;
taken as uniform and independent across keys, its standard deviation is at
most s_j = max(2^-4 p_j, 2^-10) / sqrt(3) (0 for keys with p = 0).  With the
normaliser summing the same rounded values, to first order
    dO_c = sum_j dp_j (v_jc - O_c) / l,   dLSE = sum_j dp_j / l,
so sigma_O = sqrt(sum_j s_j^2 (v_jc - O_c)^2) / l and sigma_LSE =
sqrt(sum_j s_j^2) / l.  Gates, element by element against the oracle:
  |O - O*| <= 6 sigma_O + 2^-8 |O*| (bf16 output rounding)
              + 2^-12 sum_j w_j |v_jc| (fp32 accumulation of the products);
  mean |O - O*| <= mean of (sigma_O + 2^-8 |O*| + 2^-12 sum_j w_j |v_jc|);
  |LSE - LSE*| <= 6 sigma_LSE + 1e-5 max(1, |LSE*|).
"""
import numpy as np

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 1e-3
BF16_LSE_MAX_ABS = 1e-3
F32_REL = 1e-5


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def errors(o, o_ref, lse, lse_ref):
    o, lse = np.asarray(o, np.float64), np.asarray(lse, np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), "LSE finiteness differs from the oracle"
    assert np.isfinite(o).all(), "non-finite values in O"
    d = np.abs(o - o_ref)
    dl = np.abs(lse[fin] - lse_ref[fin]) if fin.any() else np.zeros(1)
    return dict(max_abs=float(d.max()) if d.size else 0.0,
                mean_abs=float(d.mean()) if d.size else 0.0,
                rel=float(d.max() / max(np.abs(o_ref).max(), 1e-30)) if d.size else 0.0,
                lse_max_abs=float(dl.max()),
                lse_rel=float(dl.max() / max(np.abs(lse_ref[fin]).max(), 1e-30)) if fin.any() else 0.0)


def check(o, o_ref, lse, lse_ref, dtype: str, label: str = ""):
    e = errors(o, o_ref, lse, lse_ref)
    print(f"[parity] {label} {dtype}: " + " ".join(f"{k}={v:.3e}" for k, v in e.items()), flush=True)
    if dtype == "bf16":
        assert e["max_abs"] <= BF16_MAX_ABS, e
        assert e["mean_abs"] <= BF16_MEAN_ABS, e
        assert e["lse_max_abs"] <= BF16_LSE_MAX_ABS, e
    else:
        assert e["rel"] <= F32_REL, e
        assert e["lse_rel"] <= F32_REL, e
    return e


FP8_SIGMAS = 6.0


def fp8_sigmas(p, v):
    """p [rows, Lk] oracle probabilities of one head, v [Lk, d] its dequantised
    values -> (sigma_O [rows, d], sigma_LSE [rows], sum_j w_j |v_jc| [rows, d])."""
    p = np.asarray(p, np.float64)
    v = np.asarray(v, np.float64)
    pmax = p.max(axis=-1, keepdims=True)
    pm = np.divide(p, pmax, out=np.zeros_like(p), where=pmax > 0)
    sd = np.where(p > 0, np.maximum(pm * 2.0 ** -4, 2.0 ** -10), 0.0) / np.sqrt(3.0)
    l = pm.sum(axis=-1)
    l_safe = np.where(l > 0, l, 1.0)
    o = p @ v
    s2 = sd * sd
    var = s2 @ (v * v) - 2.0 * (s2 @ v) * o + s2.sum(axis=-1, keepdims=True) * o * o
    sig_o = np.sqrt(np.maximum(var, 0.0)) / l_safe[:, None]
    sig_l = np.sqrt(s2.sum(axis=-1)) / l_safe
    return sig_o, sig_l, p @ np.abs(v)


def check_fp8(o, o_ref, lse, lse_ref, sig_o, sig_l, wabs, label: str = ""):
    o, lse = np.asarray(o, np.float64), np.asarray(lse, np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), "LSE finiteness differs from the oracle"
    assert np.isfinite(o).all(), "non-finite values in O"
    assert (o[~fin] == 0).all(), "rows without keys must give O = 0"
    err = np.abs(o - o_ref)
    slack = 2.0 ** -8 * np.abs(o_ref) + 2.0 ** -12 * wabs
    gate = FP8_SIGMAS * sig_o + slack
    el = np.abs(lse[fin] - lse_ref[fin])
    gl = FP8_SIGMAS * sig_l[fin] + 1e-5 * np.maximum(1.0, np.abs(lse_ref[fin]))
    worst = float((err / np.maximum(gate, 1e-30)).max()) if err.size else 0.0
    worst_l = float((el / gl).max()) if el.size else 0.0
    mean_ratio = float(err.mean() / max((sig_o + slack).mean(), 1e-30)) if err.size else 0.0
    print(f"[parity] {label} fp8: max_abs={err.max() if err.size else 0:.3e} mean_abs={err.mean() if err.size else 0:.3e} "
          f"worst/gate={worst:.3f} mean/expected={mean_ratio:.3f} lse_worst/gate={worst_l:.3f}", flush=True)
    assert worst <= 1.0, f"O outside the e4m3 rounding gate ({worst:.3f})"
    assert mean_ratio <= 1.0, f"mean O error above the rounding model ({mean_ratio:.3f})"
    assert worst_l <= 1.0, f"LSE outside the e4m3 rounding gate ({worst_l:.3f})"
    return dict(worst=worst, mean_ratio=mean_ratio, worst_lse=worst_l)
