"""Comparison helpers for the GPU-vs-oracle parity tests.

Gates (per output tensor, element by element against the float64 oracle fed
the very same input values):
  bf16 inputs: max |O - O*| <= 2e-2 and mean |O - O*| <= 1e-3;
               LSE: max |LSE - LSE*| <= 1e-3.
  fp32 inputs: max |O - O*| / max |O*| <= 1e-5 (norm-wise relative error);
               LSE: max |LSE - LSE*| / max |LSE*| <= 1e-5.
Rows that see no key must give O == 0 exactly and LSE == -inf.
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
