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


ROUND_BF16 = 2.0 ** -8  # |bf16(x) - x| <= 2^-8 |x|: half an ulp, round to nearest even
ROUND_BF16_MEAN = 2.0 ** -9  # mean rounding error of bf16 (ulp / 4), relative


def bwd_gate(got, ref, bound=None):
    """The backward's gate for one gradient tensor against the float64
    oracle: (worst element's error over its allowance, mean error over the
    mean allowance, all values finite).  Allowance per element: the stated
    bf16 tolerance 2e-2, plus the rounding of the result to bf16 (2^-8 |ref|,
    which gradients cannot avoid since, unlike O, they are not bounded by the
    values' range), plus `bound` where given (bwd_rounding_bound: six
    standard deviations of the method's own roundings inside the sums).
    Mean: 1e-3 + 2^-9 mean |ref|, plus the mean standard deviation (bound / 6)
    where a bound is given, as the FP8 mean gate takes the mean sigma."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    a = np.abs(ref)
    bd = 0.0 if bound is None else np.asarray(bound, np.float64)
    allow = BF16_MAX_ABS + ROUND_BF16 * a + bd
    worst = float((d / allow).max()) if d.size else 0.0
    mean_allow = BF16_MEAN_ABS + ROUND_BF16_MEAN * a.mean() + (float(np.mean(bd)) / 6.0 if bound is not None else 0.0)
    mean = float(d.mean() / mean_allow) if d.size else 0.0
    return worst, mean, bool(np.isfinite(got).all())


def bwd_rounding_bound(q, k, v, do, causal: bool, scale=None):
    """Per-element allowance for what the backward's own roundings move dQ,
    dK and dV by (part of the gate, not a reference value).

    The backward of "Flash Attention原理：分块计算与重计算" (cnblogs), section
    五, as the kernel runs it: D = rowsum(dO * O) is formed from the bf16 O
    that the forward returned (O itself a product of bf16-rounded
    probabilities), and dS and P are rounded to bf16 before their products.
    In a gradient that is a sum with much cancellation (a key that every
    query sees, causal) these move the result by far more than its own
    output rounding.  Each rounding is taken as an independent error,
    uniform within +-u |x| (u = 2^-8, half an ulp), so of variance at most
    s2 x^2 with s2 = u^2 / 3.  From the float64 quantities of the
    definition, to first order (fp32 accumulation and the exponential's
    error are orders smaller):
        var D_q     = s2 (sum_c dO_qc^2 O_qc^2 + sum_j P_qj^2 dP_qj^2)
                      (O's output rounding; the forward's rounding of P)
        dS_qj moves by -P_qj dD_q (one dD_q for the whole row) plus its own
                      rounding, variance s2 dS_qj^2
        var dQ_qc   = scale^2 (var D_q (sum_j P_qj K_jc)^2 + s2 sum_j dS_qj^2 K_jc^2)
        var dK_jc   = scale^2 sum_q (P_qj^2 var D_q + s2 dS_qj^2) Q_qc^2
        var dV_jc   = s2 sum_q P_qj^2 dO_qc^2
    (dK and dV summed over the kv head's query heads).  The allowance is six
    standard deviations, as for the FP8 probabilities.  Causal is top-left
    (query i sees keys j <= i).  Returns arrays shaped like dq, dk, dv."""
    def f64(t):
        return np.asarray(to_np(t) if hasattr(t, "detach") else t, np.float64)
    q, k, v, do = f64(q), f64(k), f64(v), f64(do)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    sc = d ** -0.5 if scale is None else scale
    s2 = ROUND_BF16 ** 2 / 3.0
    vq, vk, vv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if Lq > 0 and Lk > 0:
        vis = np.tril(np.ones((Lq, Lk), bool)) if causal else np.ones((Lq, Lk), bool)
        for b in range(B):
            for h in range(Hq):
                kh, vh, qh, doh = k[b, h // group], v[b, h // group], q[b, h], do[b, h]
                s = np.where(vis, sc * (qh @ kh.T), -np.inf)
                p = np.where(vis, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
                p /= p.sum(axis=1, keepdims=True)
                o = p @ vh
                dp = doh @ vh.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                var_d = s2 * ((doh ** 2 * o ** 2).sum(axis=1) + (p ** 2 * dp ** 2).sum(axis=1))
                vq[b, h] = sc ** 2 * (var_d[:, None] * (p @ kh) ** 2 + s2 * (ds ** 2) @ kh ** 2)
                vk[b, h // group] += sc ** 2 * (p ** 2 * var_d[:, None] + s2 * ds ** 2).T @ qh ** 2
                vv[b, h // group] += s2 * (p ** 2).T @ doh ** 2
    return 6.0 * np.sqrt(vq), 6.0 * np.sqrt(vk), 6.0 * np.sqrt(vv)
