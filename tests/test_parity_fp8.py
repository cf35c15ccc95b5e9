"""FP8 prefill parity: the HIP attn_fwd_fp8 against the float64 CPU oracle fed
the dequantised values of the same e4m3 codes.

The gate is the e4m3 rounding model of parity_util (6 sigma per element,
derived from half an e4m3 step on every probability); properties that hold
exactly (constant values, a single visible key, grouped heads) are checked
bit for bit.  Full-size workloads are compared on sampled heads and rows.
"""
import numpy as np
import pytest
import torch

import scaled_dot_product_qk_amd as sdpa
import workloads as wl
from oracle import sdpa_oracle as orc
from parity_util import check_fp8, fp8_sigmas, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    return torch.device("cuda:0")


def run_gpu(q8, k8, v8, ds, dev, causal, scale=None, **kw):
    o, lse = sdpa.attn_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), ds, causal=causal, scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def oracle_with_sigmas(q8, k8, v8, ds, causal, scale=None):
    o, lse, _, p = orc.attention_forward_fp8(q8, k8, v8, *ds, causal=causal, scale=scale, return_sp=True)
    v = orc.dequantize_e4m3(v8, ds[2])
    B, Hq = o.shape[:2]
    group = Hq // v.shape[1]
    sig_o, sig_l, wabs = np.zeros_like(o), np.zeros(lse.shape), np.zeros_like(o)
    for b in range(B):
        for h in range(Hq):
            sig_o[b, h], sig_l[b, h], wabs[b, h] = fp8_sigmas(p[b, h], v[b, h // group])
    return o, lse, sig_o, sig_l, wabs


def full_check(w, dev, q_mul=1.0, scale=None, label=None, descales=None):
    q8, k8, v8, ds = wl.make_fp8_inputs(w, q_mul=q_mul)
    if descales is not None:
        ds = descales
    o, lse = run_gpu(q8, k8, v8, ds, dev, w.causal, scale)
    o_ref, lse_ref, so, sl, wa = oracle_with_sigmas(q8, k8, v8, ds, w.causal, scale)
    return check_fp8(to_np(o), o_ref, to_np(lse), lse_ref, so, sl, wa, label or w.name)


def fp8w(name, B, Hq, Hkv, Lq, Lk, d, causal, seed):
    return wl.FwdWorkload(name, B, Hq, Hkv, Lq, Lk, d, "fp8", causal, seed)


SMALL = [
    # (B, Hq, Hkv, Lq, Lk)
    (2, 4, 2, 300, 300),   # ragged: 2 full 128-row tiles + 44; 2 key tiles + 44
    (1, 2, 1, 1, 1),
    (1, 3, 3, 129, 129),
    (1, 2, 2, 64, 64),
    (1, 2, 2, 128, 128),
    (2, 8, 1, 257, 257),   # multi-query
    (1, 2, 2, 200, 1000),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL)
def test_fp8_small(dev, d, causal, shape):
    B, Hq, Hkv, Lq, Lk = shape
    full_check(fp8w("small", B, Hq, Hkv, Lq, Lk, d, causal, 500 + Lq + Lk + d),
               dev, label=f"fp8 d{d} causal={causal} {shape}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk", [(77, 500), (300, 64), (130, 1), (500, 77)])
def test_fp8_cross_attention_lengths(dev, d, causal, Lq, Lk):
    full_check(fp8w("cross", 2, 4, 4, Lq, Lk, d, causal, 600 + Lq),
               dev, label=f"fp8 cross d{d} causal={causal} Lq={Lq} Lk={Lk}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_peaky_scores_move_the_running_max(dev, d, causal):
    """Q times 4: a few dominant keys spread over the tiles exercise the
    reference max, the sum guard and the rescale."""
    full_check(fp8w("peaky", 1, 4, 2, 520, 520, d, causal, 700 + d), dev, q_mul=4.0,
               label=f"fp8 peaky d{d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_signed_scale_and_descales(dev, d):
    """A negative total multiplier flips Q's sign bits; V's descale scales O."""
    w = fp8w("signs", 1, 4, 2, 260, 260, d, True, 710 + d)
    full_check(w, dev, scale=-0.09, descales=(-0.011, 0.013, -0.7), label=f"fp8 signs d{d}")
    full_check(w, dev, scale=0.25, descales=(0.02, -0.005, 3.0), label=f"fp8 signs2 d{d}")


def test_fp8_no_keys(dev):
    q8 = torch.randint(0, 0x70, (1, 2, 50, 128), dtype=torch.uint8, device=dev)
    k8 = torch.empty(1, 2, 0, 128, dtype=torch.uint8, device=dev)
    o, lse = sdpa.attn_fwd_fp8(q8, k8, k8, (1.0, 1.0, 1.0))
    torch.cuda.synchronize()
    assert (o == 0).all().item() and torch.isneginf(lse).all().item()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_constant_values_are_returned_exactly(dev, d, causal):
    """Every V row the same: the weights P~ / sum P~ sum to one, so O is
    v_descale * value up to fp32 rounding -- within one bf16 step."""
    w = fp8w("const", 1, 2, 2, 300, 300, d, causal, 720 + d)
    q8, k8, _, ds = wl.make_fp8_inputs(w, q_mul=3.0)
    v8 = torch.full_like(k8, 0x4d)  # 0 1001 101 = 1.625 * 4 = 6.5
    o, _ = run_gpu(q8, k8, v8, ds, dev, causal)
    want = torch.tensor(6.5 * ds[2], dtype=torch.float32).to(torch.bfloat16).float().item()
    got = o.float().cpu()
    ulp = 2.0 ** (np.floor(np.log2(abs(want))) - 7)
    assert (got - want).abs().max().item() <= ulp


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_single_visible_key_is_bit_exact(dev, d):
    """Causal row 0 sees key 0 only: P~ = 1 exactly, so O[0] is the bf16
    rounding of v_descale * value(V[0]) taken in fp32."""
    w = fp8w("row0", 2, 4, 2, 140, 140, d, True, 730 + d)
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    o, lse = run_gpu(q8, k8, v8, ds, dev, True)
    vv = torch.from_numpy(orc.e4m3_decode(v8[:, :, 0].numpy())).float()  # exact in fp32
    want = (vv * torch.tensor(ds[2], dtype=torch.float32)).to(torch.bfloat16)
    want = want.repeat_interleave(2, dim=1)  # query heads 2i, 2i+1 share kv head i
    assert torch.equal(o[:, :, 0].cpu(), want)


def test_fp8_gqa_matches_expanded_heads(dev):
    w = fp8w("gqa", 1, 8, 2, 300, 300, 128, True, 740)
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    o1, l1 = run_gpu(q8, k8, v8, ds, dev, True)
    o2, l2 = run_gpu(q8, k8.repeat_interleave(4, 1), v8.repeat_interleave(4, 1), ds, dev, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_accepts_float8_tensors(dev):
    w = fp8w("f8", 1, 2, 2, 150, 150, 64, False, 750)
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    o1, l1 = run_gpu(q8, k8, v8, ds, dev, False)
    f8 = [t.view(torch.float8_e4m3fn) for t in (q8, k8, v8)]
    o2, l2 = run_gpu(*f8, ds, dev, False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_strided_layouts(dev, causal):
    """[B, L, H, d] storage viewed as [B, H, L, d]; output into a strided view."""
    w = fp8w("strided", 2, 4, 2, 200, 200, 128, causal, 760)
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    qs, ks, vs = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (q8, k8, v8))
    out = torch.zeros(2, 200, 4, 128, dtype=torch.bfloat16, device=dev).transpose(1, 2)
    o, lse = sdpa.attn_fwd_fp8(qs, ks, vs, ds, causal=causal, out=out)
    torch.cuda.synchronize()
    o_ref, lse_ref, so, sl, wa = oracle_with_sigmas(q8, k8, v8, ds, causal)
    check_fp8(to_np(out), o_ref, to_np(lse), lse_ref, so, sl, wa, f"fp8 strided causal={causal}")


def test_fp8_deterministic(dev):
    w = fp8w("det", 1, 4, 2, 700, 700, 128, True, 770)
    q8, k8, v8, ds = (x.to(dev) if torch.is_tensor(x) else x for x in wl.make_fp8_inputs(w))
    a = sdpa.attn_fwd_fp8(q8, k8, v8, ds, causal=True)
    b = sdpa.attn_fwd_fp8(q8, k8, v8, ds, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_output_guard_regions(dev):
    B, H, L, d = 1, 3, 333, 64
    w = fp8w("guard", B, H, H, L, L, d, True, 780)
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    pad = 4096
    obuf = torch.full((pad + B * H * L * d + pad,), 7.0, dtype=torch.bfloat16, device=dev)
    lbuf = torch.full((pad + B * H * L + pad,), 7.0, dtype=torch.float32, device=dev)
    o = obuf[pad:pad + B * H * L * d].view(B, H, L, d)
    lse = lbuf[pad:pad + B * H * L].view(B, H, L)
    sdpa.attn_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), ds, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7).all().item() and (obuf[-pad:] == 7).all().item()
    assert (lbuf[:pad] == 7).all().item() and (lbuf[-pad:] == 7).all().item()
    assert torch.isfinite(o.float()).all().item()


# ------------------------------------------------- the two FP8 workloads
def _sampled(w, dev, heads, rows_of):
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    o, lse = run_gpu(q8, k8, v8, ds, dev, w.causal)
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()
    o, lse = to_np(o), to_np(lse)
    group = w.Hq // w.Hkv
    for h in heads:
        rows = rows_of(h)
        o_ref, lse_ref, _, p = orc.attention_forward_fp8_rows(q8, k8, v8, *ds, 0, h, rows, causal=w.causal,
                                                              return_sp=True)
        v = orc.dequantize_e4m3(v8[0, h // group], ds[2])
        so, sl, wa = fp8_sigmas(p, v)
        check_fp8(o[0, h, rows], o_ref, lse[0, h, rows], lse_ref, so, sl, wa, f"{w.name} head {h}")


def test_workload_fp8_n4096_sampled(dev):
    """All 96 heads run; 6 heads are compared on 512 rows each."""
    w = wl.C7
    rng = np.random.default_rng(11)
    _sampled(w, dev, [0, 17, 40, 63, 80, 95],
             lambda h: np.unique(np.concatenate([np.arange(128), np.arange(w.Lq - 128, w.Lq),
                                                 rng.choice(w.Lq, 256, replace=False)])))


def test_workload_fp8_causal_gqa_n8192_sampled(dev):
    """All 32 query heads run; 8 heads spanning every kv group are compared on
    the first and last tiles, tile edges and random rows."""
    w = wl.C8
    rng = np.random.default_rng(12)
    edges = np.concatenate([np.arange(t * 128 - 2, t * 128 + 2) for t in range(1, w.Lq // 128)])
    _sampled(w, dev, [0, 3, 4, 13, 18, 22, 27, 31],
             lambda h: np.unique(np.concatenate([np.arange(128), np.arange(w.Lq - 128, w.Lq),
                                                 rng.choice(edges, 64, replace=False),
                                                 rng.choice(w.Lq, 128, replace=False)])))
