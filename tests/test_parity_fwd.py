"""Prefill parity: the HIP attn_fwd against the float64 CPU oracle.

Small and medium shapes are compared in full; the four prefill workloads at
their real sizes are compared on whole sampled heads or sampled rows that the
oracle computes one by one.  All inputs are seeded; the oracle receives the
exact values the GPU reads.
"""
import numpy as np
import pytest
import torch

import scaled_dot_product_qk_amd as sdpa
import workloads as wl
from oracle import sdpa_oracle as orc
from parity_util import check, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    return torch.device("cuda:0")


def run_gpu(q, k, v, dev, causal, scale=None):
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = sdpa.attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def full_check(w, dev, q_mul=1.0, scale=None, label=None):
    q, k, v = wl.make_fwd_inputs(w, q_mul=q_mul)
    o, lse = run_gpu(q, k, v, dev, w.causal, scale)
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=w.causal, scale=scale)
    return check(to_np(o), o_ref, to_np(lse), lse_ref, w.dtype, label or w.name)


SMALL = [
    # (B, Hq, Hkv, Lq, Lk)
    (2, 4, 2, 300, 300),   # ragged: 2 full 128-row tiles + 44, 4 key tiles + 44
    (1, 2, 1, 1, 1),
    (1, 3, 3, 129, 129),
    (1, 2, 2, 64, 64),
    (2, 8, 1, 257, 257),   # multi-query
]


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL)
def test_bf16_small(dev, d, causal, shape):
    B, Hq, Hkv, Lq, Lk = shape
    w = wl.FwdWorkload("small", B, Hq, Hkv, Lq, Lk, d, "bf16", causal, 100 + Lq + d)
    full_check(w, dev, label=f"bf16 d{d} causal={causal} {shape}")


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_small(dev, d, causal):
    w = wl.FwdWorkload("small", 2, 4, 2, 300, 300, d, "f32", causal, 200 + d)
    full_check(w, dev, label=f"f32 d{d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lq,Lk", [(77, 500), (300, 64), (130, 1)])
def test_cross_attention_lengths(dev, d, Lq, Lk):
    w = wl.FwdWorkload("cross", 2, 4, 4, Lq, Lk, d, "bf16", False, 300 + Lq)
    full_check(w, dev, label=f"cross d{d} Lq={Lq} Lk={Lk}")


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_peaky_scores_move_the_running_max(dev, d, causal):
    """Q scaled by 4 gives score rows with a few dominant keys spread over
    the tiles, so the online max and the rescale are exercised."""
    w = wl.FwdWorkload("peaky", 1, 4, 2, 520, 520, d, "bf16", causal, 400 + d)
    full_check(w, dev, q_mul=4.0, label=f"peaky d{d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_increasing_scores(dev, causal):
    """Scores grow along the key axis, so the row max changes on every tile."""
    B, H, L, d = 1, 2, 640, 64
    g = torch.Generator().manual_seed(5)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = (u * 20.0).expand(B, H, L, d).clone()
    ramp = torch.linspace(0, 6, L)[:, None] * u[None, :]
    k = (ramp + 0.05 * torch.randn(L, d, generator=g)).expand(B, H, L, d).clone()
    v = torch.randn(B, H, L, d, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    o, lse = run_gpu(q, k, v, dev, causal)
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=causal)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"increasing causal={causal}")


def test_explicit_scale(dev):
    w = wl.FwdWorkload("scale", 1, 2, 2, 200, 200, 64, "bf16", True, 9)
    full_check(w, dev, scale=0.37, label="scale=0.37")


def test_no_keys(dev):
    q = torch.randn(1, 2, 50, 64).to(torch.bfloat16).to(dev)
    k = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    o, lse = sdpa.attn_fwd(q, k, k)
    torch.cuda.synchronize()
    assert (o == 0).all().item() and torch.isneginf(lse).all().item()


def test_empty_query_is_noop(dev):
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    k = torch.randn(1, 2, 10, 64).to(torch.bfloat16).to(dev)
    o, lse = sdpa.attn_fwd(q, k, k)
    assert o.numel() == 0 and lse.numel() == 0


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_output_rows_past_lq_untouched(dev, d, causal):
    """The epilogue stores whole rows (staged through LDS at d = 64 and 128):
    with Lq = 200 the last query tile holds rows past Lq, and O is a view into
    a larger buffer whose other rows and heads carry a sentinel that must
    survive."""
    B, Hq, Hkv, L = 2, 4, 2, 200
    w = wl.FwdWorkload("rows_past_lq", B, Hq, Hkv, L, L, d, "bf16", causal, 1700 + d)
    q, k, v = wl.make_fwd_inputs(w)
    sentinel = -7.0
    big = torch.full((B, Hq + 1, L + 64, d), sentinel, dtype=torch.bfloat16, device=dev)
    out = big[:, 1:, :L]
    o, lse = sdpa.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, out=out)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=causal)
    check(to_np(out), o_ref, to_np(lse), lse_ref, "bf16", f"rows past Lq d{d} causal={causal}")
    assert (big[:, 0] == sentinel).all().item()
    assert (big[:, 1:, L:] == sentinel).all().item()


@pytest.mark.parametrize("causal", [False, True])
def test_strided_layouts(dev, causal):
    """[B, L, H, d] storage viewed as [B, H, L, d]; output into a strided view."""
    B, Hq, Hkv, L, d = 2, 4, 2, 200, 128
    g = torch.Generator().manual_seed(11)
    qs = torch.randn(B, L, Hq, d, generator=g).to(torch.bfloat16)
    ks = torch.randn(B, L, Hkv, d, generator=g).to(torch.bfloat16)
    vs = torch.randn(B, L, Hkv, d, generator=g).to(torch.bfloat16)
    qd, kd, vd = (t.to(dev).transpose(1, 2) for t in (qs, ks, vs))
    out = torch.zeros(B, L, Hq, d, dtype=torch.bfloat16, device=dev).transpose(1, 2)
    o, lse = sdpa.attn_fwd(qd, kd, vd, causal=causal, out=out)
    torch.cuda.synchronize()
    q, k, v = (t.transpose(1, 2) for t in (qs, ks, vs))
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=causal)
    check(to_np(out), o_ref, to_np(lse), lse_ref, "bf16", f"strided causal={causal}")


def test_gqa_matches_expanded_heads_on_gpu(dev):
    w = wl.FwdWorkload("gqa", 1, 8, 2, 300, 300, 128, "bf16", True, 12)
    q, k, v = wl.make_fwd_inputs(w)
    o1, l1 = run_gpu(q, k, v, dev, True)
    o2, l2 = run_gpu(q, k.repeat_interleave(4, 1), v.repeat_interleave(4, 1), dev, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic(dev):
    w = wl.FwdWorkload("det", 1, 4, 2, 700, 700, 80, "bf16", True, 13)
    q, k, v = (t.to(dev) for t in wl.make_fwd_inputs(w))
    a = sdpa.attn_fwd(q, k, v, causal=True)
    b = sdpa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_output_guard_regions(dev):
    """Writes stay inside O and LSE: canaries around both are untouched."""
    B, H, L, d = 1, 3, 333, 80
    w = wl.FwdWorkload("guard", B, H, H, L, L, d, "bf16", True, 14)
    q, k, v = (t.to(dev) for t in wl.make_fwd_inputs(w))
    pad = 4096
    obuf = torch.full((pad + B * H * L * d + pad,), 7.0, dtype=torch.bfloat16, device=dev)
    lbuf = torch.full((pad + B * H * L + pad,), 7.0, dtype=torch.float32, device=dev)
    o = obuf[pad:pad + B * H * L * d].view(B, H, L, d)
    lse = lbuf[pad:pad + B * H * L].view(B, H, L)
    sdpa.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7).all().item() and (obuf[-pad:] == 7).all().item()
    assert (lbuf[:pad] == 7).all().item() and (lbuf[-pad:] == 7).all().item()
    assert torch.isfinite(o.float()).all().item()


def test_kernel_name_reports_native_d80(dev):
    q = torch.zeros(1, 1, 16, 80, dtype=torch.bfloat16, device=dev)
    assert sdpa.kernel_name(q, q, q, causal=True) == "attn_fwd_bf16_d80_causal"


# ------------------------------------------------- the four prefill workloads
def test_workload_fwd_f32_n256(dev):
    full_check(wl.C1, dev)


def test_workload_fwd_bf16_n4096_sampled_heads(dev):
    """All 96 heads run; 6 whole heads (incl. the first and last) are compared."""
    w = wl.C2
    q, k, v = wl.make_fwd_inputs(w)
    o, lse = run_gpu(q, k, v, dev, False)
    heads = [0, 17, 40, 63, 80, 95]
    o_ref, lse_ref = orc.attention_forward(q[:, heads], k[:, heads], v[:, heads])
    check(to_np(o[:, heads]), o_ref, to_np(lse[:, heads]), lse_ref, "bf16", w.name)
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()


def test_workload_fwd_causal_d80_full(dev):
    full_check(wl.C3, dev)


def test_workload_fwd_causal_gqa_n8192_sampled_rows(dev):
    """All 32 query heads run; 8 heads spanning every kv group are compared on
    384 rows each: the first and last tiles, tile edges and random rows."""
    w = wl.C4
    q, k, v = wl.make_fwd_inputs(w)
    o, lse = run_gpu(q, k, v, dev, True)
    o_np, lse_np = to_np(o), to_np(lse)
    rng = np.random.default_rng(0)
    fixed = [0, 1, 2, 63, 64, 127, 128, 129, 4095, 4096, 8063, 8064, 8190, 8191]
    heads = [0, 3, 5, 12, 18, 23, 26, 31]
    os_, osr, ls, lsr = [], [], [], []
    for h in heads:
        rows = sorted(set(fixed) | set(rng.choice(w.Lq, 384 - len(fixed), replace=False).tolist()))
        orow, lrow = orc.attention_forward_rows(q, k, v, 0, h, rows, causal=True)
        os_.append(o_np[0, h, rows]); osr.append(orow)
        ls.append(lse_np[0, h, rows]); lsr.append(lrow)
    check(np.concatenate(os_), np.concatenate(osr), np.concatenate(ls), np.concatenate(lsr),
          "bf16", w.name)
    assert np.isfinite(o_np).all() and np.isfinite(lse_np).all()


# Head_dim 64 without causal masking or a mask runs a schedule that pipelines
# the two key halves across tiles, rotates through three LDS buffers, and
# hands the last one or two unmasked tiles to the masked loop.  These key
# counts give 1 to 7 key tiles, full and ragged, so every position of the
# three-buffer rotation is both the last tile and the masked tail.
PIPE_LK = [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 320, 383, 384, 385, 448]


@pytest.mark.parametrize("lk", PIPE_LK)
def test_bf16_d64_pipeline_tiles(dev, lk):
    w = wl.FwdWorkload("pipe", 1, 3, 1, 150, lk, 64, "bf16", False, 7000 + lk)
    full_check(w, dev, label=f"bf16 d64 pipelined Lk={lk}")


@pytest.mark.parametrize("lk", [64, 192, 448])
def test_bf16_d64_pipeline_rescale(dev, lk):
    """Scores three times larger: the reference max moves (and O is rescaled)
    in later tiles, between pipelined halves."""
    w = wl.FwdWorkload("pipe_big", 1, 2, 2, 200, lk, 64, "bf16", False, 7100 + lk)
    full_check(w, dev, q_mul=3.0, label=f"bf16 d64 pipelined q x3 Lk={lk}")


def test_bf16_d64_pipeline_rising_scores(dev):
    """Keys whose scores grow along the sequence: the reference max moves up
    in almost every tile, so O is rescaled while the previous half's products
    are still in flight in the pipelined schedule."""
    w = wl.FwdWorkload("pipe_rise", 1, 2, 1, 130, 448, 64, "bf16", False, 7200)
    q, k, v = wl.make_fwd_inputs(w)
    ramp = torch.linspace(0.5, 4.0, w.Lk).view(1, 1, w.Lk, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    q = (q.float().abs() * torch.sign(k.float().mean(dim=2, keepdim=True))).to(torch.bfloat16)
    o, lse = run_gpu(q, k, v, dev, causal=False)
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=False)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", "bf16 d64 pipelined rising scores")
