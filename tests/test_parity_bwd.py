"""Backward parity: the HIP attn_bwd against the float64 CPU oracle.

The GPU forward supplies O and LSE exactly as a caller's would; the oracle's
gradients come from the bf16 input values widened to float64.  Small and
medium shapes are compared in full; the causal GQA n=8192 d=128 workload at
its real size on sampled query rows and keys.

Gate, element by element: |got - ref| <= 2e-2 + 2^-8 |ref|, and per tensor
mean |got - ref| <= 1e-3 + 2^-9 mean |ref|.  The constant terms are the
stated bf16 tolerance.  The other terms are the rounding of the result to
bf16, which the gradients cannot avoid: unlike O they are not bounded by the
values' range (a kv head's dV sums the output gradients of all its query rows
and heads, |dV| reaches 10-13 here), and round-to-nearest-even to bf16 moves
a value x by at most half an ulp, <= 2^-8 |x|, by ulp/4 <= 2^-9 |x| on
average.  So an element of magnitude below ~1 is held to the stated 2e-2,
and only the part of the error that output rounding explains is added above
that.  Where the gradients are compared in full, each element also gets the
allowance of parity_util.bwd_rounding_bound: six standard deviations of what
the method's own roundings (D formed from the bf16 O, dS and P rounded to
bf16 before their products) move it by.  In a sum with much cancellation (a
key that every query sees, causal) those move a gradient by more than its
output rounding; a float64 emulation of exactly that arithmetic reproduces
such elements to the last bf16 bit (tests/test_bwd_gate.py).  The sampled
comparisons at full size keep the plain gate.
"""
import numpy as np
import pytest
import torch

import scaled_dot_product_qk_amd as sdpa
import workloads as wl
from oracle import sdpa_oracle as orc
from parity_util import bwd_gate, bwd_rounding_bound, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    return torch.device("cuda:0")


def grad_check(name, got, ref, label, bound=None):
    worst, mean, finite = bwd_gate(got, ref, bound)
    d = np.abs(np.asarray(got, np.float64) - ref)
    print(f"[parity] {label} {name}: max_abs={d.max() if d.size else 0.0:.3e} "
          f"mean_abs={d.mean() if d.size else 0.0:.3e} worst_over_gate={worst:.3e} mean_over_gate={mean:.3e}"
          + (" (with rounding allowance)" if bound is not None else ""), flush=True)
    assert finite, f"non-finite values in {name}"
    assert worst <= 1.0, (name, label, worst)
    assert mean <= 1.0, (name, label, mean)


def full_check(dq, dk, dv, q, k, v, do, causal, label):
    """Full comparison of the three gradients against the oracle, each element
    allowed the method's own rounding in addition (bwd_rounding_bound)."""
    rq, rk, rv = orc.attention_backward(q, k, v, do, causal=causal)
    bq, bk, bv = bwd_rounding_bound(q, k, v, do, causal)
    grad_check("dq", to_np(dq), rq, label, bq)
    grad_check("dk", to_np(dk), rk, label, bk)
    grad_check("dv", to_np(dv), rv, label, bv)


def inputs(w, seed_do):
    q, k, v = wl.make_fwd_inputs(w)
    g = torch.Generator().manual_seed(seed_do)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)
    return q, k, v, do


def run_gpu(q, k, v, do, dev, causal):
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = sdpa.attn_fwd(qd, kd, vd, causal=causal)
    dq, dk, dv = sdpa.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal)
    torch.cuda.synchronize()
    return dq, dk, dv


SHAPES = [
    # (B, Hq, Hkv, Lq, Lk)
    (2, 4, 2, 300, 300),   # ragged: query and key tiles of 128 with a 44-row tail
    (1, 2, 1, 1, 1),
    (1, 4, 4, 129, 129),
    (2, 8, 1, 257, 257),   # multi-query: dK, dV summed over 8 heads
    (2, 4, 2, 77, 500),    # cross-attention lengths
    (1, 4, 2, 500, 77),
]


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_bwd_small(dev, d, causal, shape):
    B, Hq, Hkv, Lq, Lk = shape
    w = wl.FwdWorkload("bwd", B, Hq, Hkv, Lq, Lk, d, "bf16", causal, 900 + Lq + Lk + d)
    q, k, v, do = inputs(w, 950 + d)
    dq, dk, dv = run_gpu(q, k, v, do, dev, causal)
    full_check(dq, dk, dv, q, k, v, do, causal, f"bwd d{d} causal={causal} {shape}")


@pytest.mark.parametrize("d,Lq,Lk", [(64, 360, 360), (80, 360, 360), (128, 360, 360), (128, 300, 420)])
def test_bwd_causal_key_blocks_walking_up(dev, d, Lq, Lk):
    """Causal, with as many (batch, kv head) pairs as compute units: only the
    first one or two key blocks of each pair are resident from the start,
    and the later ones walk their query tiles upward from their diagonal.
    Full comparison; the last key block ragged, and one case with more keys
    than queries."""
    B, Hq, Hkv = 16, 32, 16
    w = wl.FwdWorkload("bwd_up", B, Hq, Hkv, Lq, Lk, d, "bf16", True, 990 + d + Lk)
    q, k, v, do = inputs(w, 991 + d + Lk)
    dq, dk, dv = run_gpu(q, k, v, do, dev, True)
    full_check(dq, dk, dv, q, k, v, do, True, f"bwd walking up d{d} Lq={Lq} Lk={Lk}")


def test_bwd_random_shapes(dev):
    """Seeded random shapes: head_dim, grouping, odd lengths on both sides,
    causal or not, [B, L, H, d] strided or contiguous, and the call made on a
    side stream of the caller's (outputs copied there right after it); full
    comparison with the rounding allowance."""
    side = torch.cuda.Stream(device=dev)
    for case in range(48):
        r = np.random.default_rng(93000 + case)
        d = int(r.choice([64, 80, 128]))
        Hkv = int(r.integers(1, 4))
        group = int(r.choice([1, 2, 4, 5]))
        B = int(r.integers(1, 3))
        Lq = int(r.choice([1, 7, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 257, 300]))
        Lk = Lq if r.random() < 0.6 else int(r.choice([1, 30, 64, 100, 257, 400]))
        causal = bool(r.random() < 0.5)
        strided = bool(r.random() < 0.3)
        on_side = bool(r.random() < 0.3)
        w = wl.FwdWorkload("bwd_rand", B, Hkv * group, Hkv, Lq, Lk, d, "bf16", causal, 94000 + case)
        q, k, v, do = inputs(w, 95000 + case)
        label = (f"bwd random {case}: B={B} Hq={Hkv * group} Hkv={Hkv} Lq={Lq} Lk={Lk} d={d} causal={causal} "
                 f"strided={strided} side={on_side}")
        print(label, flush=True)
        if strided:
            t = [x.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for x in (q, k, v, do)]
        else:
            t = [x.to(dev) for x in (q, k, v, do)]
        o, lse = sdpa.attn_fwd(t[0], t[1], t[2], causal=causal)
        if on_side:
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                g = sdpa.attn_bwd(t[0], t[1], t[2], o, lse, t[3], causal=causal, stream=side)
                g = [x.clone() for x in g]
        else:
            g = sdpa.attn_bwd(t[0], t[1], t[2], o, lse, t[3], causal=causal)
        torch.cuda.synchronize()
        full_check(*g, q, k, v, do, causal, label)


def test_bwd_deterministic(dev):
    w = wl.FwdWorkload("bwd_det", 1, 8, 2, 700, 700, 128, "bf16", True, 960)
    q, k, v, do = inputs(w, 961)
    a = run_gpu(q, k, v, do, dev, True)
    b = run_gpu(q, k, v, do, dev, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [64, 80, 128])
def test_bwd_results_ordered_on_callers_stream(dev, d):
    """At head_dim 64 and 80 the dQ kernel runs on the library's second
    stream, forked after the row sums and joined back before attn_bwd
    returns.  On a side stream of the caller's, the workspace and outputs are
    poisoned with NaN right before each call and copied right after it, all
    on that stream with no host wait in between: the copies must hold the
    gradients of a plain call (the fork orders the row sums before dQ, the
    join orders dQ before the copies)."""
    w = wl.FwdWorkload("bwd_order", 1, 16, 4, 2048, 2048, d, "bf16", True, 990 + d)
    q, k, v, do = inputs(w, 991 + d)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = sdpa.attn_fwd(qd, kd, vd, causal=True)
    ref = sdpa.attn_bwd(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    s2 = torch.cuda.Stream(device=dev)
    ws = torch.empty(sdpa.attn_bwd_workspace_bytes(w.B, w.Hq, w.Lq), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)]
    copies = []
    s2.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s2):
        for _ in range(3):
            ws.fill_(255)  # all-ones bytes: NaN as fp32
            for t in outs:
                t.fill_(float("nan"))
            sdpa.attn_bwd(qd, kd, vd, o, lse, dod, causal=True, dq=outs[0], dk=outs[1], dv=outs[2],
                          workspace=ws, stream=s2)
            copies.append([t.clone() for t in outs])
    torch.cuda.synchronize()
    for got in copies:
        for name, x, y in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(x, y), name


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_graph_replays(dev, d):
    """attn_bwd captured into a graph after an eager call (so that at d = 64
    the capture holds the fork to the library's second stream and the join
    back), replayed three times with eager work between the replays that
    poisons the outputs and workspace: every replay must reproduce the eager
    gradients exactly."""
    w = wl.FwdWorkload("bwd_graph", 1, 8, 2, 1024, 1024, d, "bf16", True, 1010 + d)
    q, k, v, do = inputs(w, 1011 + d)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = sdpa.attn_fwd(qd, kd, vd, causal=True)
    ws = torch.empty(sdpa.attn_bwd_workspace_bytes(w.B, w.Hq, w.Lq), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)]
    ref = sdpa.attn_bwd(qd, kd, vd, o, lse, dod, causal=True)
    sdpa.attn_bwd(qd, kd, vd, o, lse, dod, causal=True, dq=outs[0], dk=outs[1], dv=outs[2], workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sdpa.attn_bwd(qd, kd, vd, o, lse, dod, causal=True, dq=outs[0], dk=outs[1], dv=outs[2], workspace=ws)
    for _ in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), outs, ref):
            assert torch.equal(x, y), name
        sdpa.attn_fwd(qd, kd, vd, causal=True)  # eager work between replays


def test_bwd_no_queries_gives_zero_key_gradients(dev):
    q = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    k = torch.randn(1, 2, 100, 64, device=dev).to(torch.bfloat16)
    v = torch.randn(1, 2, 100, 64, device=dev).to(torch.bfloat16)
    lse = torch.zeros(1, 2, 0, device=dev)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    sdpa.attn_bwd(q, k, v, q, lse, q, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()


def test_bwd_strided_layout(dev):
    """[B, L, H, d] tensors viewed as [B, H, L, d] (token stride H*d)."""
    B, H, L, d = 2, 4, 200, 64
    w = wl.FwdWorkload("bwd_strided", B, H, H, L, L, d, "bf16", False, 970)
    q, k, v, do = inputs(w, 971)
    t = [x.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for x in (q, k, v, do)]
    o, lse = sdpa.attn_fwd(t[0], t[1], t[2])
    dq, dk, dv = sdpa.attn_bwd(t[0], t[1], t[2], o, lse, t[3])
    torch.cuda.synchronize()
    full_check(dq, dk, dv, q, k, v, do, False, "bwd strided")


def test_workload_bwd_causal_gqa_n8192_sampled(dev):
    """The causal GQA n=8192 d=128 workload at full size, as the benchmark
    runs it; sampled query rows (every head of kv group 0 and 7) and sampled
    keys against the oracle's per-head evaluation."""
    w = wl.C4
    q, k, v, do = inputs(w, wl.C4.seed + 50)
    dq, dk, dv = run_gpu(q, k, v, do, dev, True)
    dq, dk, dv = to_np(dq), to_np(dk), to_np(dv)
    rows = [0, 1, 127, 128, 4095, 8191]
    keys = [0, 63, 64, 4096, 8190, 8191]
    g = w.Hq // w.Hkv
    for hk in (0, w.Hkv - 1):
        sq, sk, sv = orc.attention_backward_sampled(q, k, v, do, 0, hk, rows, keys, causal=True)
        grad_check("dq", dq[0, hk * g:(hk + 1) * g][:, rows], sq, f"C4 bwd kv head {hk}")
        grad_check("dk", dk[0, hk, keys], sk, f"C4 bwd kv head {hk}")
        grad_check("dv", dv[0, hk, keys], sv, f"C4 bwd kv head {hk}")


def test_workload_bwd_causal_d80_sampled(dev):
    """The causal d=80 workload (B=4, H=16, n=2048): head_dim 80 rows sit in
    256-byte LDS rows and the last 32-row head_dim block is half padding;
    sampled query rows and keys of two (batch, head) pairs."""
    w = wl.C3
    q, k, v, do = inputs(w, w.seed + 50)
    dq, dk, dv = run_gpu(q, k, v, do, dev, True)
    dq, dk, dv = to_np(dq), to_np(dk), to_np(dv)
    rows = [0, 1, 31, 32, 1023, 2047]
    keys = [0, 31, 32, 1024, 2046, 2047]
    for b, h in ((0, 0), (3, 15)):
        sq, sk, sv = orc.attention_backward_sampled(q, k, v, do, b, h, rows, keys, causal=True)
        grad_check("dq", dq[b, h:h + 1][:, rows], sq, f"C3 bwd b{b} h{h}")
        grad_check("dk", dk[b, h, keys], sk, f"C3 bwd b{b} h{h}")
        grad_check("dv", dv[b, h, keys], sv, f"C3 bwd b{b} h{h}")
