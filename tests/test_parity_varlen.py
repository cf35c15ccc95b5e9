"""Packed variable-length prefill and causal cross-attention: the HIP path
against the float64 CPU oracle, sequence by sequence.

Small packed batches are compared in full; the packed serving workload at its
real size on sampled rows of every sequence, which the oracle computes one by
one.  Equal lengths must reproduce the dense entry point bit for bit.
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


def run_varlen(w, dev, lens_q, lens_k=None, max_seqlen_q=None, cu_override=None):
    q, k, v, cu_q, cu_k = wl.make_varlen_inputs(w, lens_q, lens_k)
    if cu_override is not None:
        cu_q, cu_k = (torch.tensor(c, dtype=torch.int32) for c in cu_override)
    mq = max_seqlen_q if max_seqlen_q is not None else int((cu_q[1:] - cu_q[:-1]).max())
    o, lse = sdpa.attn_fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cu_q.to(dev), cu_k.to(dev), mq,
                                  causal=w.causal)
    torch.cuda.synchronize()
    return q, k, v, cu_q, cu_k, o, lse


MIXES = [
    # (query lengths, key lengths or None for equal)
    ([300, 1, 0, 129, 64, 200], None),   # ragged tiles, a single token, an empty sequence
    ([77, 300, 5], [500, 64, 1]),        # cross-attention lengths per sequence
    ([40, 260], [0, 260]),               # a sequence without keys
]


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mix", range(len(MIXES)))
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 1)])
def test_varlen_small(dev, d, causal, mix, Hq, Hkv):
    lq, lk = MIXES[mix]
    w = wl.VarlenWorkload("varlen_small", len(lq), Hq, Hkv, 1, 1, d, "bf16", causal, 500 + 7 * mix + d)
    q, k, v, cu_q, cu_k, o, lse = run_varlen(w, dev, lq, lk)
    o_ref, lse_ref = orc.attention_forward_varlen(q, k, v, cu_q.tolist(), cu_k.tolist(), causal=causal)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"varlen d{d} causal={causal} mix{mix} {Hq}/{Hkv}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_dense_bit_for_bit(dev, d, causal):
    B, Hq, Hkv, L = 3, 4, 2, 257
    w = wl.VarlenWorkload("varlen_eq", B, Hq, Hkv, 1, 1, d, "bf16", causal, 600 + d)
    q, k, v, cu_q, cu_k, o, lse = run_varlen(w, dev, [L] * B)
    qd = q.view(B, L, Hq, d).transpose(1, 2).contiguous().to(dev)
    kd = k.view(B, L, Hkv, d).transpose(1, 2).contiguous().to(dev)
    vd = v.view(B, L, Hkv, d).transpose(1, 2).contiguous().to(dev)
    od, lsed = sdpa.attn_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.view(B, L, Hq, d).transpose(1, 2).cpu(), od.cpu())
    assert torch.equal(lse.view(Hq, B, L).transpose(0, 1).cpu(), lsed.cpu())


def test_varlen_sequence_without_keys_is_zero(dev):
    w = wl.VarlenWorkload("varlen_nokeys", 2, 4, 4, 1, 1, 64, "bf16", True, 700)
    _, _, _, cu_q, _, o, lse = run_varlen(w, dev, [50, 70], [0, 70])
    assert (o[:50] == 0).all() and torch.isneginf(lse[:, :50]).all()
    assert torch.isfinite(lse[:, 50:]).all()


def test_varlen_out_of_range_offsets_are_clamped(dev):
    """Offsets past the packed extents are clamped on the device: the result
    equals the oracle on the clamped offsets and nothing outside is touched."""
    w = wl.VarlenWorkload("varlen_clamp", 3, 4, 2, 1, 1, 64, "bf16", False, 701)
    lq = [100, 100, 100]
    bad = ([0, 100, 250, 900], [0, 100, 9999, 9999])   # totals are 300 and 300
    q, k, v, _, _, o, lse = run_varlen(w, dev, lq, cu_override=bad, max_seqlen_q=300)
    cq, ck = [0, 100, 250, 300], [0, 100, 300, 300]
    o_ref, lse_ref = orc.attention_forward_varlen(q, k, v, cq, ck)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", "varlen clamped offsets")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lq,Lk", [(77, 500), (500, 77), (1, 300)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dense_causal_cross_attention(dev, d, Lq, Lk, dtype):
    """Causal with Lq != Lk: top-left, query i sees keys j <= i."""
    w = wl.FwdWorkload("cross_causal", 2, 4, 2, Lq, Lk, d, dtype, True, 800 + Lq + d)
    q, k, v = wl.make_fwd_inputs(w)
    o, lse = sdpa.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=True)
    check(to_np(o), o_ref, to_np(lse), lse_ref, dtype, f"cross causal {dtype} d{d} {Lq}x{Lk}")


def test_workload_varlen_packed_sampled_rows(dev):
    """The packed serving workload at full size, launched as the benchmark
    launches it; the first, a middle and the last row of every sequence for
    two query heads are checked against the oracle."""
    w = wl.C6
    q, k, v, cu_q, cu_k, o, lse = run_varlen(w, dev, None)
    o, lse = to_np(o), to_np(lse)
    for b in range(w.B):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        L = qe - qs
        rows = sorted({0, L // 2, L - 1})
        qb = q[qs:qe].transpose(0, 1)[None]
        kb = k[ks:ke].transpose(0, 1)[None]
        vb = v[ks:ke].transpose(0, 1)[None]
        for h in (0, w.Hq - 1):
            o_ref, lse_ref = orc.attention_forward_rows(qb, kb, vb, 0, h, rows, causal=w.causal)
            idx = [qs + r for r in rows]
            check(o[idx, h], o_ref, lse[h, idx], lse_ref, "bf16", f"C6 seq{b} h{h}")
