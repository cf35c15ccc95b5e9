"""Masked prefill parity: the HIP attn_fwd_masked against the float64 oracle.

Boolean masks (True: the pair takes part) and additive bf16 masks, per head
and broadcast over heads and batches, alone and combined with causal; rows
that lose every key; rows whose only keys lie in the last tile.  An all-True
mask and a lower-triangular mask must reproduce attn_fwd bit for bit.
"""
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


def run(q, k, v, mask, dev, causal):
    o, lse = sdpa.attn_fwd_masked(q.to(dev), k.to(dev), v.to(dev), mask.to(dev), causal=causal)
    torch.cuda.synchronize()
    return o, lse


SHAPES = [
    # (B, Hq, Hkv, Lq, Lk)
    (2, 4, 2, 300, 320),
    (1, 2, 2, 64, 64),
    (2, 8, 1, 257, 256),
]


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add"])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bcast", ["per_head", "shared"])
def test_masked_small(dev, d, causal, kind, shape, bcast):
    B, Hq, Hkv, Lq, Lk = shape
    w = wl.FwdWorkload("masked", B, Hq, Hkv, Lq, Lk, d, "bf16", causal, 1100 + Lq + d)
    q, k, v = wl.make_fwd_inputs(w)
    mshape = (B, Hq, Lq, Lk) if bcast == "per_head" else (1, 1, Lq, Lk)
    m = wl.make_mask(mshape, kind, 1200 + d + Lq)
    o, lse = run(q, k, v, m, dev, causal)
    o_ref, lse_ref = orc.attention_forward(q, k, v, causal=causal, attn_mask=m)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"masked {kind} {bcast} d{d} causal={causal} {shape}")


@pytest.mark.parametrize("d", [64, 128])
def test_rows_without_keys_and_late_keys(dev, d):
    """Row 3 loses every key; rows 5..9 keep only keys in the last 64-key tile,
    so their reference max stays -inf through the earlier tiles."""
    B, H, Lq, Lk = 1, 2, 40, 320
    w = wl.FwdWorkload("masked_rows", B, H, H, Lq, Lk, d, "bf16", False, 1300 + d)
    q, k, v = wl.make_fwd_inputs(w)
    m = wl.make_mask((B, H, Lq, Lk), "bool", 1301)
    m[:, :, 3, :] = False
    m[:, :, 5:10, :256] = False
    o, lse = run(q, k, v, m, dev, False)
    o_ref, lse_ref = orc.attention_forward(q, k, v, attn_mask=m)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"masked rows d{d}")
    assert (o[:, :, 3] == 0).all() and torch.isneginf(lse[:, :, 3]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_all_true_mask_is_attn_fwd(dev, causal):
    w = wl.FwdWorkload("masked_true", 2, 4, 2, 300, 320, 64, "bf16", causal, 1400)
    q, k, v = wl.make_fwd_inputs(w)
    m = torch.ones(1, 1, 300, 320, dtype=torch.bool)
    o, lse = run(q, k, v, m, dev, causal)
    o2, lse2 = sdpa.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("d", [64, 128])
def test_triangular_mask_is_causal(dev, d):
    w = wl.FwdWorkload("masked_tril", 1, 4, 4, 320, 320, d, "bf16", False, 1500 + d)
    q, k, v = wl.make_fwd_inputs(w)
    m = torch.ones(320, 320, dtype=torch.bool).tril()[None, None]
    o, lse = run(q, k, v, m, dev, False)
    o2, lse2 = sdpa.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_large_negative_additive_mask_removes_keys(dev):
    """-3e4 added to a score leaves exp underflowing to exactly 0: the same
    result as a boolean mask on those pairs."""
    w = wl.FwdWorkload("masked_neg", 1, 2, 2, 100, 128, 64, "bf16", False, 1600)
    q, k, v = wl.make_fwd_inputs(w)
    mb = wl.make_mask((1, 2, 100, 128), "bool", 1601)
    mb[..., 0] = True
    ma = torch.where(mb, torch.tensor(0.0), torch.tensor(-3e4)).to(torch.bfloat16)
    ob, lb = run(q, k, v, mb, dev, False)
    oa, la = run(q, k, v, ma, dev, False)
    assert torch.equal(oa, ob)
    assert (la - lb).abs().max() <= 1e-5
