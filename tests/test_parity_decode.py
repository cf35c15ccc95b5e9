"""Decode parity: the HIP split-KV attn_decode against the float64 CPU oracle.

Cache slots at or beyond each sequence's length hold NaN, so a read of any of
them would poison the output.
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


def run_decode(w, dev, lengths=None, poison=True, scale=None):
    q, kc, vc, lens = wl.make_decode_inputs(w, poison_tail=poison, lengths=lengths)
    o, lse = sdpa.attn_decode(q.to(dev), kc.to(dev), vc.to(dev), lens.to(dev), scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_decode(q, kc, vc, lens.numpy(), scale=scale)
    return o, lse, o_ref, lse_ref, lens


EDGE_LENGTHS = [0, 1, 2, 31, 32, 33, 127, 128, 129, 511, 512, 513, 1023, 1100]


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (32, 8), (20, 1), (40, 2)])
def test_decode_small(dev, d, Hq, Hkv):
    B = len(EDGE_LENGTHS)
    w = wl.DecodeWorkload("dec_small", B, Hq, Hkv, 1100, d, 1, 1100, "bf16", 500 + Hq + d)
    o, lse, o_ref, lse_ref, lens = run_decode(w, dev, lengths=torch.tensor(EDGE_LENGTHS))
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"decode d{d} Hq={Hq} Hkv={Hkv}")
    assert (o[0] == 0).all().item() and torch.isneginf(lse[0]).all().item()


@pytest.mark.parametrize("d", [64, 80, 128])
def test_decode_many_short_sequences(dev, d):
    """300 sequences of 0..200 slots (every 17th empty): the split kernel's
    prefix sums over the lengths take five 64-sequence passes, and one piece
    of the balanced split (at least 512 slots) spans several sequences."""
    B = 300
    g = torch.Generator().manual_seed(81 + d)
    lens = torch.randint(0, 201, (B,), generator=g, dtype=torch.int32)
    lens[::17] = 0
    w = wl.DecodeWorkload("dec_many", B, 8, 2, 200, d, 1, 200, "bf16", 80 + d)
    o, lse, o_ref, lse_ref, _ = run_decode(w, dev, lengths=lens)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"decode B=300 d{d}")
    assert (o[0] == 0).all().item() and torch.isneginf(lse[0]).all().item()


def test_decode_lengths_beyond_cache_are_clamped(dev):
    w = wl.DecodeWorkload("dec_clamp", 3, 8, 2, 600, 128, 1, 600, "bf16", 77)
    o, lse, o_ref, lse_ref, _ = run_decode(w, dev, lengths=torch.tensor([-5, 600, 100000]),
                                          poison=False)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", "decode clamped lengths")


def test_decode_explicit_scale(dev):
    w = wl.DecodeWorkload("dec_scale", 4, 8, 2, 900, 128, 1, 900, "bf16", 78)
    o, lse, o_ref, lse_ref, _ = run_decode(w, dev, scale=0.21)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", "decode scale=0.21")


def test_decode_empty_cache(dev):
    q = torch.randn(2, 4, 128).to(torch.bfloat16).to(dev)
    kc = torch.empty(2, 2, 0, 128, dtype=torch.bfloat16, device=dev)
    lens = torch.zeros(2, dtype=torch.int32, device=dev)
    o, lse = sdpa.attn_decode(q, kc, kc, lens)
    torch.cuda.synchronize()
    assert (o == 0).all().item() and torch.isneginf(lse).all().item()


@pytest.mark.parametrize("d", [80, 128])
def test_decode_strided_cache(dev, d):
    """Cache stored [B, Lmax, Hkv, d] and viewed as [B, Hkv, Lmax, d]: at
    head_dim 80 a row is 160 bytes and the next kv head's row follows it, so
    a read past head_dim would take that row's values."""
    B, Hq, Hkv, Lmax = 5, 8, 2, 700
    g = torch.Generator().manual_seed(21)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    ks = torch.randn(B, Lmax, Hkv, d, generator=g).to(torch.bfloat16)
    vs = torch.randn(B, Lmax, Hkv, d, generator=g).to(torch.bfloat16)
    lens = torch.tensor([700, 1, 350, 513, 64], dtype=torch.int32)
    o, lse = sdpa.attn_decode(q.to(dev), ks.to(dev).transpose(1, 2), vs.to(dev).transpose(1, 2),
                              lens.to(dev))
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.attention_decode(q, ks.transpose(1, 2), vs.transpose(1, 2), lens.numpy())
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", f"decode strided cache d{d}")


def test_decode_equals_last_row_of_causal_prefill_on_gpu(dev):
    """attn_decode of each sequence agrees with the last row of attn_fwd(causal)
    over the same keys, both within the bf16 gate of the oracle."""
    B, Hq, Hkv, d = 3, 8, 2, 128
    lens = [257, 64, 1000]
    g = torch.Generator().manual_seed(31)
    Lmax = max(lens)
    qfull = torch.randn(B, Hq, Lmax, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, Lmax, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, Lmax, d, generator=g).to(torch.bfloat16)
    qd = torch.stack([qfull[b, :, lens[b] - 1] for b in range(B)])
    o, lse = sdpa.attn_decode(qd.to(dev), kc.to(dev), vc.to(dev),
                              torch.tensor(lens, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        of, lf = sdpa.attn_fwd(qfull[b:b + 1, :, :L].to(dev), kc[b:b + 1, :, :L].to(dev),
                               vc[b:b + 1, :, :L].to(dev), causal=True)
        torch.cuda.synchronize()
        assert (o[b].float() - of[0, :, L - 1].float()).abs().max().item() <= 2e-2
        assert (lse[b] - lf[0, :, L - 1]).abs().max().item() <= 1e-3


def test_decode_deterministic(dev):
    w = wl.DecodeWorkload("dec_det", 6, 16, 4, 3000, 128, 1, 3000, "bf16", 79)
    q, kc, vc, lens = (t.to(dev) for t in wl.make_decode_inputs(w))
    a = sdpa.attn_decode(q, kc, vc, lens)
    b = sdpa.attn_decode(q, kc, vc, lens)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_workload_decode_full(dev):
    """The batched decode workload at its real size, every output compared."""
    w = wl.C5
    o, lse, o_ref, lse_ref, lens = run_decode(w, dev, poison=True)
    print(f"[parity] decode total keys {int(lens.sum())}", flush=True)
    check(to_np(o), o_ref, to_np(lse), lse_ref, "bf16", w.name)


def test_decode_workspace_of_another_dtype(dev):
    """A caller's workspace is counted in bytes whatever its dtype: a float32
    tensor of exactly the required bytes is accepted, and the result equals
    that of the call with the library-sized uint8 workspace."""
    w = wl.DecodeWorkload("dec_ws", 5, 16, 4, 2100, 128, 1, 2100, "bf16", 83)
    q, kc, vc, lens = (t.to(dev) for t in wl.make_decode_inputs(w))
    need = sdpa.attn_decode_workspace_bytes(w.B, w.Hq, w.Lmax, w.d)
    assert need % 4 == 0
    ws32 = torch.empty(need // 4, dtype=torch.float32, device=dev)
    a = sdpa.attn_decode(q, kc, vc, lens, workspace=ws32)
    b = sdpa.attn_decode(q, kc, vc, lens)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    with pytest.raises(sdpa.AttnError):
        sdpa.attn_decode(q, kc, vc, lens, workspace=ws32[:-1])
