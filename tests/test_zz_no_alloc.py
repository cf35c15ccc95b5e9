"""attn_decode_noalloc — the decode entry point for callers that cannot
allocate device memory — against attn_decode, through the C ABI.

Both run the same kernels on the same inputs, so the outputs must be
bit-identical; the small case is also held to the bf16 gates against the
float64 oracle.  The first call fills the static workspace almost to its
limit, the second is smaller, so stale partial results left in the shared
array by the first call would show in the second.
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
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def both(q, kc, vc, lens):
    o_ref, l_ref = sdpa.attn_decode(q, kc, vc, lens)
    o = torch.full_like(q, float("nan"))
    l = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=q.device)
    sdpa.attn_decode_noalloc(q, kc, vc, lens, o, l)
    torch.cuda.synchronize()
    return o, l, o_ref, l_ref


def test_noalloc_equals_decode_large_then_small(dev):
    # 1) B=16, Hq=64, Hkv=4 (groups of 16), d=128, Lmax=31744: 63 pieces per
    #    sequence, 16*64*63 partial rows, 33.29 MB of the 33.55 MB of scratch
    B, Hq, Hkv, Lmax, d = 16, 64, 4, 31744, 128
    need = sdpa.attn_decode_workspace_bytes(B, Hq, Lmax, d)
    assert 0.99 * sdpa.ATTN_DECODE_NOALLOC_SCRATCH_BYTES < need <= sdpa.ATTN_DECODE_NOALLOC_SCRATCH_BYTES
    g = torch.Generator(device=dev).manual_seed(7101)
    q = torch.randn(B, Hq, d, generator=g, device=dev).to(torch.bfloat16)
    kc = torch.randn(B, Hkv, Lmax, d, generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, Lmax, d, generator=g, device=dev).to(torch.bfloat16)
    lens = torch.randint(1, Lmax + 1, (B,), generator=g, device=dev, dtype=torch.int32)
    lens[0], lens[1] = Lmax, 0
    print(f"[noalloc] large B={B} Hq={Hq} Hkv={Hkv} Lmax={Lmax} need={need}", flush=True)
    o, l, o_ref, l_ref = both(q, kc, vc, lens)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    del kc, vc
    # 2) a smaller call right after: edge lengths, NaN beyond each length
    lengths = [0, 1, 31, 32, 33, 511, 512, 513, 1100]
    w = wl.DecodeWorkload("dec_noalloc_small", len(lengths), 8, 2, 1100, 128, 1, 1100, "bf16", 7102)
    qs, kcs, vcs, lns = wl.make_decode_inputs(w, poison_tail=True, lengths=torch.tensor(lengths))
    print(f"[noalloc] small B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lmax={w.Lmax}", flush=True)
    o, l, o_ref, l_ref = both(*(t.to(dev) for t in (qs, kcs, vcs, lns)))
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    o_orc, l_orc = orc.attention_decode(qs, kcs, vcs, lns.numpy())
    check(to_np(o), o_orc, to_np(l), l_orc, "bf16", "decode_noalloc small")


def test_noalloc_decode_workload(dev):
    """The batched decode workload (B=64, Hq=32, Hkv=8, d=128, lengths
    U{1024..8192}) through both entry points."""
    q, kc, vc, lens = (t.to(dev) for t in wl.make_decode_inputs(wl.C5))
    print(f"[noalloc] {wl.C5.name}", flush=True)
    o, l, o_ref, l_ref = both(q, kc, vc, lens)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
