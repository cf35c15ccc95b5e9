"""Seeded synthetic inputs for the attention forward and decode workloads.

This module only draws numbers and fixes shapes.  It holds none of the
attention arithmetic, so both the CPU oracle (through the tests) and the GPU
path (through the tests and the benchmark) can consume the very same bits.

Recipe (one per workload):
  g = torch.Generator().manual_seed(seed)
  Q, K, V = randn(shape, generator=g) in float32, drawn in that order
  bf16 workloads: each tensor rounded to bfloat16 (round-to-nearest-even,
                  torch's own conversion); the oracle receives exactly those
                  values widened to float64
  decode workloads, after V: lengths = randint(lo, hi + 1, (B,), generator=g)
  FP8 workloads: Q, K, V drawn as above, each then stored as e4m3 codes of
                  x / descale with descale = max|x| / 448 (torch's
                  float8_e4m3fn rounding); the oracle receives the codes and
                  the descales
  packed variable-length workloads: lengths = randint(lo, hi + 1, (B,),
                  generator=g) first (query and key lengths equal unless
                  given), then Q [total_q, Hq, d], K, V [total_k, Hkv, d]

The five named workloads are the shapes the attention pages discuss:
the GPT-3-scale layer (B=1, 96 heads, n=4096, d=64) from "Flash Attention原理"
section 一, the d=80 head size that needed padding on other hardware from
"SDPA backend 与 FlashAttention" section 9, n=8k prefill with grouped KV heads
from the same page's section 12, and batched decode against a KV cache from its
section 5.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class FwdWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    d: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    seed: int

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lmax: int
    d: int
    len_lo: int
    len_hi: int          # inclusive
    dtype: str
    seed: int

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


# The five workloads, smallest first.
C1 = FwdWorkload("fwd_f32_b1_h2_n256_d64", 1, 2, 2, 256, 256, 64, "f32", False, 1001)
C2 = FwdWorkload("fwd_bf16_b1_h96_n4096_d64", 1, 96, 96, 4096, 4096, 64, "bf16", False, 1002)
C3 = FwdWorkload("fwd_bf16_causal_b4_h16_n2048_d80", 4, 16, 16, 2048, 2048, 80, "bf16", True, 1003)
C4 = FwdWorkload("fwd_bf16_causal_gqa_b1_hq32_hkv8_n8192_d128", 1, 32, 8, 8192, 8192, 128, "bf16", True, 1004)
C5 = DecodeWorkload("decode_bf16_gqa_b64_hq32_hkv8_lmax8192_d128", 64, 32, 8, 8192, 128, 1024, 8192, "bf16", 1005)



@dataclass(frozen=True)
class VarlenWorkload:
    """Packed sequences of random lengths (cnblogs FAQ Q10): the serving-prefill
    shape, one kernel over sequences of different lengths without padding."""
    name: str
    B: int
    Hq: int
    Hkv: int
    len_lo: int
    len_hi: int          # inclusive
    d: int
    dtype: str
    causal: bool
    seed: int


# Packed causal GQA prefill of 16 sequences of 256..4096 tokens at the n=8192
# workload's head shape.
C6 = VarlenWorkload("varlen_bf16_causal_gqa_b16_hq32_hkv8_len256_4096_d128", 16, 32, 8, 256, 4096, 128,
                    "bf16", True, 1006)

# FP8 (e4m3) inputs at the shapes of the n=4096 and the n=8192 workloads.
C7 = FwdWorkload("fwd_fp8_b1_h96_n4096_d64", 1, 96, 96, 4096, 4096, 64, "fp8", False, 1011)
C8 = FwdWorkload("fwd_fp8_causal_gqa_b1_hq32_hkv8_n8192_d128", 1, 32, 8, 8192, 8192, 128, "fp8", True, 1012)

FWD_WORKLOADS = {w.name: w for w in (C1, C2, C3, C4)}
FP8_WORKLOADS = {w.name: w for w in (C7, C8)}
DECODE_WORKLOADS = {C5.name: C5}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def make_fwd_inputs(w: FwdWorkload, q_mul: float = 1.0):
    """Q [B,Hq,Lq,d], K and V [B,Hkv,Lk,d] on the CPU in the workload's dtype.

    q_mul scales Q before rounding; values above 1 give peaky score rows whose
    running maximum moves from tile to tile.
    """
    g = torch.Generator().manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.Lq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Hkv, w.Lk, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Hkv, w.Lk, w.d), generator=g, dtype=torch.float32)
    if q_mul != 1.0:
        q = q * q_mul
    dt = torch_dtype(w.dtype)
    return q.to(dt), k.to(dt), v.to(dt)


E4M3_MAX = 448.0  # largest finite e4m3 value


def make_fp8_inputs(w: FwdWorkload, q_mul: float = 1.0):
    """e4m3 codes (uint8) q8 [B,Hq,Lq,d], k8 and v8 [B,Hkv,Lk,d] on the CPU and
    their descales (q_descale, k_descale, v_descale).

    Q, K and V are drawn as make_fwd_inputs draws them (float32, same order,
    Q times q_mul); each tensor gets descale = max|x| / 448 and codes =
    torch's float8_e4m3fn rounding of x / descale, so the codes span the
    format's range and a code stands for descale times its value.
    """
    g = torch.Generator().manual_seed(w.seed)
    xs = [torch.randn((w.B, w.Hq, w.Lq, w.d), generator=g, dtype=torch.float32),
          torch.randn((w.B, w.Hkv, w.Lk, w.d), generator=g, dtype=torch.float32),
          torch.randn((w.B, w.Hkv, w.Lk, w.d), generator=g, dtype=torch.float32)]
    if q_mul != 1.0:
        xs[0] = xs[0] * q_mul
    codes, descales = [], []
    for x in xs:
        amax = float(x.abs().max()) if x.numel() else 1.0
        ds = amax / E4M3_MAX if amax > 0 else 1.0
        codes.append((x / ds).to(torch.float8_e4m3fn).view(torch.uint8))
        descales.append(ds)
    return codes[0], codes[1], codes[2], tuple(descales)


def make_decode_inputs(w: DecodeWorkload, poison_tail: bool = False,
                       lengths: Optional[torch.Tensor] = None):
    """q [B,Hq,d]; k_cache and v_cache [B,Hkv,Lmax,d]; seqlens int32 [B].

    With poison_tail, every cache slot at or beyond a sequence's length holds
    NaN, so any read of it would show up in the output.
    """
    g = torch.Generator().manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Hkv, w.Lmax, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Hkv, w.Lmax, w.d), generator=g, dtype=torch.float32)
    lens = torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=g, dtype=torch.int32)
    if lengths is not None:
        lens = lengths.to(torch.int32).clone()
    dt = torch_dtype(w.dtype)
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    if poison_tail:
        for b in range(w.B):
            L = int(lens[b])
            k[b, :, L:, :] = float("nan")
            v[b, :, L:, :] = float("nan")
    return q, k, v, lens


def make_varlen_inputs(w: VarlenWorkload, lens_q=None, lens_k=None):
    """q [total_q,Hq,d], k and v [total_k,Hkv,d] in the workload's dtype and the
    int32 offsets cu_q, cu_k [B+1] on the CPU.  Lengths are drawn first (query
    and key lengths equal) unless given."""
    g = torch.Generator().manual_seed(w.seed)
    lens = torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=g, dtype=torch.int64)
    lq = torch.as_tensor(lens_q, dtype=torch.int64) if lens_q is not None else lens
    lk = torch.as_tensor(lens_k, dtype=torch.int64) if lens_k is not None else lq
    cu_q = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lq, 0)]).to(torch.int32)
    cu_k = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lk, 0)]).to(torch.int32)
    q = torch.randn((int(cu_q[-1]), w.Hq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((int(cu_k[-1]), w.Hkv, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((int(cu_k[-1]), w.Hkv, w.d), generator=g, dtype=torch.float32)
    dt = torch_dtype(w.dtype)
    return q.to(dt), k.to(dt), v.to(dt), cu_q, cu_k


def make_mask(shape, kind: str, seed: int, keep: float = 0.7):
    """A seeded attention mask of the given [B|1, H|1, Lq, Lk] shape: "bool"
    keeps each pair with probability `keep`; "add" draws N(0, 1) * 2 values
    rounded to bf16."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(shape, generator=g, dtype=torch.float32)
    if kind == "bool":
        return u < keep
    return (torch.randn(shape, generator=g, dtype=torch.float32) * 2.0).to(torch.bfloat16)


def shrink(w, **kw):
    """A copy of a workload with some sizes replaced (name and seed kept unless given)."""
    return replace(w, **kw)


# ---------------------------------------------------------------------------
# Work and traffic accounting (counts from shapes; no attention arithmetic).

def algorithmic_flops_fwd(B, Hq, Lq, Lk, d, causal) -> int:
    """4 * Lq * Lk * d per (batch, query head): Q K^T and P V are 2 * Lq * Lk * d
    each.  Causal work is credited as exactly half; padding is never credited."""
    f = 4 * B * Hq * Lq * Lk * d
    return f // 2 if causal else f


def algorithmic_bytes_fwd(B, Hq, Hkv, Lq, Lk, d, elem_bytes) -> int:
    """Q, K, V read once and O written once in the input dtype, LSE once in fp32.

    Q/K/V are the traffic that cannot be avoided ("Flash Attention原理", section
    六); S and P never leave the chip.
    """
    return (B * Hq * Lq * d * 2 + B * Hkv * Lk * d * 2) * elem_bytes + B * Hq * Lq * 4


def algorithmic_flops_bwd(B, Hq, Lq, Lk, d, causal) -> int:
    """The backward's five products (Q K^T recomputed, dP = dO V^T, dV = P^T dO,
    dQ = dS K, dK = dS^T Q), 2 Lq Lk d flops each per (batch, query head):
    2.5 times the forward's count; causal credited as exactly half."""
    f = 10 * B * Hq * Lq * Lk * d
    return f // 2 if causal else f


def algorithmic_bytes_bwd(B, Hq, Hkv, Lq, Lk, d, elem_bytes) -> int:
    """Q, K, V, O, dO and LSE read once; dQ, dK, dV written once."""
    return (3 * B * Hq * Lq * d + 4 * B * Hkv * Lk * d) * elem_bytes + B * Hq * Lq * 4


def algorithmic_flops_varlen(lens_q, lens_k, Hq, d, causal) -> int:
    """Sum over sequences of the dense count; causal credited as exactly half."""
    return sum(algorithmic_flops_fwd(1, Hq, int(a), int(b), d, causal) for a, b in zip(lens_q, lens_k))


def algorithmic_bytes_varlen(total_q, total_k, Hq, Hkv, d, elem_bytes, B) -> int:
    """Q, K, V read once, O written once, LSE once, plus the two offset arrays."""
    return algorithmic_bytes_fwd(1, Hq, Hkv, total_q, total_k, d, elem_bytes) + 2 * (B + 1) * 4


def algorithmic_flops_decode(seqlens, Hq, d, Lmax) -> int:
    tot = sum(max(0, min(int(x), Lmax)) for x in seqlens)
    return 4 * tot * Hq * d


def algorithmic_bytes_decode(seqlens, Hq, Hkv, d, elem_bytes, Lmax) -> int:
    """Valid K and V cache rows read once, Q read and O written once, LSE in fp32."""
    lens = [max(0, min(int(x), Lmax)) for x in seqlens]
    B = len(lens)
    return sum(lens) * Hkv * d * 2 * elem_bytes + B * Hq * d * 2 * elem_bytes + B * Hq * 4


def score_matrix_bytes(n: int, elem_bytes: int = 4) -> int:
    """Bytes of one materialised n x n score (or probability) matrix."""
    return n * n * elem_bytes
