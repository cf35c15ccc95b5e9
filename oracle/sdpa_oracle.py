"""CPU oracle for scaled dot-product attention: plain, slow, float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check in __graft_entry__ and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

What it computes is the plain definition of attention, written out with the
n x n score matrix S and probability matrix P materialised, in the order the
pages give it:

  * "Flash Attention原理：分块计算与重计算" (cnblogs), section 一: inputs
    shaped (batch, num_heads, seq_len, head_dim); S = Q K^T; P = softmax(S /
    sqrt(d)) taken along the key axis; O = P V.  Its listing applies the scale
    Q.size(-1) ** -0.5 to S when no scale is given.
  * "PyTorch Profiler 實戰：五種 Attention 實現的 GPU 核心剖析", section
    "核心概念": the step order is Q K^T, scale, causal mask, softmax, times V.
  * The same cnblogs page, section 四: the softmax subtracts the row maximum
    before exponentiating, and section 五: the per-row statistics kept instead
    of S and P are the row maximum m and the normaliser l.  Here they are
    returned together as the natural-log log-sum-exp, LSE = m + ln l.

Readings where the pages leave a step open (each also listed in the design
notes):
  * causal means top-left alignment: query i sees keys j <= i, for any Lq
    and Lk (the convention of the scaled_dot_product_attention call the pages
    use; they do not say where the diagonal sits when Lq != Lk);
  * packed variable-length batches (cnblogs FAQ Q10): sequence b owns query
    rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1 and
    attends only to its own keys, each sequence exactly as a batch of one;
  * a grouped-query head h reads key/value head h // (Hq / Hkv);
  * decode is one query token per sequence that sees cache slots 0..L_b-1;
    a length above the cache size is clamped to it;
  * a row that sees no key at all gets O = 0 and LSE = -inf;
  * the backward pass (cnblogs section 五: the forward keeps only the row
    statistics and the backward recomputes the softmax values from them) is
    the textbook chain rule through S, P and O, which the pages do not write
    out: dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)),
    dQ = scale dS K, dK = scale dS^T Q; a grouped key/value head receives the
    sum over its query heads;
  * FP8 inputs (cnblogs section 六 and FAQ Q8: the third version runs on
    8-bit floating-point matrix units; the pages fix no format and no
    scaling): every element is an e4m3 code and every tensor carries one
    float multiplier, its descale, so an element stands for descale times the
    code's value; the attention is the definition above applied to those
    values.

All functions take and return numpy float64 arrays.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional, Sequence

import numpy as np

try:  # keep BLAS single-threaded inside the per-head thread pool
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None


def default_scale(d: int) -> float:
    """1/sqrt(d), the default scale of the cnblogs page's section 一 listing."""
    return 1.0 / math.sqrt(d)


def _head_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    causal: bool, row_ids: Optional[np.ndarray] = None,
                    n_keys: Optional[int] = None, return_sp: bool = False,
                    mask: Optional[np.ndarray] = None):
    """One (batch, head) pair: q [n_rows, d], k and v [Lk, d].

    row_ids are the absolute query positions of the rows of q (needed for the
    causal mask when only some rows are asked for).  n_keys limits the keys to
    the first n_keys rows of k and v (decode lengths).  mask [n_rows, Lk] is a
    boolean (True: the pair takes part) or an additive float mask.
    """
    if n_keys is not None:
        k = k[:n_keys]
        v = v[:n_keys]
    n_rows, lk = q.shape[0], k.shape[0]
    d_v = v.shape[1]
    if lk == 0:
        o = np.zeros((n_rows, d_v))
        lse = np.full(n_rows, -np.inf)
        if return_sp:
            return o, lse, np.zeros((n_rows, 0)), np.zeros((n_rows, 0))
        return o, lse
    # Step 1: scores, materialised, then scaled; an additive mask is added to
    # the scaled scores, a boolean one removes the pairs it marks False.
    s = (q @ k.T) * scale
    if mask is not None:
        mask = np.asarray(mask)[:, :lk]
        s = np.where(mask, s, -np.inf) if mask.dtype == bool else s + mask.astype(np.float64)
    # Step 2: causal mask.
    if causal:
        if row_ids is None:
            row_ids = np.arange(n_rows)
        cols = np.arange(lk)
        s = np.where(cols[None, :] > row_ids[:, None], -np.inf, s)
    # Step 3: safe softmax along the key axis.
    m = s.max(axis=-1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=-1)
    l_safe = np.where(empty, 1.0, l)
    p = e / l_safe[:, None]
    # Step 4: weighted sum of values.
    o = p @ v
    # Step 5: row statistics as one log-sum-exp.
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    o = np.where(empty[:, None], 0.0, o)
    if return_sp:
        return o, lse, s, p
    return o, lse


def _as64(x) -> np.ndarray:
    """Widen to float64 (accepts numpy arrays and CPU torch tensors, bf16 included)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _as_mask(m) -> np.ndarray:
    """A boolean mask stays boolean; any other mask is widened to float64."""
    if str(getattr(m, "dtype", "")) in ("torch.bool", "bool"):
        return np.asarray(m.numpy() if hasattr(m, "numpy") else m, dtype=bool)
    return _as64(m)


def _pool_map(fn, items: Sequence, threads: Optional[int]):
    if threads is None:
        threads = min(len(items), os.cpu_count() or 1)
    if threads <= 1 or len(items) <= 1:
        return [fn(it) for it in items]
    ctx = threadpool_limits(limits=1) if threadpool_limits is not None else None
    try:
        if ctx is not None:
            ctx.__enter__()
        with ThreadPoolExecutor(max_workers=threads) as ex:
            return list(ex.map(fn, items))
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def attention_forward(q, k, v, causal: bool = False, scale: Optional[float] = None,
                      threads: Optional[int] = None, return_sp: bool = False, attn_mask=None):
    """Prefill attention. q [B,Hq,Lq,d]; k, v [B,Hkv,Lk,d] -> O [B,Hq,Lq,d], LSE [B,Hq,Lq].

    attn_mask, broadcastable to [B,Hq,Lq,Lk]: boolean (True: the pair takes
    part) or additive (added to the scaled scores), as the pages' SDPA call
    takes it; it combines with causal.  With return_sp the materialised S and
    P [B,Hq,Lq,Lk] are returned as well (small shapes only).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Lq, d = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if Bk != B or dk != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("q, k, v shapes disagree")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    if scale is None:
        scale = default_scale(d)
    group = Hq // Hkv
    o = np.zeros((B, Hq, Lq, v.shape[3]))
    lse = np.zeros((B, Hq, Lq))
    s_all = np.zeros((B, Hq, Lq, Lk)) if return_sp else None
    p_all = np.zeros((B, Hq, Lq, Lk)) if return_sp else None
    items = [(b, h) for b in range(B) for h in range(Hq)]

    if attn_mask is not None:
        attn_mask = np.broadcast_to(_as_mask(attn_mask), (B, Hq, Lq, Lk))

    def one(item):
        b, h = item
        hk = h // group
        return _head_attention(q[b, h], k[b, hk], v[b, hk], scale, causal,
                               return_sp=return_sp,
                               mask=None if attn_mask is None else attn_mask[b, h])

    results = _pool_map(one, items, threads)
    for (b, h), res in zip(items, results):
        o[b, h], lse[b, h] = res[0], res[1]
        if return_sp:
            s_all[b, h], p_all[b, h] = res[2], res[3]
    if return_sp:
        return o, lse, s_all, p_all
    return o, lse


def _head_backward(q, k, v, do, scale: float, causal: bool):
    """Gradients for one (batch, query head): q, do [Lq, d]; k, v [Lk, d].

    Recomputes S and P as the forward defines them, then applies the chain
    rule step by step.  Returns dq [Lq, d], dk [Lk, d], dv [Lk, d].
    """
    lq, lk = q.shape[0], k.shape[0]
    if lk == 0 or lq == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    _, _, s, p = _head_attention(q, k, v, scale, causal, return_sp=True)
    dv = p.T @ do                                    # O = P V
    dp = do @ v.T
    dsum = (p * dp).sum(axis=-1, keepdims=True)      # softmax along keys
    ds = p * (dp - dsum)
    dq = (ds @ k) * scale                            # S = Q K^T * scale
    dk = (ds.T @ q) * scale
    return dq, dk, dv


def attention_backward(q, k, v, do, causal: bool = False, scale: Optional[float] = None,
                       threads: Optional[int] = None):
    """Gradients of the prefill attention output O with respect to q, k, v
    for the output gradient do [B,Hq,Lq,d].  Returns dq [B,Hq,Lq,d],
    dk and dv [B,Hkv,Lk,d] (each kv head summed over its query heads)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Hq, Lq, d = q.shape
    Hkv = k.shape[1]
    if do.shape != q.shape or k.shape[0] != B or v.shape != k.shape:
        raise ValueError("q, k, v, do shapes disagree")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    if scale is None:
        scale = default_scale(d)
    group = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    items = [(b, h) for b in range(B) for h in range(Hq)]

    def one(item):
        b, h = item
        return _head_backward(q[b, h], k[b, h // group], v[b, h // group], do[b, h], scale, causal)

    for (b, h), (gq, gk, gv) in zip(items, _pool_map(one, items, threads)):
        dq[b, h] = gq
        dk[b, h // group] += gk
        dv[b, h // group] += gv
    return dq, dk, dv


def attention_backward_sampled(q, k, v, do, b: int, hk: int, q_rows: Iterable[int], keys: Iterable[int],
                               causal: bool = False, scale: Optional[float] = None):
    """The backward's definition for a few outputs of one (batch, kv head), at
    any size: dQ of the given query rows for every query head of the group, and
    dK, dV of the given keys (summed over the group).  Each query head's full
    score matrix is formed once (n x n float64), then only the asked-for rows
    and columns of the chain rule are evaluated.
    Returns dq [group, len(q_rows), d], dk and dv [len(keys), d]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    group = Hq // Hkv
    d = q.shape[-1]
    if scale is None:
        scale = default_scale(d)
    q_rows = np.asarray(list(q_rows), dtype=np.int64)
    keys = np.asarray(list(keys), dtype=np.int64)
    kk, vv = _as64(k[b, hk]), _as64(v[b, hk])
    dq = np.zeros((group, len(q_rows), d))
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), vv.shape[1]))
    for hg in range(group):
        h = hk * group + hg
        qq, dd = _as64(q[b, h]), _as64(do[b, h])
        o, _, s, p = _head_attention(qq, kk, vv, scale, causal, return_sp=True)
        drow = (dd * o).sum(axis=-1)                 # rowsum(P * dP) = rowsum(dO * O)
        # dQ rows: dS of those rows over all keys
        dp_r = dd[q_rows] @ vv.T
        ds_r = p[q_rows] * (dp_r - drow[q_rows, None])
        dq[hg] = (ds_r @ kk) * scale
        # dK, dV of the sampled keys: those columns over all queries
        dp_c = dd @ vv[keys].T
        ds_c = p[:, keys] * (dp_c - drow[:, None])
        dk += (ds_c.T @ qq) * scale
        dv += p[:, keys].T @ dd
    return dq, dk, dv


def attention_forward_varlen(q, k, v, cu_q: Sequence[int], cu_k: Sequence[int], causal: bool = False,
                             scale: Optional[float] = None, threads: Optional[int] = None):
    """Packed variable-length prefill (cnblogs FAQ Q10, cross-attention FAQ Q15).

    q [total_q, Hq, d]; k, v [total_k, Hkv, d]; cu_q, cu_k the B + 1 sequence
    offsets.  Each sequence is attention_forward's computation on its own rows
    and keys.  Returns O [total_q, Hq, d] and LSE [Hq, total_q].
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    if dk != d or v.shape[:2] != k.shape[:2] or len(cu_q) != len(cu_k):
        raise ValueError("q, k, v or the offsets disagree")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    if scale is None:
        scale = default_scale(d)
    group = Hq // Hkv
    o = np.zeros((total_q, Hq, v.shape[2]))
    lse = np.full((Hq, total_q), -np.inf)
    items = [(b, h) for b in range(len(cu_q) - 1) for h in range(Hq)]

    def one(item):
        b, h = item
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        return _head_attention(q[qs:qe, h], k[ks:ke, h // group], v[ks:ke, h // group], scale, causal)

    for (b, h), (ob, lb) in zip(items, _pool_map(one, items, threads)):
        o[cu_q[b]:cu_q[b + 1], h] = ob
        lse[h, cu_q[b]:cu_q[b + 1]] = lb
    return o, lse


def attention_forward_rows(q, k, v, b: int, h: int, rows: Iterable[int],
                           causal: bool = False, scale: Optional[float] = None, attn_mask=None):
    """The same definition for a few query rows of one (batch, query head).

    Used to check full-size runs on sampled outputs: each row needs only its
    own score row, so any row of any size can be computed on its own.
    Returns O [len(rows), d] and LSE [len(rows)].
    """
    q_bh = _as64(q[b, h])
    Hq, Hkv = q.shape[1], k.shape[1]
    hk = h // (Hq // Hkv)
    rows = np.asarray(list(rows), dtype=np.int64)
    if scale is None:
        scale = default_scale(q.shape[-1])
    m = None
    if attn_mask is not None:
        m = np.broadcast_to(_as_mask(attn_mask), (q.shape[0], q.shape[1], q.shape[2], k.shape[2]))[b, h][rows]
    return _head_attention(q_bh[rows], _as64(k[b, hk]), _as64(v[b, hk]), scale,
                           causal, row_ids=rows, mask=m)


def attention_decode(q, k_cache, v_cache, seqlens, scale: Optional[float] = None,
                     threads: Optional[int] = None, batches: Optional[Sequence[int]] = None):
    """One query token per sequence against a KV cache.

    q [B,Hq,d]; k_cache, v_cache [B,Hkv,Lmax,d]; seqlens [B] integers.
    Sequence b sees cache slots 0..min(seqlens[b], Lmax)-1.
    Returns O [B,Hq,d] and LSE [B,Hq] (rows of batches not listed stay 0).
    """
    q = _as64(q)
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    if scale is None:
        scale = default_scale(d)
    group = Hq // Hkv
    lens = [max(0, min(int(x), Lmax)) for x in np.asarray(seqlens).reshape(-1)]
    if batches is None:
        batches = range(B)
    o = np.zeros((B, Hq, v_cache.shape[3]))
    lse = np.zeros((B, Hq))
    items = [(b, hk) for b in batches for hk in range(Hkv)]

    def one(item):
        b, hk = item
        L = lens[b]
        kk = _as64(k_cache[b, hk, :L])
        vv = _as64(v_cache[b, hk, :L])
        qq = q[b, hk * group:(hk + 1) * group]
        return _head_attention(qq, kk, vv, scale, causal=False)

    results = _pool_map(one, items, threads)
    for (b, hk), (ob, lb) in zip(items, results):
        o[b, hk * group:(hk + 1) * group] = ob
        lse[b, hk * group:(hk + 1) * group] = lb
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Combine attention results computed over disjoint key subsets.

    o_parts [S, ..., d] holds each part's normalised output, lse_parts [S, ...]
    each part's log-sum-exp.  This is the normaliser identity of the cnblogs
    page's section 四 (rescale each block's exponent sum by exp(m_block - m)
    and add), applied to whole parts: with M = max_s LSE_s,
      LSE = M + ln sum_s exp(LSE_s - M),  O = sum_s exp(LSE_s - LSE) O_s.
    Parts with LSE = -inf carry no keys and get weight 0.  Works in the dtype
    it is given.
    """
    o_parts = np.asarray(o_parts)
    lse_parts = np.asarray(lse_parts)
    M = lse_parts.max(axis=0)
    empty = ~np.isfinite(M)
    M_safe = np.where(empty, 0.0, M).astype(lse_parts.dtype)
    w = np.exp(lse_parts - M_safe[None])
    tot = w.sum(axis=0)
    tot_safe = np.where(empty, 1.0, tot).astype(lse_parts.dtype)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, M_safe + np.log(tot_safe)).astype(lse_parts.dtype)
    o = (w[..., None] * o_parts).sum(axis=0) / tot_safe[..., None]
    o = np.where(empty[..., None], 0.0, o).astype(o_parts.dtype)
    return o, lse


def brute_force_attention(q, k, v, causal: bool = False, scale: Optional[float] = None,
                          n_keys: Optional[Sequence[int]] = None, mask=None):
    """Per-element pure-Python evaluation for tiny shapes (no numpy arithmetic).

    q [B][Hq][Lq][d], k and v [B][Hkv][Lk][d] as nested sequences; n_keys
    optionally limits the keys seen by batch b (decode lengths); mask
    [B][Hq][Lq][Lk] of booleans (False removes the pair) or numbers (added to
    the scaled score).  Every score
    is a math.fsum of products; every row is normalised with math.fsum.
    Returns nested lists O [B][Hq][Lq][d] and LSE [B][Hq][Lq].
    """
    B, Hq = len(q), len(q[0])
    Hkv = len(k[0])
    d = len(q[0][0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = Hq // Hkv
    O, LSE = [], []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(Hq):
            hk = h // group
            keys = k[b][hk]
            vals = v[b][hk]
            nk = len(keys) if n_keys is None else min(int(n_keys[b]), len(keys))
            Oh, Lh = [], []
            for i, qi in enumerate(q[b][h]):
                visible = [j for j in range(nk) if not (causal and j > i)]
                add = {}
                if mask is not None:
                    mrow = mask[b][h][i]
                    if isinstance(mrow[0], (bool, np.bool_)):
                        visible = [j for j in visible if mrow[j]]
                    else:
                        add = {j: float(mrow[j]) for j in visible}
                if not visible:
                    Oh.append([0.0] * len(vals[0]) if vals else [])
                    Lh.append(-math.inf)
                    continue
                s = {j: math.fsum(float(qi[t]) * float(keys[j][t]) for t in range(d)) * scale
                     + add.get(j, 0.0) for j in visible}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in visible}
                l = math.fsum(e.values())
                Oh.append([math.fsum(e[j] * float(vals[j][c]) for j in visible) / l
                           for c in range(len(vals[0]))])
                Lh.append(m + math.log(l))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        LSE.append(Lb)
    return O, LSE


# ---------------------------------------------------------------------------
# FP8 inputs.  An e4m3 code is 1 sign bit, 4 exponent bits (bias 7) and 3
# mantissa bits: exponent field e in 1..15 gives (1 + m/8) 2^(e-7), field 0
# gives the subnormals (m/8) 2^-6, and the one pattern with every exponent and
# mantissa bit set is not a number (there is no infinity).  The largest finite
# value is 1.75 * 2^8 = 448.

def e4m3_decode(codes) -> np.ndarray:
    """Values of e4m3 codes (uint8, any shape) as float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, val)


def dequantize_e4m3(codes, descale: float) -> np.ndarray:
    """The values a tensor of e4m3 codes stands for: descale * value(code)."""
    if hasattr(codes, "numpy"):
        codes = codes.numpy()
    return e4m3_decode(codes) * float(descale)


def attention_forward_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                          causal: bool = False, scale: Optional[float] = None,
                          threads: Optional[int] = None, return_sp: bool = False):
    """Prefill attention of FP8 inputs: q8 [B,Hq,Lq,d], k8 and v8 [B,Hkv,Lk,d]
    e4m3 codes with one descale each.  Exactly attention_forward applied to
    the dequantised values; returns O [B,Hq,Lq,d] and LSE [B,Hq,Lq] (and S, P
    with return_sp)."""
    return attention_forward(dequantize_e4m3(q8, q_descale), dequantize_e4m3(k8, k_descale),
                             dequantize_e4m3(v8, v_descale), causal=causal, scale=scale,
                             threads=threads, return_sp=return_sp)


def attention_forward_fp8_rows(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                               b: int, h: int, rows: Iterable[int], causal: bool = False,
                               scale: Optional[float] = None, return_sp: bool = False):
    """attention_forward_fp8 for a few query rows of one (batch, query head);
    only that head's codes are dequantised.  Returns O [len(rows), d], LSE
    (and the rows of S and P with return_sp)."""
    Hq, Hkv = q8.shape[1], k8.shape[1]
    hk = h // (Hq // Hkv)
    rows = np.asarray(list(rows), dtype=np.int64)
    if scale is None:
        scale = default_scale(q8.shape[-1])
    q = dequantize_e4m3(q8[b, h], q_descale)[rows]
    return _head_attention(q, dequantize_e4m3(k8[b, hk], k_descale), dequantize_e4m3(v8[b, hk], v_descale),
                           scale, causal, row_ids=rows, return_sp=return_sp)
