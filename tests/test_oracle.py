"""Pins on the CPU oracle: facts fixed by the pages and by mathematics, not by
the oracle itself.  No GPU needed.

Each test names the part of the oracle a plausible slip would break (a dropped
term, a wrong sign or index, a transposed operand); test_planted_mistakes
checks that the pins do catch such slips.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sdpa_oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def rnd(shape, seed, mul=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mul


# ---------------------------------------------------------------- P-1 softmax
@pytest.mark.parametrize("causal", [False, True])
def test_prob_rows_sum_to_one(causal):
    q, k, v = rnd((2, 3, 17, 8), 1), rnd((2, 3, 17, 8), 2), rnd((2, 3, 17, 8), 3)
    _, _, s, p = orc.attention_forward(q, k, v, causal=causal, return_sp=True)
    assert np.abs(p.sum(-1) - 1.0).max() <= 1e-13
    assert (p >= 0).all()
    if causal:
        iu = np.triu_indices(17, 1)
        assert (p[..., iu[0], iu[1]] == 0).all()
        assert np.isneginf(s[..., iu[0], iu[1]]).all()


# ------------------------------------------------------ P-2 constant V rows
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_return_the_constant(causal):
    q, k = rnd((1, 2, 23, 16), 4, 3.0), rnd((1, 2, 23, 16), 5)
    c = rnd((16,), 6)
    v = np.broadcast_to(c, (1, 2, 23, 16)).copy()
    o, _ = orc.attention_forward(q, k, v, causal=causal)
    assert np.abs(o - c).max() <= 1e-13


# ------------------------------------------------------- P-3 causal row 0
def test_causal_first_row_is_first_value():
    q, k, v = rnd((1, 1, 9, 8), 7), rnd((1, 1, 9, 8), 8), rnd((1, 1, 9, 8), 9)
    o, lse = orc.attention_forward(q, k, v, causal=True)
    assert np.abs(o[0, 0, 0] - v[0, 0, 0]).max() <= 1e-15
    s00 = float(np.dot(q[0, 0, 0], k[0, 0, 0])) / math.sqrt(8)
    assert abs(lse[0, 0, 0] - s00) <= 1e-14


# --------------------------------------------------- P-4 brute force (fsum)
@pytest.mark.parametrize("causal,Hq,Hkv,n,d", [
    (False, 2, 2, 5, 4), (True, 2, 2, 7, 8), (False, 4, 2, 6, 8), (True, 4, 1, 16, 8),
    (False, 3, 3, 1, 4), (True, 2, 1, 3, 2)])
def test_matches_brute_force(causal, Hq, Hkv, n, d):
    B = 2
    q, k, v = rnd((B, Hq, n, d), 10, 2.0), rnd((B, Hkv, n, d), 11), rnd((B, Hkv, n, d), 12)
    o, lse = orc.attention_forward(q, k, v, causal=causal)
    ob, lb = orc.brute_force_attention(q.tolist(), k.tolist(), v.tolist(), causal=causal)
    ob, lb = np.array(ob), np.array(lb)
    assert np.abs(o - ob).max() <= 1e-12 * max(1.0, np.abs(ob).max())
    assert np.abs(lse - lb).max() <= 1e-12 * max(1.0, np.abs(lb).max())


def test_decode_matches_brute_force():
    B, Hq, Hkv, L, d = 3, 4, 2, 9, 8
    q, k, v = rnd((B, Hq, d), 13), rnd((B, Hkv, L, d), 14), rnd((B, Hkv, L, d), 15)
    lens = [9, 1, 4]
    o, lse = orc.attention_decode(q, k, v, lens)
    ob, lb = orc.brute_force_attention(q[:, :, None, :].tolist(), k.tolist(), v.tolist(),
                                       n_keys=lens)
    assert np.abs(o - np.array(ob)[:, :, 0]).max() <= 1e-12
    assert np.abs(lse - np.array(lb)[:, :, 0]).max() <= 1e-12


# ------------------------------------------- P-5 zero queries: uniform rows
@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_uniform_weights(causal):
    n = 13
    q = np.zeros((1, 1, n, 8))
    k, v = rnd((1, 1, n, 8), 16), rnd((1, 1, n, 8), 17)
    o, lse = orc.attention_forward(q, k, v, causal=causal)
    for i in range(n):
        vis = i + 1 if causal else n
        assert np.abs(o[0, 0, i] - v[0, 0, :vis].mean(0)).max() <= 1e-14
        assert abs(lse[0, 0, i] - math.log(vis)) <= 1e-14


# ----------------------------------- P-6 shifting every key by one vector
@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_moves_only_lse(causal):
    n, d = 11, 8
    q, k, v = rnd((1, 2, n, d), 18), rnd((1, 2, n, d), 19), rnd((1, 2, n, d), 20)
    u = rnd((d,), 21)
    o1, l1 = orc.attention_forward(q, k, v, causal=causal)
    o2, l2 = orc.attention_forward(q, k + u, v, causal=causal)
    assert np.abs(o1 - o2).max() <= 1e-12
    expect = l1 + (q @ u) / math.sqrt(d)
    assert np.abs(l2 - expect).max() <= 1e-12


# ---------------------------------- P-7 joint permutation of keys and values
def test_key_value_permutation_invariance():
    n, d = 19, 8
    q, k, v = rnd((2, 2, 7, d), 22), rnd((2, 2, n, d), 23), rnd((2, 2, n, d), 24)
    perm = np.random.default_rng(25).permutation(n)
    o1, l1 = orc.attention_forward(q, k, v)
    o2, l2 = orc.attention_forward(q, k[:, :, perm], v[:, :, perm])
    assert np.abs(o1 - o2).max() <= 1e-13 and np.abs(l1 - l2).max() <= 1e-13
    # A single key row moved without its value row must change the result.
    k3 = k.copy()
    k3[:, :, [0, 1]] = k3[:, :, [1, 0]]
    o3, _ = orc.attention_forward(q, k3, v)
    assert np.abs(o1 - o3).max() > 1e-3


# ----------------------------------------------- P-8 grouped-query heads
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_expanded_mha(causal):
    B, Hq, Hkv, n, d = 2, 8, 2, 10, 8
    q, k, v = rnd((B, Hq, n, d), 26), rnd((B, Hkv, n, d), 27), rnd((B, Hkv, n, d), 28)
    o1, l1 = orc.attention_forward(q, k, v, causal=causal)
    kx = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1).numpy()
    vx = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1).numpy()
    o2, l2 = orc.attention_forward(q, kx, vx, causal=causal)
    assert np.abs(o1 - o2).max() == 0 and np.abs(l1 - l2).max() == 0
    # and head 1 must not read kv head 1 (the h % Hkv slip)
    o3, _ = orc.attention_forward(q[:, 1:2], k[:, 1:2], v[:, 1:2], causal=causal)
    assert np.abs(o1[:, 1:2] - o3).max() > 1e-3


# ------------------------------- P-9 decode = last row of causal prefill
def test_decode_is_last_row_of_causal_prefill():
    B, Hq, Hkv, Lmax, d = 3, 4, 2, 12, 8
    kc, vc = rnd((B, Hkv, Lmax, d), 29), rnd((B, Hkv, Lmax, d), 30)
    qfull = rnd((B, Hq, Lmax, d), 31)
    lens = [12, 5, 1]
    qd = np.stack([qfull[b, :, lens[b] - 1] for b in range(B)])
    o, lse = orc.attention_decode(qd, kc, vc, lens)
    for b, L in enumerate(lens):
        op, lp = orc.attention_forward(qfull[b:b + 1, :, :L], kc[b:b + 1, :, :L],
                                       vc[b:b + 1, :, :L], causal=True)
        assert np.abs(o[b] - op[0, :, L - 1]).max() <= 1e-13
        assert np.abs(lse[b] - lp[0, :, L - 1]).max() <= 1e-13


def test_decode_clamps_and_empty():
    B, Hq, Hkv, Lmax, d = 2, 2, 1, 6, 4
    q, kc, vc = rnd((B, Hq, d), 32), rnd((B, Hkv, Lmax, d), 33), rnd((B, Hkv, Lmax, d), 34)
    o, lse = orc.attention_decode(q, kc, vc, [0, 100])
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all()
    o6, l6 = orc.attention_decode(q, kc, vc, [0, 6])
    assert np.array_equal(o[1], o6[1]) and np.array_equal(lse[1], l6[1])


# ------------------------------------------- P-10 block / part merging
@pytest.mark.parametrize("cuts", [[5], [1, 2, 30], [16, 17], [0, 40]])
def test_merge_of_key_parts_equals_whole(cuts):
    n, d = 40, 8
    q, k, v = rnd((1, 3, 6, d), 35, 2.0), rnd((1, 3, n, d), 36), rnd((1, 3, n, d), 37)
    o, lse = orc.attention_forward(q, k, v)
    bounds = [0] + list(cuts) + [n]
    parts = [orc.attention_forward(q, k[:, :, a:b], v[:, :, a:b]) for a, b in zip(bounds, bounds[1:])]
    om, lm = orc.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    assert np.abs(om - o).max() <= 1e-14 and np.abs(lm - lse).max() <= 1e-13


def test_merge_all_empty_parts():
    o, l = orc.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


def test_two_key_blocks_merged_reproduce_page_demo():
    """The online-softmax demo: scores randn(2, 512, 4096) * 2 split into two
    key blocks; the page expects the blockwise result to agree with the
    standard softmax near machine precision (1e-6) in fp32.

    Each block is run through the oracle's own attention with unit keys and
    values (key j and value j are the j-th unit vector, scale 1), so that a
    query whose d-vector is its score row has exactly those scores and its
    output row is its probability row.  The two blocks' (O, LSE) pairs are
    merged with merge_partials: in float32, as the page's demo runs, against
    torch's float32 softmax; in float64 against torch's float64 softmax."""
    fig = json.load(open(GOLDEN))["online_softmax_demo"]
    x = torch.randn(*fig["shape"], generator=torch.Generator().manual_seed(0)) * fig["x_scale"]
    B, R, n = x.shape
    mid = n // 2
    q = x.numpy().astype(np.float64)[:, None]  # [B, 1, R, n]
    eye = np.eye(n)
    parts = []
    for a, b in ((0, mid), (mid, n)):
        kv = np.broadcast_to(eye[a:b], (B, 1, b - a, n))
        parts.append(orc.attention_forward(q, kv, kv, scale=1.0))
    o32, l32 = orc.merge_partials([p[0].astype(np.float32) for p in parts],
                                  [p[1].astype(np.float32) for p in parts])
    assert o32.dtype == np.float32
    ref32 = torch.softmax(x, dim=-1).numpy()[:, None]
    assert np.abs(o32 - ref32).max() <= 10 * fig["max_abs_diff_fp32_order"]
    o64, l64 = orc.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    x64 = x.double()
    assert np.abs(o64 - torch.softmax(x64, dim=-1).numpy()[:, None]).max() <= 1e-15
    assert np.abs(l64 - torch.logsumexp(x64, dim=-1).numpy()[:, None]).max() <= 1e-12


# ------------------------------------------ P-11 large score magnitudes
def test_large_scores_stay_finite_and_pick_the_max():
    n, d = 9, 8
    q, k, v = rnd((1, 1, n, d), 38, 100.0), rnd((1, 1, n, d), 39), rnd((1, 1, n, d), 40)
    o, lse, s, _ = orc.attention_forward(q, k, v, return_sp=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    for i in range(n):
        row = s[0, 0, i]
        j = int(np.argmax(row))
        assert np.abs(row).max() > 100  # far outside exp's float range unless shifted
        # |O - V_j| <= sum_{j' != j} e^(s_j' - s_j) |V_j' - V_j|, and
        # 0 <= LSE - s_j = ln(1 + sum_{j' != j} e^(s_j' - s_j)) <= that sum.
        w = np.exp(np.delete(row, j) - row[j])
        dv = np.abs(np.delete(v[0, 0], j, axis=0) - v[0, 0, j]).max(-1)
        assert np.abs(o[0, 0, i] - v[0, 0, j]).max() <= (w * dv).sum() + 1e-12
        assert -1e-12 <= lse[0, 0, i] - row[j] <= w.sum() + 1e-12


# ------------------------------------------------------------ P-12 n = 1
def test_single_key():
    q, k, v = rnd((2, 2, 1, 8), 41), rnd((2, 2, 1, 8), 42), rnd((2, 2, 1, 8), 43)
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, causal=causal)
        assert np.abs(o - v).max() <= 1e-15
        s = (q * k).sum(-1) / math.sqrt(8)
        assert np.abs(lse - s).max() <= 1e-14


def test_no_keys():
    q = rnd((1, 1, 3, 4), 44)
    o, lse = orc.attention_forward(q, np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 0, 4)))
    assert (o == 0).all() and np.isneginf(lse).all()


# ------------------------------------------------ P-13 independent library
@pytest.mark.parametrize("causal,Hq,Hkv", [(False, 4, 4), (True, 4, 4), (True, 8, 2)])
def test_matches_torch_sdpa_float64(causal, Hq, Hkv):
    B, n, d = 2, 33, 16
    q, k, v = rnd((B, Hq, n, d), 45, 2.0), rnd((B, Hkv, n, d), 46), rnd((B, Hkv, n, d), 47)
    o, lse, s, _ = orc.attention_forward(q, k, v, causal=causal, return_sp=True)
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, 1)
    tv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal).numpy()
    assert np.abs(o - ref).max() <= 1e-12
    ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
    assert np.abs(lse - ref_lse).max() <= 1e-12


def test_explicit_scale():
    q, k, v = rnd((1, 2, 7, 8), 48), rnd((1, 2, 7, 8), 49), rnd((1, 2, 7, 8), 50)
    o, _ = orc.attention_forward(q, k, v, scale=0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.3).numpy()
    assert np.abs(o - ref).max() <= 1e-12


# --------------------------------------- sampled rows = the same definition
def test_rows_helper_agrees_with_full():
    q, k, v = rnd((2, 4, 30, 8), 51), rnd((2, 2, 30, 8), 52), rnd((2, 2, 30, 8), 53)
    o, lse = orc.attention_forward(q, k, v, causal=True)
    rows = [0, 7, 29]
    orow, lrow = orc.attention_forward_rows(q, k, v, 1, 3, rows, causal=True)
    assert np.array_equal(orow, o[1, 3, rows]) and np.array_equal(lrow, lse[1, 3, rows])


def test_threaded_equals_serial():
    q, k, v = rnd((2, 6, 20, 8), 54), rnd((2, 3, 20, 8), 55), rnd((2, 3, 20, 8), 56)
    a = orc.attention_forward(q, k, v, causal=True, threads=1)
    b = orc.attention_forward(q, k, v, causal=True, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------ page figures for the accounting
def test_accounting_matches_page_figures():
    fig = json.load(open(GOLDEN))
    MB, GB, KB = 2 ** 20, 2 ** 30, 2 ** 10
    assert wl.score_matrix_bytes(4096) / MB == fig["score_matrix_fp32_n4096_MB"]["value"]
    tot = wl.score_matrix_bytes(4096) * 96 * 40 / GB
    assert abs(tot - fig["score_matrix_fp32_n4096_h96_l40_GB"]["value"]) <= \
        fig["score_matrix_fp32_n4096_h96_l40_GB"]["tolerance_rel"] * tot
    assert 2 * wl.score_matrix_bytes(4096) / MB == fig["score_plus_prob_fp32_n4096_MB"]["value"]
    # Q, K, V, O + LSE for one head in fp32; Q/K/V alone is the page's 3.0 MB
    qkv = wl.algorithmic_bytes_fwd(1, 1, 1, 4096, 4096, 64, 4) - 4096 * 64 * 4 - 4096 * 4
    assert qkv / MB == fig["qkv_fp32_n4096_d64_one_head_MB"]["value"]
    assert 2 * 4096 * 4 / KB == fig["row_stats_fp32_n4096_KB"]["value"]
    assert 2 * wl.score_matrix_bytes(4096) // (2 * 4096 * 4) == fig["stats_saving_ratio_n4096"]["value"]


def test_workload_flop_counts():
    assert wl.algorithmic_flops_fwd(1, 96, 4096, 4096, 64, False) == 412_316_860_416
    assert wl.algorithmic_flops_fwd(4, 16, 2048, 2048, 80, True) == 42_949_672_960
    assert wl.algorithmic_flops_fwd(1, 32, 8192, 8192, 128, True) == 549_755_813_888


def test_input_recipe_is_bf16_round_to_nearest_even():
    """The bf16 inputs are torch's RNE rounding of the float32 draws; check it
    against a bit-level round-to-nearest-even written out here."""
    x = torch.randn(200_000, generator=torch.Generator().manual_seed(3)) * 3
    bits = x.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = x.to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(rounded, got)


# ------------------------------------- P-14 cross-attention, Lq != Lk
@pytest.mark.parametrize("Lq,Lk", [(5, 9), (9, 5), (1, 7), (7, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_cross_attention_matches_brute_force(Lq, Lk, causal):
    q, k, v = rnd((1, 2, Lq, 4), 70, 2.0), rnd((1, 2, Lk, 4), 71), rnd((1, 2, Lk, 4), 72)
    o, lse = orc.attention_forward(q, k, v, causal=causal)
    ob, lb = orc.brute_force_attention(q.tolist(), k.tolist(), v.tolist(), causal=causal)
    assert np.abs(o - np.array(ob)).max() <= 1e-12
    assert np.abs(lse - np.array(lb)).max() <= 1e-12


@pytest.mark.parametrize("Lq,Lk", [(20, 33), (33, 20)])
def test_cross_attention_causal_matches_torch_sdpa_float64(Lq, Lk):
    # torch's is_causal is top-left (a lower-triangular L x S mask), the reading taken
    q, k, v = rnd((2, 4, Lq, 16), 73, 2.0), rnd((2, 4, Lk, 16), 74), rnd((2, 4, Lk, 16), 75)
    o, _ = orc.attention_forward(q, k, v, causal=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    assert np.abs(o - ref).max() <= 1e-12


def test_causal_rows_past_the_last_key_see_every_key():
    # top-left with Lq > Lk: rows i >= Lk - 1 see all keys, i.e. equal the non-causal rows
    q, k, v = rnd((1, 2, 30, 8), 76), rnd((1, 2, 12, 8), 77), rnd((1, 2, 12, 8), 78)
    oc, lc = orc.attention_forward(q, k, v, causal=True)
    on, ln = orc.attention_forward(q, k, v, causal=False)
    assert np.array_equal(oc[:, :, 11:], on[:, :, 11:]) and np.array_equal(lc[:, :, 11:], ln[:, :, 11:])
    assert np.abs(oc[:, :, :11] - on[:, :, :11]).max() > 1e-3


# ------------------------------------------- P-15 packed variable length
VARLEN_CASES = [  # (query lengths, key lengths)
    ([3, 0, 5, 1], [4, 2, 5, 3]),   # an empty sequence
    ([2, 4], [0, 6]),               # a sequence with queries but no keys
    ([6], [6]),
    ([4, 7, 2], [7, 4, 2]),         # Lq != Lk per sequence
]


@pytest.mark.parametrize("case", range(len(VARLEN_CASES)))
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_brute_force_per_sequence(case, causal):
    lq, lk = VARLEN_CASES[case]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    Hq, Hkv, d = 4, 2, 4
    q = rnd((cu_q[-1], Hq, d), 80 + case, 2.0)
    k, v = rnd((cu_k[-1], Hkv, d), 90 + case), rnd((cu_k[-1], Hkv, d), 100 + case)
    o, lse = orc.attention_forward_varlen(q, k, v, cu_q, cu_k, causal=causal)
    for b in range(len(lq)):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe == qs:
            continue
        qb = q[qs:qe].transpose(1, 0, 2)[None]   # [1, Hq, Lq_b, d]
        kb = k[ks:ke].transpose(1, 0, 2)[None]
        vb = v[ks:ke].transpose(1, 0, 2)[None]
        ob, lb = orc.brute_force_attention(qb.tolist(), kb.tolist(), vb.tolist(), causal=causal)
        ob = np.array(ob)[0].transpose(1, 0, 2) if ke > ks else np.zeros((qe - qs, Hq, d))
        assert np.abs(o[qs:qe] - ob).max() <= 1e-12
        assert np.array_equal(np.isneginf(lse[:, qs:qe]), np.isneginf(np.array(lb)[0]))
        fin = np.isfinite(np.array(lb)[0])
        assert np.abs(lse[:, qs:qe][fin] - np.array(lb)[0][fin]).max(initial=0.0) <= 1e-12
    if 0 in lk:  # rows of a sequence without keys
        b = lk.index(0)
        assert (o[cu_q[b]:cu_q[b + 1]] == 0).all() and np.isneginf(lse[:, cu_q[b]:cu_q[b + 1]]).all()


def test_varlen_single_sequence_is_dense():
    q, k, v = rnd((1, 4, 9, 8), 110), rnd((1, 2, 11, 8), 111), rnd((1, 2, 11, 8), 112)
    o, lse = orc.attention_forward(q, k, v, causal=True)
    ov, lv = orc.attention_forward_varlen(q[0].transpose(1, 0, 2), k[0].transpose(1, 0, 2),
                                          v[0].transpose(1, 0, 2), [0, 9], [0, 11], causal=True)
    assert np.array_equal(ov, o[0].transpose(1, 0, 2)) and np.array_equal(lv, lse[0])


# ---------------------------------------------------- P-17 attention masks
def _masks(shape, seed):
    r = np.random.default_rng(seed)
    bm = r.random(shape) < 0.7
    bm[..., 0] = True                      # every row keeps a key (torch gives NaN otherwise)
    am = r.standard_normal(shape) * 2.0
    return bm, am


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_mask_matches_brute_force(causal, kind):
    q, k, v = rnd((1, 2, 6, 4), 140, 2.0), rnd((1, 2, 8, 4), 141), rnd((1, 2, 8, 4), 142)
    bm, am = _masks((1, 2, 6, 8), 143)
    m = bm if kind == "bool" else am
    o, lse = orc.attention_forward(q, k, v, causal=causal, attn_mask=m)
    ob, lb = orc.brute_force_attention(q.tolist(), k.tolist(), v.tolist(), causal=causal, mask=m.tolist())
    assert np.abs(o - np.array(ob)).max() <= 1e-12 and np.abs(lse - np.array(lb)).max() <= 1e-12


@pytest.mark.parametrize("kind", ["bool", "add"])
def test_mask_matches_torch_sdpa_float64(kind):
    q, k, v = rnd((2, 4, 19, 16), 144, 2.0), rnd((2, 4, 27, 16), 145), rnd((2, 4, 27, 16), 146)
    bm, am = _masks((2, 1, 19, 27), 147)          # broadcast over heads
    m = bm if kind == "bool" else am
    o, _ = orc.attention_forward(q, k, v, attn_mask=m)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(m)).numpy()
    assert np.abs(o - ref).max() <= 1e-12


def test_mask_closed_forms():
    q, k, v = rnd((1, 2, 9, 8), 148), rnd((1, 2, 9, 8), 149), rnd((1, 2, 9, 8), 150)
    o, lse = orc.attention_forward(q, k, v, causal=True)
    # all-True boolean mask = no mask
    o1, l1 = orc.attention_forward(q, k, v, causal=True, attn_mask=np.ones((9, 9), bool))
    assert np.array_equal(o1, o) and np.array_equal(l1, lse)
    # a constant per row added to every score leaves O and shifts LSE by that constant
    c = rnd((9, 1), 151)
    o2, l2 = orc.attention_forward(q, k, v, causal=True, attn_mask=np.broadcast_to(c, (9, 9)))
    assert np.abs(o2 - o).max() <= 1e-12 and np.abs(l2 - (lse + c[:, 0])).max() <= 1e-12
    # a boolean mask that keeps only key 0 makes every row return V[0]
    m = np.zeros((9, 9), bool)
    m[:, 0] = True
    o3, _ = orc.attention_forward(q, k, v, attn_mask=m)
    assert np.abs(o3 - v[:, :, :1]).max() <= 1e-15


def test_fully_masked_row_gives_zero_and_minus_inf():
    q, k, v = rnd((1, 1, 4, 4), 152), rnd((1, 1, 5, 4), 153), rnd((1, 1, 5, 4), 154)
    m = np.ones((4, 5), bool)
    m[2] = False
    o, lse = orc.attention_forward(q, k, v, attn_mask=m)
    assert (o[0, 0, 2] == 0).all() and np.isneginf(lse[0, 0, 2]) and np.isfinite(lse[0, 0, [0, 1, 3]]).all()
    ob, lb = orc.brute_force_attention(q.tolist(), k.tolist(), v.tolist(), mask=m[None, None].tolist())
    assert np.abs(o - np.array(ob)).max() <= 1e-12


# --------------------------------------------------- P-16 backward pass
def _loss(q, k, v, w, causal):
    o, _ = orc.attention_forward(q, k, v, causal=causal)
    return float((o * w).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk", [(5, 5), (4, 7)])
def test_backward_matches_finite_differences(causal, Lq, Lk):
    """Central differences of sum(O * W) need no derivation at all."""
    q, k, v = rnd((1, 2, Lq, 4), 120), rnd((1, 1, Lk, 4), 121), rnd((1, 1, Lk, 4), 122)
    w = rnd((1, 2, Lq, 4), 123)
    dq, dk, dv = orc.attention_backward(q, k, v, w, causal=causal)
    eps = 1e-6
    rng = np.random.default_rng(124)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], w, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], w, causal)
            assert abs((lp - lm) / (2 * eps) - g[idx]) <= 1e-7, (name, idx)


@pytest.mark.parametrize("causal,Hq,Hkv,Lq,Lk", [(False, 4, 4, 33, 33), (True, 4, 4, 33, 33),
                                                 (True, 8, 2, 20, 29), (False, 8, 2, 29, 20)])
def test_backward_matches_torch_autograd_float64(causal, Hq, Hkv, Lq, Lk):
    q, k, v = rnd((2, Hq, Lq, 16), 125, 2.0), rnd((2, Hkv, Lk, 16), 126), rnd((2, Hkv, Lk, 16), 127)
    do = rnd((2, Hq, Lq, 16), 128)
    dq, dk, dv = orc.attention_backward(q, k, v, do, causal=causal)
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    g = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk.repeat_interleave(g, 1),
                                                         tv.repeat_interleave(g, 1), is_causal=causal)
    o.backward(torch.from_numpy(do))
    assert np.abs(dq - tq.grad.numpy()).max() <= 1e-12
    assert np.abs(dk - tk.grad.numpy()).max() <= 1e-12
    assert np.abs(dv - tv.grad.numpy()).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    q, k, v, do = rnd((1, 2, 11, 8), 129), rnd((1, 2, 11, 8), 130), rnd((1, 2, 11, 8), 131), rnd((1, 2, 11, 8), 132)
    dq, dk, dv = orc.attention_backward(q, k, v, do, causal=causal)
    # each score row's dS sums to zero, so the key gradients sum to zero over keys
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12
    # each probability row sums to one, so the value gradients sum to the output gradients
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() <= 1e-12
    # identical value rows make O independent of the scores: no gradient reaches Q or K
    vc = np.broadcast_to(v[:, :, :1], v.shape).copy()
    dq0, dk0, _ = orc.attention_backward(q, k, vc, do, causal=causal)
    assert np.abs(dq0).max() <= 1e-12 and np.abs(dk0).max() <= 1e-12


# -------------------------------------------- planted mistakes are caught
def _mutant(kind):
    """Copies of the oracle's per-head step with one plausible slip each."""
    def f(q, k, v, scale, causal, row_ids=None, n_keys=None, return_sp=False, mask=None):
        if kind == "scale_1_over_d":
            scale = scale * scale
        s = (q @ k.T) * scale
        if mask is not None:
            s = np.where(mask, s, -np.inf) if np.asarray(mask).dtype == bool else s + mask
        if kind == "transposed" and s.shape[0] == s.shape[1]:
            s = s.T.copy()
        n_rows, lk = s.shape
        rid = np.arange(n_rows) if row_ids is None else row_ids
        if causal:
            off = 1 if kind == "mask_off_by_one" else 0
            s = np.where(np.arange(lk)[None, :] > rid[:, None] + off, -np.inf, s)
        m = s.max(-1)
        e = np.exp(s - m[:, None])
        l = e.sum(-1)
        p = e / l[:, None]
        o = (p @ v) if kind != "unnormalised" else (e @ v)
        lse = m + np.log(l) if kind != "lse_drops_max" else np.log(l)
        if return_sp:
            return o, lse, s, p
        return o, lse
    return f


@pytest.mark.parametrize("kind", ["scale_1_over_d", "transposed", "mask_off_by_one",
                                  "unnormalised", "lse_drops_max"])
def test_planted_mistakes(monkeypatch, kind):
    monkeypatch.setattr(orc, "_head_attention", _mutant(kind))
    failures = 0
    for fn in (lambda: test_matches_torch_sdpa_float64(True, 4, 4),
               lambda: test_causal_first_row_is_first_value(),
               lambda: test_key_shift_moves_only_lse(True),
               lambda: test_constant_values_return_the_constant(False),
               lambda: test_cross_attention_causal_matches_torch_sdpa_float64(20, 33),
               lambda: test_varlen_matches_brute_force_per_sequence(3, True),
               lambda: test_mask_matches_torch_sdpa_float64("add")):
        try:
            fn()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"planted mistake {kind} not caught"


@pytest.mark.parametrize("causal", [False, True])
def test_backward_sampled_is_the_same_definition(causal):
    q, k, v = rnd((2, 4, 23, 8), 133), rnd((2, 2, 23, 8), 134), rnd((2, 2, 23, 8), 135)
    do = rnd((2, 4, 23, 8), 136)
    dq, dk, dv = orc.attention_backward(q, k, v, do, causal=causal)
    rows, keys = [0, 9, 22], [1, 11, 22]
    sq, sk, sv = orc.attention_backward_sampled(q, k, v, do, 1, 1, rows, keys, causal=causal)
    assert np.abs(sq - dq[1, 2:4][:, rows]).max() <= 1e-12
    assert np.abs(sk - dk[1, 1, keys]).max() <= 1e-12 and np.abs(sv - dv[1, 1, keys]).max() <= 1e-12


def _backward_mutant(kind):
    """Copies of the oracle's per-head backward with one plausible slip each."""
    def f(q, k, v, do, scale, causal):
        lq, lk = q.shape[0], k.shape[0]
        if lk == 0 or lq == 0:
            return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        _, _, s, p = orc._head_attention(q, k, v, scale, causal, return_sp=True)
        dv = (p.T @ do) if kind != "dv_untransposed" else (p[:lk, :lq] @ do[:lk]) if lq == lk else p.T @ do * 2
        dp = do @ v.T
        dsum = (p * dp).sum(axis=-1, keepdims=True) if kind != "no_softmax_correction" else 0.0
        ds = p * (dp - dsum)
        dq = (ds @ k) * (scale if kind != "dq_no_scale" else 1.0)
        dk = (ds.T @ q) * scale if kind != "dk_from_dq_side" else (ds @ q[:lk]) * scale if lq == lk else ds.T @ q
        return dq, dk, dv
    return f


@pytest.mark.parametrize("kind", ["dv_untransposed", "no_softmax_correction", "dq_no_scale", "dk_from_dq_side"])
def test_planted_backward_mistakes(monkeypatch, kind):
    monkeypatch.setattr(orc, "_head_backward", _backward_mutant(kind))
    failures = 0
    for fn in (lambda: test_backward_matches_finite_differences(True, 5, 5),
               lambda: test_backward_matches_torch_autograd_float64(True, 4, 4, 33, 33),
               lambda: test_backward_invariants(False)):
        try:
            fn()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"planted backward mistake {kind} not caught"


# ---------------------------------------------------------- P-18 FP8 inputs
def test_e4m3_decode_matches_torch_and_the_format():
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref, equal_nan=True)
    # closed forms of the format: unit, largest, smallest subnormal, smallest normal, NaN, -0
    assert ours[0x38] == 1.0 and ours[0xb8] == -1.0 and ours[0x7e] == 448.0 and ours[0xfe] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x07] == 7 * 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7f]) and np.isnan(ours[0xff]) and ours[0x80] == 0 and np.signbit(ours[0x80])
    # the 127 non-negative finite codes are strictly increasing; the sign bit mirrors them
    pos = ours[:0x7f]
    assert np.all(np.diff(pos) > 0) and np.array_equal(ours[0x80:0xff], -pos)
    # 8 codes per binade, evenly spaced: binade e (codes 8e .. 8e+7) steps by 2^(e-10), the
    # subnormals by 2^-9 like binade 1
    step = np.diff(pos)
    assert (step[:8] == 2.0 ** -9).all()
    for e in range(1, 16):
        assert (step[8 * e: min(8 * e + 7, 126)] == 2.0 ** (e - 10)).all()


# values of a few codes, from the format's definition worked by hand
E4M3_BY_HAND = {0x00: 0.0, 0x38: 1.0, 0xb8: -1.0, 0x40: 2.0, 0xc0: -2.0, 0x30: 0.5, 0xb0: -0.5,
                0x3c: 1.5, 0x44: 3.0, 0xc4: -3.0, 0x04: 2.0 ** -7, 0x2e: 0.4375}


def _hand_codes(shape, seed):
    keys = np.array(sorted(E4M3_BY_HAND), dtype=np.uint8)
    return np.random.default_rng(seed).choice(keys, size=shape).astype(np.uint8)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_matches_brute_force_on_hand_decoded_values(causal):
    q8, k8, v8 = _hand_codes((1, 4, 6, 8), 160), _hand_codes((1, 2, 7, 8), 161), _hand_codes((1, 2, 7, 8), 162)
    dq, dk, dv = 0.75, 1.25, -0.5
    o, lse = orc.attention_forward_fp8(q8, k8, v8, dq, dk, dv, causal=causal)
    val = np.vectorize(lambda c: E4M3_BY_HAND[int(c)])
    ob, lb = orc.brute_force_attention((val(q8) * dq).tolist(), (val(k8) * dk).tolist(), (val(v8) * dv).tolist(),
                                       causal=causal)
    assert np.abs(o - np.array(ob)).max() <= 1e-12 and np.abs(lse - np.array(lb)).max() <= 1e-12


def test_fp8_descale_invariants():
    r = np.random.default_rng(163)
    q8, k8, v8 = (r.integers(0, 256, (1, 2, 9, 16)) for _ in range(3))
    q8, k8, v8 = (np.where((c & 0x7f) == 0x7f, 0, c).astype(np.uint8) for c in (q8, k8, v8))  # no NaN codes
    o, lse = orc.attention_forward_fp8(q8, k8, v8, 0.01, 0.02, 0.03, causal=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    # the scores see only the product q_descale * k_descale * scale
    o1, l1 = orc.attention_forward_fp8(q8, k8, v8, 0.02, 0.01, 0.03, causal=True)
    o2, l2 = orc.attention_forward_fp8(q8, k8, v8, 0.0002, 1.0, 0.03, causal=True, scale=0.25)
    for a, b in ((o1, o), (o2, o)):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(o).max())
    assert np.abs(l1 - lse).max() <= 1e-12 and np.abs(l2 - lse).max() <= 1e-12
    # O is linear in the value descale, LSE does not see it
    o3, l3 = orc.attention_forward_fp8(q8, k8, v8, 0.01, 0.02, 0.06, causal=True)
    assert np.array_equal(o3, 2 * o) and np.array_equal(l3, lse)
    # the rows helper is the same definition
    orow, lrow = orc.attention_forward_fp8_rows(q8, k8, v8, 0.01, 0.02, 0.03, 0, 1, [0, 4, 8], causal=True)
    assert np.abs(orow - o[0, 1, [0, 4, 8]]).max() <= 1e-13 and np.abs(lrow - lse[0, 1, [0, 4, 8]]).max() <= 1e-13


def test_fp8_recipe_codes_stand_for_the_drawn_values():
    w = wl.shrink(wl.C8, Lq=40, Lk=40)
    q8, k8, v8, ds = wl.make_fp8_inputs(w)
    g = torch.Generator().manual_seed(w.seed)
    x = torch.randn((w.B, w.Hq, w.Lq, w.d), generator=g, dtype=torch.float32).double().numpy()
    deq = orc.dequantize_e4m3(q8, ds[0])
    # every code is the nearest e4m3 value: within half a step (2^-4 relative, 2^-10 absolute at the bottom)
    err = np.abs(deq - x) / ds[0]
    assert (err <= np.maximum(np.abs(x / ds[0]) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)).all()
    assert np.abs(deq).max() == pytest.approx(np.abs(x).max(), rel=1e-6)  # the largest maps to 448


def _fp8_mutant(kind):
    def f(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where((c & 0x80) != 0, -1.0, 1.0)
        e, m = (c >> 3) & 0xF, (c & 7).astype(np.float64)
        bias = 8.0 if kind == "bias_8" else 7.0
        normal = (1.0 + m / 8.0) * np.exp2(e - bias)
        sub = (m / 8.0) * 2.0 ** (-6 if kind != "subnormal_exponent" else -7)
        if kind == "no_subnormals":
            sub = np.zeros_like(sub)
        val = sign * np.where(e == 0, sub, normal)
        if kind == "sign_ignored":
            val = np.abs(val)
        return np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return f


@pytest.mark.parametrize("kind", ["bias_8", "subnormal_exponent", "no_subnormals", "sign_ignored", "v_descale_dropped"])
def test_planted_fp8_mistakes(monkeypatch, kind):
    if kind == "v_descale_dropped":
        real = orc.dequantize_e4m3
        calls = []

        def deq(codes, descale):
            calls.append(descale)
            return real(codes, 1.0 if len(calls) % 3 == 0 else descale)
        monkeypatch.setattr(orc, "dequantize_e4m3", deq)
    else:
        monkeypatch.setattr(orc, "e4m3_decode", _fp8_mutant(kind))
    failures = 0
    for fn in (test_e4m3_decode_matches_torch_and_the_format,
               lambda: test_fp8_attention_matches_brute_force_on_hand_decoded_values(True),
               test_fp8_descale_invariants):
        try:
            fn()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"planted FP8 mistake {kind} not caught"
