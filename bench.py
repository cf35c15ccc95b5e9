"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over synthetic, HBM-resident inputs:
  1. attn_fwd, non-causal, B=1, H=96, n=4096, d=64, bf16     (headline workload)
  2. attn_fwd, causal GQA, B=1, Hq=32, Hkv=8, n=8192, d=128, bf16
  3. attn_decode, B=64, Hq=32, Hkv=8, d=128, cache lengths U{1024..8192}, bf16
Each call is timed with HIP events recorded on the stream the kernels run on
(median, minimum, maximum and mean per call are reported; rates use the
median); the step as a whole is timed with host clocks between device
synchronisations.  The host-side cost of a call (argument checks, marshalling
and the launches, no device synchronisation) is timed separately with a CPU
clock, through the Python binding and through the bare C entry point.
After the step loop, attn_fwd_varlen on 16 packed causal GQA sequences of
256..4096 tokens (d=128), attn_bwd on the causal GQA n=8192 d=128 workload
and on the same shape at d=64 (where the dQ kernel runs beside dK/dV),
attn_fwd_masked on the n=4096 d=64 workload with one boolean mask shared by
all heads, attn_fwd_fp8 on e4m3 versions of the two prefill workloads,
attn_fwd on the causal B=4, H=16, n=2048, d=80 workload (the head size that
is not a power of two), and
the headline shape at n = 2048, 4096 and 8192 (the time should grow 4x per
doubling of n) are timed the same way, each on its own, and reported in
`extra` (they are not part of the step).

Prints ONE JSON line.  `value` is the headline workload's attention-forward
throughput in TFLOP/s (credited flops 4 n^2 d H B, halved when causal).
`roofline` covers the headline kernel; the other two calls are reported in
`extra` with their own rooflines (bf16 matrix peak for prefill, HBM peak for
decode).  `cpu_baseline` times the CPU oracle on a bounded sample of the
headline workload (`value`), and per workload: the fp32 n=256 case, the
headline, the d=80 causal workload and the decode workload with every host
thread it may use and on one core, and four query heads of the n=8192 causal
workload; it records the host's CPU model and core count.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 matrix peak (twice the bf16 rate)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E peak
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "scaled_dot_product_qk_amd", "csrc", f)
                  for f in ("attn_api.hip", "device_common.h", "fwd_bf16.h", "fwd_f32.h", "fwd_fp8.h", "decode.h",
                            "bwd_bf16.h")]


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed, so
    that counters stay attached to a build whose code has not changed."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counted_traffic(tag: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary for
    this kernel, or None if there is none or the kernel sources changed since
    the counters were taken."""
    path = os.path.join(PROFILES, f"{tag}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--only", choices=["all", "fwd_n4096", "fwd_causal_n8192", "decode", "fwd_varlen", "bwd", "bwd_d64",
                                       "fwd_scaling",
                                       "fwd_masked", "fwd_fp8_n4096", "fwd_fp8_causal_n8192", "fwd_c3_d80"],
                    default="all",
                    help="time one call of the step only (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=96)
    ap.add_argument("--no-host-timing", action="store_true", help="skip the host-side cost per call")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 256 * 2 ** 20  # bytes
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def host_info():
    """The machine the CPU legs run on: logical CPUs, the CPUs this process
    may use, and the CPU model."""
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count() or 1, "usable_cpus": usable, "cpu_model": model}


def _timed(fn, threads):
    """Wall time of fn(threads); one thread also pins BLAS to one thread."""
    from threadpoolctl import threadpool_limits
    if threads == 1:
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            fn(1)
            return time.perf_counter() - t0
    t0 = time.perf_counter()
    fn(threads)
    return time.perf_counter() - t0


def cpu_baseline(q, k, v, heads: int, gpu_ms=None):
    """The CPU oracle (untuned) on `heads` whole heads of the headline
    workload (the reported value), then on the other workloads, each on a
    bounded sample, with every host thread it may use (at most 16) and on
    one core.  gpu_ms maps a workload to the GPU's median time for the whole
    workload, for the oracle-to-GPU ratio."""
    from oracle import sdpa_oracle as orc
    import workloads as wl
    gpu_ms = gpu_ms or {}
    host = host_info()
    cap = min(host["usable_cpus"], 16)
    threads = min(cap, heads)
    idx = list(range(heads))
    dt = _timed(lambda t: orc.attention_forward(q[:, idx], k[:, idx], v[:, idx], causal=False, threads=t), threads)
    B, _, L, d = q.shape
    flops = wl.algorithmic_flops_fwd(B, heads, L, L, d, False)
    per = {}

    def fwd_leg(label, w, inputs, sl, threads_, note):
        qq, kk, vv = inputs
        qs, ks, vs = qq[sl[0], sl[1]], kk[sl[0], sl[2]], vv[sl[0], sl[2]]
        t = _timed(lambda n: orc.attention_forward(qs, ks, vs, causal=w.causal, threads=n), threads_)
        f = wl.algorithmic_flops_fwd(qs.shape[0], qs.shape[1], w.Lq, w.Lk, w.d, w.causal)
        r = {"workload": w.name, "sample": note, "threads": threads_, "s": t, "tflops": f / t / 1e12}
        g = gpu_ms.get(w.name)
        if g:  # oracle time for the whole workload at this rate, over the GPU's
            r["oracle_over_gpu"] = (wl.algorithmic_flops_fwd(w.B, w.Hq, w.Lq, w.Lk, w.d, w.causal) / f * t) / (g / 1e3)
        per[label] = r

    per["fwd_n4096_d64"] = {"workload": wl.C2.name, "sample": f"{heads} of 96 heads", "threads": threads, "s": dt,
                            "tflops": flops / dt / 1e12}
    if gpu_ms.get(wl.C2.name):
        per["fwd_n4096_d64"]["oracle_over_gpu"] = (dt * 96 / heads) / (gpu_ms[wl.C2.name] / 1e3)
    all_ = slice(None)
    c1 = wl.make_fwd_inputs(wl.C1)
    fwd_leg("fwd_f32_n256_d64_1core", wl.C1, c1, (all_, all_, all_), 1, "whole workload")
    c3 = wl.make_fwd_inputs(wl.C3)
    fwd_leg("fwd_causal_n2048_d80", wl.C3, c3, (all_, all_, all_), cap, "whole workload (64 heads)")
    fwd_leg("fwd_causal_n2048_d80_1core", wl.C3, c3, (slice(0, 1), all_, all_), 1, "batch 0 (16 of 64 heads)")
    del c3
    c4 = wl.make_fwd_inputs(wl.C4)
    fwd_leg("fwd_causal_gqa_n8192_d128", wl.C4, c4, (all_, slice(0, 4), slice(0, 1)), min(cap, 4),
            "query heads 0-3 (kv head 0) of 32")
    del c4
    qd, kc, vc, lens = wl.make_decode_inputs(wl.C5)
    ln = lens.numpy()
    bd = wl.algorithmic_bytes_decode(lens.tolist(), wl.C5.Hq, wl.C5.Hkv, wl.C5.d, 2, wl.C5.Lmax)
    for label, thr, batches in (("decode_b64_d128", cap, range(wl.C5.B)), ("decode_b64_d128_1core", 1, range(16))):
        sub = wl.algorithmic_bytes_decode([int(ln[b]) for b in batches], wl.C5.Hq, wl.C5.Hkv, wl.C5.d, 2, wl.C5.Lmax)
        t = _timed(lambda n: orc.attention_decode(qd, kc, vc, ln, threads=n, batches=list(batches)), thr)
        r = {"workload": wl.C5.name, "sample": f"{len(batches)} of 64 sequences", "threads": thr, "s": t,
             "gbps": sub / t / 1e9}
        if gpu_ms.get(wl.C5.name):
            r["oracle_over_gpu"] = (bd / sub * t) / (gpu_ms[wl.C5.name] / 1e3)
        per[label] = r
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} of 96 heads (all 4096 rows each) of the n=4096 d=64 workload, "
                      f"float64 numpy, {threads} threads, {dt:.2f} s wall",
            "host": host, "per_workload": per}


def host_cost_us(fn, n=40):
    """Median, minimum and maximum host time (us) of fn(), which enqueues
    device work and returns; the device is idle before each call."""
    import torch
    ts = []
    for _ in range(n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        ts.append((time.perf_counter() - t0) * 1e6)
    torch.cuda.synchronize()
    return {"median": statistics.median(ts), "min": min(ts), "max": max(ts), "calls": n}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); multi-GPU sharding is a "
              "design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import scaled_dot_product_qk_amd as sdpa
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    SOLO = ("fwd_c3_d80", "fwd_varlen", "bwd", "bwd_d64", "fwd_masked", "fwd_fp8_n4096", "fwd_fp8_causal_n8192",
            "fwd_scaling_2048", "fwd_scaling_4096", "fwd_scaling_8192")
    names = ["fwd_n4096", "fwd_causal_n8192", "decode"] if args.only == "all" else \
        ([] if args.only in SOLO or args.only == "fwd_scaling" else [args.only])
    solo = [n for n in SOLO if args.only in ("all", n) or (args.only == "fwd_scaling" and n.startswith("fwd_scaling"))]
    with_varlen, with_bwd, with_masked = ("fwd_varlen" in solo), ("bwd" in solo), ("fwd_masked" in solo)

    # ---- inputs, generated on the host and copied once to HBM ----
    calls = {}
    if "fwd_n4096" in names:
        q2, k2, v2 = wl.make_fwd_inputs(wl.C2)
        G2 = [t.to(dev) for t in (q2, k2, v2)]
        o2 = torch.empty_like(G2[0])
        l2 = torch.empty(G2[0].shape[:3], dtype=torch.float32, device=dev)
        calls["fwd_n4096"] = lambda: sdpa.attn_fwd(*G2, causal=False, out=o2, lse=l2, stream=stream)
    if "fwd_causal_n8192" in names:
        q4, k4, v4 = wl.make_fwd_inputs(wl.C4)
        G4 = [t.to(dev) for t in (q4, k4, v4)]
        del q4, k4, v4
        o4 = torch.empty_like(G4[0])
        l4 = torch.empty(G4[0].shape[:3], dtype=torch.float32, device=dev)
        calls["fwd_causal_n8192"] = lambda: sdpa.attn_fwd(*G4, causal=True, out=o4, lse=l4, stream=stream)
    if "decode" in names:
        qd, kc, vc, lens = wl.make_decode_inputs(wl.C5)
        GD = [t.to(dev) for t in (qd, kc, vc, lens)]
        del kc, vc
        od = torch.empty_like(GD[0])
        ld = torch.empty(GD[0].shape[:2], dtype=torch.float32, device=dev)
        ws = torch.empty(sdpa.attn_decode_workspace_bytes(wl.C5.B, wl.C5.Hq, wl.C5.Lmax, wl.C5.d),
                         dtype=torch.uint8, device=dev)
        calls["decode"] = lambda: sdpa.attn_decode(*GD, workspace=ws, out=od, lse=ld, stream=stream)
    if "fwd_c3_d80" in solo:
        G3 = [t.to(dev) for t in wl.make_fwd_inputs(wl.C3)]
        o3 = torch.empty_like(G3[0])
        l3 = torch.empty(G3[0].shape[:3], dtype=torch.float32, device=dev)
        calls["fwd_c3_d80"] = lambda: sdpa.attn_fwd(*G3, causal=True, out=o3, lse=l3, stream=stream)
    if with_varlen:
        qv, kv_, vv, cqv, ckv = wl.make_varlen_inputs(wl.C6)
        GV = [t.to(dev) for t in (qv, kv_, vv, cqv, ckv)]
        lens_v = (cqv[1:] - cqv[:-1]).tolist()
        ov = torch.empty_like(GV[0])
        lv = torch.empty((wl.C6.Hq, GV[0].shape[0]), dtype=torch.float32, device=dev)
        calls["fwd_varlen"] = lambda: sdpa.attn_fwd_varlen(*GV, max(lens_v), causal=True, out=ov, lse=lv,
                                                           stream=stream)
    if with_bwd:
        qb, kb, vb = wl.make_fwd_inputs(wl.C4)
        gdo = torch.Generator().manual_seed(wl.C4.seed + 50)
        dob = torch.randn(qb.shape, generator=gdo, dtype=torch.float32).to(qb.dtype)
        GB = [t.to(dev) for t in (qb, kb, vb, dob)]
        del qb, kb, vb, dob
        ob, lb = sdpa.attn_fwd(GB[0], GB[1], GB[2], causal=True, stream=stream)
        dqb, dkb, dvb = torch.empty_like(GB[0]), torch.empty_like(GB[1]), torch.empty_like(GB[2])
        wsb = torch.empty(sdpa.attn_bwd_workspace_bytes(wl.C4.B, wl.C4.Hq, wl.C4.Lq), dtype=torch.uint8, device=dev)
        calls["bwd"] = lambda: sdpa.attn_bwd(GB[0], GB[1], GB[2], ob, lb, GB[3], causal=True, dq=dqb, dk=dkb,
                                             dv=dvb, workspace=wsb, stream=stream)
    if with_masked:
        qm, km, vm = wl.make_fwd_inputs(wl.C2)
        GM = [t.to(dev) for t in (qm, km, vm)]
        del qm, km, vm
        mm = wl.make_mask((1, 1, wl.C2.Lq, wl.C2.Lk), "bool", 1007).to(dev)
        om = torch.empty_like(GM[0])
        lm = torch.empty(GM[0].shape[:3], dtype=torch.float32, device=dev)
        calls["fwd_masked"] = lambda: sdpa.attn_fwd_masked(*GM, mm, out=om, lse=lm, stream=stream)
    C4D64 = wl.shrink(wl.C4, name="fwd_bf16_causal_gqa_b1_hq32_hkv8_n8192_d64", d=64)
    if "bwd_d64" in solo:
        q6, k6, v6 = wl.make_fwd_inputs(C4D64)
        gdo6 = torch.Generator().manual_seed(C4D64.seed + 50)
        do6 = torch.randn(q6.shape, generator=gdo6, dtype=torch.float32).to(q6.dtype)
        GB6 = [t.to(dev) for t in (q6, k6, v6, do6)]
        del q6, k6, v6, do6
        ob6, lb6 = sdpa.attn_fwd(GB6[0], GB6[1], GB6[2], causal=True, stream=stream)
        dq6, dk6, dv6 = torch.empty_like(GB6[0]), torch.empty_like(GB6[1]), torch.empty_like(GB6[2])
        ws6 = torch.empty(sdpa.attn_bwd_workspace_bytes(C4D64.B, C4D64.Hq, C4D64.Lq), dtype=torch.uint8, device=dev)
        calls["bwd_d64"] = lambda: sdpa.attn_bwd(GB6[0], GB6[1], GB6[2], ob6, lb6, GB6[3], causal=True, dq=dq6,
                                                 dk=dk6, dv=dv6, workspace=ws6, stream=stream)
    fp8_in = {}
    for n, w in (("fwd_fp8_n4096", wl.C7), ("fwd_fp8_causal_n8192", wl.C8)):
        if n in solo:
            q8, k8, v8, ds8 = wl.make_fp8_inputs(w)
            G8 = [t.to(dev) for t in (q8, k8, v8)]
            o8 = torch.empty(G8[0].shape, dtype=torch.bfloat16, device=dev)
            l8 = torch.empty(G8[0].shape[:3], dtype=torch.float32, device=dev)
            fp8_in[n] = (w, G8)
            calls[n] = (lambda G8=G8, ds8=ds8, o8=o8, l8=l8, c=w.causal:
                        sdpa.attn_fwd_fp8(*G8, ds8, causal=c, out=o8, lse=l8, stream=stream))
    # the headline shape at n = 2048, 4096, 8192: time should grow 4x per doubling of n
    scal = {}
    for n_s in (2048, 4096, 8192):
        nm = f"fwd_scaling_{n_s}"
        if nm in solo:
            ws_ = wl.FwdWorkload(f"fwd_bf16_b1_h96_n{n_s}_d64", 1, 96, 96, n_s, n_s, 64, "bf16", False, 1020 + n_s)
            GS = [t.to(dev) for t in wl.make_fwd_inputs(ws_)]
            os_ = torch.empty_like(GS[0])
            ls_ = torch.empty(GS[0].shape[:3], dtype=torch.float32, device=dev)
            scal[nm] = ws_
            calls[nm] = (lambda GS=GS, os_=os_, ls_=ls_:
                         sdpa.attn_fwd(*GS, causal=False, out=os_, lse=ls_, stream=stream))
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for n in names + solo:
            calls[n]()
    torch.cuda.synchronize()

    ev = {n: [] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for n in names:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            calls[n]()
            b.record(stream)
            ev[n].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for n in solo:  # each timed on its own, outside the step
        ev[n] = []
        for _ in range(args.steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            calls[n]()
            b.record(stream)
            ev[n].append((a, b))
        torch.cuda.synchronize()
    times = {n: [a.elapsed_time(b) for a, b in ev[n]] for n in ev}
    ms = {n: statistics.median(t) for n, t in times.items()}
    spread = {n: {"ms_min": min(t), "ms_max": max(t), "ms_mean": sum(t) / len(t), "calls": len(t)}
              for n, t in times.items()}

    # ---- host-side cost per call: CPU clock around the call, no device sync ----
    host_us = {}
    if not args.no_host_timing:
        raw = {}
        if "fwd_n4096" in calls:
            a2 = sdpa.make_fwd_args(*G2, o2, l2, False, None)
            raw["fwd_n4096"] = lambda: sdpa.lib().attn_fwd(sdpa.ctypes.byref(a2), stream.cuda_stream)
        if "decode" in calls:
            ad = sdpa.make_decode_args(*GD, od, ld, None)
            raw["decode"] = lambda: sdpa.lib().attn_decode(sdpa.ctypes.byref(ad), ws.data_ptr(), ws.numel(),
                                                           stream.cuda_stream)
        for n, fn in raw.items():
            assert fn() == 0
            host_us[n] = {"python_binding": host_cost_us(calls[n]), "c_abi": host_cost_us(fn)}

    # ---- accounting ----
    C2, C4, C5 = wl.C2, wl.C4, wl.C5
    f2 = wl.algorithmic_flops_fwd(C2.B, C2.Hq, C2.Lq, C2.Lk, C2.d, C2.causal)
    f4 = wl.algorithmic_flops_fwd(C4.B, C4.Hq, C4.Lq, C4.Lk, C4.d, C4.causal)
    res = {}
    if "fwd_n4096" in ms:
        t = ms["fwd_n4096"] / 1e3
        res["fwd_n4096"] = {"kernel": sdpa.kernel_name(*G2, causal=False), "ms": ms["fwd_n4096"],
                            "tflops": f2 / t / 1e12, "algorithmic_flops": f2}
    if "fwd_causal_n8192" in ms:
        t = ms["fwd_causal_n8192"] / 1e3
        res["fwd_causal_n8192"] = {"kernel": sdpa.kernel_name(*G4, causal=True),
                                   "ms": ms["fwd_causal_n8192"], "tflops": f4 / t / 1e12,
                                   "algorithmic_flops": f4}
    if "decode" in ms:
        t = ms["decode"] / 1e3
        bd = wl.algorithmic_bytes_decode(lens.tolist(), C5.Hq, C5.Hkv, C5.d, 2, C5.Lmax)
        res["decode"] = {"kernel": "attn_decode_split_kernel<128> + attn_decode_merge_kernel<128>",
                         "ms": ms["decode"], "gbps": bd / t / 1e9, "algorithmic_bytes": bd,
                         "total_cache_keys": int(lens.sum())}

    if "fwd_c3_d80" in ms:
        C3 = wl.C3
        f3 = wl.algorithmic_flops_fwd(C3.B, C3.Hq, C3.Lq, C3.Lk, C3.d, C3.causal)
        t = ms["fwd_c3_d80"] / 1e3
        res["fwd_c3_d80"] = {"kernel": sdpa.kernel_name(*G3, causal=True), "ms": ms["fwd_c3_d80"],
                             "tflops": f3 / t / 1e12, "algorithmic_flops": f3,
                             "algorithmic_bytes": wl.algorithmic_bytes_fwd(C3.B, C3.Hq, C3.Hkv, C3.Lq, C3.Lk, C3.d, 2),
                             "workload": C3.name}

    if "fwd_varlen" in ms:
        C6 = wl.C6
        t = ms["fwd_varlen"] / 1e3
        fv = wl.algorithmic_flops_varlen(lens_v, lens_v, C6.Hq, C6.d, C6.causal)
        res["fwd_varlen"] = {"kernel": "attn_fwd_bf16_d128_causal (packed sequences)", "ms": ms["fwd_varlen"],
                             "tflops": fv / t / 1e12, "algorithmic_flops": fv,
                             "total_tokens": int(sum(lens_v)), "sequences": C6.B}

    if "bwd" in ms:
        t = ms["bwd"] / 1e3
        fb = wl.algorithmic_flops_bwd(C4.B, C4.Hq, C4.Lq, C4.Lk, C4.d, C4.causal)
        res["bwd"] = {"kernel": "attn_bwd_delta_kernel<128> + attn_bwd_dkdv_kernel<128, true> + "
                                "attn_bwd_dq_kernel<128, true>", "ms": ms["bwd"], "tflops": fb / t / 1e12,
                      "algorithmic_flops": fb,
                      "algorithmic_bytes": wl.algorithmic_bytes_bwd(C4.B, C4.Hq, C4.Hkv, C4.Lq, C4.Lk, C4.d, 2)}

    if "bwd_d64" in ms:
        t = ms["bwd_d64"] / 1e3
        w6 = C4D64
        fb = wl.algorithmic_flops_bwd(w6.B, w6.Hq, w6.Lq, w6.Lk, w6.d, w6.causal)
        res["bwd_d64"] = {"kernel": "attn_bwd_delta_kernel<64>, then attn_bwd_dq_kernel<64, true> on a second "
                                    "stream beside attn_bwd_dkdv_kernel<64, true>", "ms": ms["bwd_d64"],
                          "tflops": fb / t / 1e12, "algorithmic_flops": fb,
                          "algorithmic_bytes": wl.algorithmic_bytes_bwd(w6.B, w6.Hq, w6.Hkv, w6.Lq, w6.Lk, w6.d, 2)}

    if "fwd_masked" in ms:
        t = ms["fwd_masked"] / 1e3
        res["fwd_masked"] = {"kernel": "attn_fwd_bf16_kernel<64, false, 1> (boolean mask, shared by all heads)",
                             "ms": ms["fwd_masked"], "tflops": f2 / t / 1e12, "algorithmic_flops": f2,
                             "algorithmic_bytes": wl.algorithmic_bytes_fwd(C2.B, C2.Hq, C2.Hkv, C2.Lq, C2.Lk, C2.d, 2)
                             + C2.Lq * C2.Lk}

    for n, (w, _) in fp8_in.items():
        if n in ms:
            t = ms[n] / 1e3
            ff = wl.algorithmic_flops_fwd(w.B, w.Hq, w.Lq, w.Lk, w.d, w.causal)
            res[n] = {"kernel": f"attn_fwd_fp8_kernel<{w.d}, {'true' if w.causal else 'false'}>", "ms": ms[n],
                      "tflops": ff / t / 1e12, "algorithmic_flops": ff,
                      "algorithmic_bytes": wl.algorithmic_bytes_fwd(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.d, 1)
                      + w.B * w.Hq * w.Lq * w.d,  # O is bf16: one more byte per element
                      "workload": w.name}

    if scal and all(n in ms for n in scal):
        ns_ = sorted(scal, key=lambda n: scal[n].Lq)
        ts = [ms[n] for n in ns_]
        res["fwd_scaling"] = {
            "workload": "fwd_bf16_b1_h96_d64 (non-causal), each n timed on its own",
            "n": [scal[n].Lq for n in ns_], "ms": ts,
            "tflops": [wl.algorithmic_flops_fwd(1, 96, scal[n].Lq, scal[n].Lk, 64, False) / (ms[n] / 1e3) / 1e12
                       for n in ns_],
            "time_ratio_per_doubling": [ts[i + 1] / ts[i] for i in range(len(ts) - 1)]}

    for n, r in res.items():
        if n in spread:
            r.update(spread[n])
        if n in host_us:
            r["host_us_per_call"] = host_us[n]

    def roof_fwd(r, tag, peak=PEAK_BF16_TFLOPS):
        tr = counted_traffic(tag)
        return {"bound": "mfma", "achieved": r["tflops"], "peak": peak, "unit": "TFLOP/s",
                "frac": r["tflops"] / peak, "traffic": tr}

    headline = res.get("fwd_n4096")
    out = {
        "metric": "attention fwd TFLOPS (causal-adj) at n=4096-8192; decode HBM GB/s",
        "value": headline["tflops"] if headline else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1), bf16 round-to-nearest-even)",
        "config": {"workload": "fwd_bf16_b1_h96_n4096_d64 (non-causal)",
                   "step": names, "B": 1, "H": 96, "n": 4096, "d": 64},
        "roofline": roof_fwd(headline, "attn_fwd_bf16_d64_n4096") if headline else None,
        "extra": {},
    }
    if "fwd_causal_n8192" in res:
        r = res["fwd_causal_n8192"]
        out["extra"]["fwd_causal_gqa_n8192_d128"] = dict(r, roofline=roof_fwd(r, "attn_fwd_bf16_d128_causal_n8192"))
    if "decode" in res:
        r = res["decode"]
        out["extra"]["decode_b64_gqa_d128"] = dict(r, roofline={
            "bound": "hbm", "achieved": r["gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": r["gbps"] / PEAK_HBM_GBPS, "traffic": counted_traffic("attn_decode_d128_b64")})
    if "fwd_c3_d80" in res:
        r = res["fwd_c3_d80"]
        out["extra"]["fwd_causal_b4_h16_n2048_d80"] = dict(r, roofline=roof_fwd(r, "attn_fwd_bf16_d80_causal_n2048"))
    if "fwd_varlen" in res:
        r = res["fwd_varlen"]
        out["extra"]["fwd_varlen_causal_gqa_b16_d128"] = dict(r, roofline=roof_fwd(r, "attn_fwd_varlen_d128_causal_b16"))
    if "fwd_masked" in res:
        r = res["fwd_masked"]
        out["extra"]["fwd_masked_bool_shared_n4096_d64"] = dict(r, roofline=roof_fwd(r, "attn_fwd_masked_d64_n4096"))
    if "bwd" in res:
        r = res["bwd"]
        out["extra"]["bwd_causal_gqa_n8192_d128"] = dict(r, roofline=roof_fwd(r, "attn_bwd_d128_causal_n8192"))
    if "bwd_d64" in res:
        r = res["bwd_d64"]
        out["extra"]["bwd_causal_gqa_n8192_d64"] = dict(r, roofline=roof_fwd(r, "attn_bwd_d64_causal_n8192"))
    if "fwd_fp8_n4096" in res:
        r = res["fwd_fp8_n4096"]
        out["extra"]["fwd_fp8_n4096_d64"] = dict(r, roofline=roof_fwd(r, "attn_fwd_fp8_d64_n4096", PEAK_FP8_TFLOPS))
    if "fwd_fp8_causal_n8192" in res:
        r = res["fwd_fp8_causal_n8192"]
        out["extra"]["fwd_fp8_causal_gqa_n8192_d128"] = dict(
            r, roofline=roof_fwd(r, "attn_fwd_fp8_d128_causal_n8192", PEAK_FP8_TFLOPS))
    if "fwd_scaling" in res:
        out["extra"]["fwd_scaling_n2048_4096_8192_d64"] = res["fwd_scaling"]
    if headline:
        out["extra"]["fwd_n4096_d64"] = headline
    if not args.no_cpu_baseline and args.only in ("all", "fwd_n4096"):
        gpu_ms = {wl.C2.name: ms.get("fwd_n4096"), wl.C3.name: ms.get("fwd_c3_d80"),
                  wl.C4.name: ms.get("fwd_causal_n8192"), wl.C5.name: ms.get("decode")}
        out["cpu_baseline"] = cpu_baseline(q2, k2, v2, args.cpu_sample_heads, gpu_ms)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
