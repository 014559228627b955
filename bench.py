#!/usr/bin/env python3
"""Benchmark: attention forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

One step is one fa_fwd call (the whole forward hot path: schedule, Q load,
K/V streaming, QK^T, masking, online softmax, PV, epilogue) over the
workload's batch, with inputs already resident in HBM. Prints one JSON line
with the throughput in TFLOP/s (4*B*H*N_q*N_kv*d, halved when causal), the
roofline fraction against the dense-bf16 MFMA peak, and the CPU oracle timed
on a bounded sample of the same workload on this host's cores.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (DECODE_WORKLOADS, VARLEN_WORKLOADS, WORKLOADS, cu_seqlens,  # noqa: E402
                       make_inputs, make_packed_inputs)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA: twice the bf16 rate
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_fa_fwd.json")
_NO_CLOCK_SAMPLE = False  # set by --no-clock-sample


def kernel_source_hash() -> str:
    """Hash of the sources the forward kernel is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_109_amd", "csrc")
    for f in ("fa_device.hpp", "fa_fwd_bf16.hip"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel source; otherwise None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if rec.get("kernel_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def device_clock_khz(torch):
    """Peak engine clock of device 0 in kHz, from the HIP runtime that torch
    loaded (hipDeviceGetAttribute with hipDeviceAttributeClockRate = 5)."""
    try:
        lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        value = ctypes.c_int(0)
        if lib.hipDeviceGetAttribute(ctypes.byref(value), 5, 0) == 0 and value.value > 0:
            return value.value
    except OSError:
        pass
    return None


def sample_clock_power():
    """One read-only amd-smi query of GPU 0 under load: socket power (W) and
    the gfx clock of each XCD (MHz). None when amd-smi is unavailable."""
    import subprocess
    # Under a profiler (rocprofv3 preloads its library into every child
    # process, which initialises the GPU there before amd-smi's launcher
    # replaces itself with python3) the query is skipped.
    if _NO_CLOCK_SAMPLE or any(key.startswith("ROCPROF") for key in os.environ) \
            or "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", "0", "--json"],
                           capture_output=True, text=True, timeout=20)
        js = json.loads(r.stdout)
    except Exception:
        return None
    g = js[0] if isinstance(js, list) and js else js
    if isinstance(g, dict) and "gpu_data" in g and g["gpu_data"]:
        g = g["gpu_data"][0]
    if not isinstance(g, dict):
        return None
    power = g.get("power", {}).get("socket_power", {})
    clocks = []
    for key, val in g.get("clock", {}).items():
        if key.startswith("gfx_") and isinstance(val, dict) and isinstance(val.get("clk"), dict):
            try:
                clocks.append(float(val["clk"]["value"]))
            except (TypeError, ValueError, KeyError):
                pass
    if not clocks:
        return None
    return {"socket_power_w": power.get("value") if isinstance(power, dict) else None,
            "gfx_clock_mhz_mean": round(float(np.mean(clocks)), 1),
            "gfx_clock_mhz_min": min(clocks), "gfx_clock_mhz_max": max(clocks)}


def _oracle_heads(w, inp, budget_s: float, backward: bool = False):
    """Run the oracle on whole heads of workload w (in order) until budget_s
    has passed or every head is done. Returns (heads, seconds, metric FLOP of
    those heads): the forward FLOP, or for the backward the 2.5x convention."""
    import oracle
    G = w.H_q // w.H_kv
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    do = inp.f64("do") if backward else None
    heads = 0
    t0 = time.perf_counter()
    done = False
    for b in range(w.B):
        for h in range(w.H_q):
            if backward:
                oracle.head_backward(q[b, h], k[b, h // G], v[b, h // G], do[b, h], w.causal, w.scale)
            else:
                oracle.head_forward(q[b, h], k[b, h // G], v[b, h // G], w.causal, w.scale)
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                done = True
                break
        if done:
            break
    el = time.perf_counter() - t0
    per_head = (w.bwd_flop if backward else w.fwd_flop) / (w.B * w.H_q)
    return heads, el, per_head * heads


def _baseline_entry(w, heads, el, flop, what):
    return {"seconds": round(el, 3), "tflops": flop / el / 1e12, "heads": heads, "of_heads": w.B * w.H_q,
            "sample": f"{what}: {heads} of {w.B * w.H_q} heads of {w.name} (all {w.N_q} rows each)"}


def cpu_baseline(w, inp, budget_s: float = 12.0):
    """The fp64 oracle timed on this host: the bench workload on whole heads
    for about budget_s (the line's value), then every configuration -- c1 and
    c2 in full, c4 and the c5 backward on whole heads for a few seconds each --
    with the host's BLAS threads, and c1 and c2 in full on one core."""
    blas = None
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)" for i in info]
    except Exception:
        threads = os.cpu_count() or 1
    heads, el, flop = _oracle_heads(w, inp, budget_s)
    out = {
        "value": flop / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H_q} heads (all {w.N_q} rows each) of {w.name}, fp64 numpy, "
                  f"{el:.1f} s",
        "host_cpus": len(os.sched_getaffinity(0)),
        "os_cpu_count": os.cpu_count(),
        "blas": blas,
    }
    per = {}
    for name, budget, backward in (("c1", 1e9, False), ("c2", 1e9, False), ("c4", budget_s * 0.6, False),
                                   ("c5", budget_s * 0.4, True)):
        if name not in WORKLOADS or name == w.name:
            continue
        wc = WORKLOADS[name]
        ic = make_inputs(wc)
        h, e, f = _oracle_heads(wc, ic, budget, backward)
        per[name] = _baseline_entry(wc, h, e, f, "backward (2.5x FLOP convention)" if backward else "forward")
        del ic
    out["per_config"] = per
    try:
        from threadpoolctl import threadpool_limits
        single = {}
        with threadpool_limits(limits=1):
            for name in ("c1", "c2"):
                wc = WORKLOADS[name]
                ic = make_inputs(wc)
                h, e, f = _oracle_heads(wc, ic, 1e9)
                single[name] = _baseline_entry(wc, h, e, f, "forward, one core")
        out["single_core"] = single
    except ImportError:
        out["single_core"] = None
    return out


def time_other_forward(fa, torch, steps: int, main_name: str):
    """The forward on the other bf16 configurations (inputs resident, outputs
    preallocated): per-launch HIP-event times on the launch stream, median and
    minimum, with the roofline fraction against the dense-bf16 MFMA peak."""
    out = {}
    for name in ("c2", "c4", "c4x"):
        if name == main_name or name not in WORKLOADS:
            continue
        w = WORKLOADS[name]
        inp = make_inputs(w)
        q, k, v = (inp.torch(n, "cuda") for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H_q, w.N_q), dtype=torch.float32, device="cuda")
        import threading
        load = {}

        def _sampler():
            time.sleep(1.2)
            load["v"] = sample_clock_power()
            time.sleep(0.6)  # launches continue a while after the query before timing

        th = threading.Thread(target=_sampler, daemon=True)
        th.start()
        t0 = time.perf_counter()
        n = 0
        while n < 5 or time.perf_counter() - t0 < 1.3 or th.is_alive():
            fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
            n += 1
            if n % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
            b.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        med = float(np.median(ms))
        tf = w.fwd_flop / (med * 1e-3) / 1e12
        out[name] = {"workload": w.name, "median_launch_ms": round(med, 4),
                     "min_launch_ms": round(float(np.min(ms)), 4), "tflops": round(tf, 2),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        if load.get("v") is not None:
            cus = torch.cuda.get_device_properties(0).multi_processor_count
            out[name]["under_load"] = dict(load["v"], mfma_frac_at_sustained_clock=round(
                tf / (4096 * cus * load["v"]["gfx_clock_mhz_mean"] * 1e6 / 1e12), 4))
        del q, k, v, o, lse, inp
    return out


def time_backward(fa, torch, steps: int, warmup: int):
    """fa_bwd (pre + dK/dV + dQ kernels) on the c5 workload, inputs and the
    forward's O/LSE resident in HBM."""
    w = WORKLOADS["c5"]
    inp = make_inputs(w)
    q, k, v, do = (inp.torch(n, "cuda") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    ws = torch.empty((fa.fa_bwd_workspace_size(w.B, w.H_q, w.N_q),), dtype=torch.uint8, device="cuda")
    import threading
    load = {}

    def _sampler():
        time.sleep(1.2)
        load["v"] = sample_clock_power()
        time.sleep(0.6)  # launches continue a while after the query before timing

    th = threading.Thread(target=_sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < 1.3 or th.is_alive():
        fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, workspace=ws)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, workspace=ws)
        b.record(stream)
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.median(per_call))
    return {"workload": w.name, "ms_per_call": round(ms, 4), "mean_ms": round(float(np.mean(per_call)), 4),
            "min_ms": round(float(np.min(per_call)), 4),
            "tflops_2p5x_convention": round(w.bwd_flop / (ms * 1e-3) / 1e12, 2),
            "frac_of_peak": round(w.bwd_flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "note": "FLOP = 2.5 x forward FLOP; the kernels issue 3.5 x (S, dP recomputed in both passes)",
            "under_load": None if load.get("v") is None else dict(
                load["v"],
                # MFMA work actually issued (3.5 x forward) over the sustained clock's peak
                mfma_frac_at_sustained_clock=round(
                    1.4 * w.bwd_flop / (ms * 1e-3) / (4096 * torch.cuda.get_device_properties(0).multi_processor_count
                                                      * load["v"]["gfx_clock_mhz_mean"] * 1e6), 4))}


def time_decode(fa, torch, steps: int):
    """Split-KV forward on the decode workload: HBM-bound, reported as the
    algorithmic bytes (Q, K, V read once; O, LSE written once) per second
    against the 8 TB/s HBM peak."""
    w = DECODE_WORKLOADS["d1"]
    inp = make_inputs(w)
    q, k, v = (inp.torch(n, "cuda") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H_q, w.N_q), dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = fa.default_num_splits(w.B, w.H_kv, w.N_kv, cus)
    ws = torch.empty((max(256, fa.fa_fwd_splitkv_workspace_size(w.B, w.H_q, w.N_q, w.d, splits)),),
                     dtype=torch.uint8, device="cuda")
    nbytes = (q.numel() + k.numel() + v.numel() + o.numel()) * 2 + lse.numel() * 4
    t0 = time.perf_counter()
    n = 0
    while n < 5 or time.perf_counter() - t0 < 0.5:
        fa.fwd_splitkv(q, k, v, splits, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)
        n += 1
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in per:
        a.record(stream)
        fa.fwd_splitkv(q, k, v, splits, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in per]
    med = float(np.median(ms))
    gbs = nbytes / (med * 1e-3) / 1e9
    # context: a plain device-to-device copy of 512 MiB (read + write bytes)
    src = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    # the same decode step against an FP8 copy of the cache (quantized on the GPU)
    k8, kd = fa.quantize_fp8(k)
    v8, vd = fa.quantize_fp8(v)
    o8 = torch.empty_like(q)
    lse8 = torch.empty_like(lse)
    for _ in range(20):
        fa.fwd_splitkv_fp8(q, k8, kd, v8, vd, splits, causal=w.causal, scale=w.scale, out=o8, lse=lse8, workspace=ws)
    torch.cuda.synchronize()
    per8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a8, b8 in per8:
        a8.record(stream)
        fa.fwd_splitkv_fp8(q, k8, kd, v8, vd, splits, causal=w.causal, scale=w.scale, out=o8, lse=lse8, workspace=ws)
        b8.record(stream)
    torch.cuda.synchronize()
    ms8 = [a8.elapsed_time(b8) for a8, b8 in per8]
    med8 = float(np.median(ms8))
    nbytes8 = (q.numel() + o.numel()) * 2 + k8.numel() + v8.numel() + 4 * (kd.numel() + vd.numel()) + lse.numel() * 4
    gbs8 = nbytes8 / (med8 * 1e-3) / 1e9
    d8 = o8.float() - o.float()
    fp8_kv = {
        "entry_point": "fa_fwd_splitkv_fp8",
        "dtype": "bf16 queries, e4m3 K and V (128-key block scales)",
        "median_ms": round(med8, 4),
        "min_ms": round(float(np.min(ms8)), 4),
        "algorithmic_bytes": nbytes8,
        "roofline": {"bound": "hbm", "achieved": round(gbs8, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs8 / 8000.0, 4)},
        "speedup_vs_bf16_cache": round(med / med8, 3),
        "vs_bf16_cache": {"o_rel_rms": round(float(d8.square().mean().sqrt() / o.float().square().mean().sqrt()), 5),
                          "lse_max_abs": round(float((lse8 - lse).abs().max()), 5)},
    }
    return {
        "workload": w.name,
        "entry_point": "fa_fwd_splitkv",
        "num_splits": splits,
        "median_ms": round(med, 4),
        "min_ms": round(float(np.min(ms)), 4),
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4)},
        "tflops": round(w.fwd_flop / (med * 1e-3) / 1e12, 2),
        "device_copy_gbs": round(copy_gbs, 1),
        "fp8_kv_cache": fp8_kv,
    }


def time_varlen(fa, torch, steps: int):
    """Packed variable-length forward: TFLOP/s over the sum of the per-sequence
    FLOP counts (4*H_q*n^2*d, halved when causal)."""
    w = VARLEN_WORKLOADS["v1"]
    lengths = w.lengths()
    total = int(lengths.sum())
    inp = make_packed_inputs(1, w.H_q, w.H_kv, total, total, w.d, w.seed)
    q, k, v = (inp.torch(n, "cuda") for n in ("q", "k", "v"))
    cu = torch.from_numpy(cu_seqlens(lengths)).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.H_q, total), dtype=torch.float32, device="cuda")
    mx = int(lengths.max())
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < 0.5:
        fa.fwd_varlen(q, k, v, cu, cu, mx, causal=w.causal, scale=w.scale, out=o, lse=lse)
        n += 1
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in per:
        a.record(stream)
        fa.fwd_varlen(q, k, v, cu, cu, mx, causal=w.causal, scale=w.scale, out=o, lse=lse)
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in per]
    med = float(np.median(ms))
    tf = w.fwd_flop() / (med * 1e-3) / 1e12
    return {
        "workload": w.name,
        "entry_point": "fa_fwd_varlen",
        "lengths": [int(x) for x in lengths],
        "median_ms": round(med, 4),
        "min_ms": round(float(np.min(ms)), 4),
        "tflops": round(tf, 2),
        "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
    }


def time_fp8(fa, torch, steps: int):
    """FP8 forward on the bench configuration: the bf16 inputs are block-
    quantized on the GPU (fa_quantize_fp8, row-major), then
    fa_fwd_fp8 is timed. Throughput against the dense-fp8 MFMA peak; the
    output's deviation from the bf16 forward on the unquantized inputs is
    reported beside it (relative RMS and max |dO| over all elements, max
    |dLSE|)."""
    w = WORKLOADS["c3"]
    inp = make_inputs(w)
    q, k, v = (inp.torch(n, "cuda") for n in ("q", "k", "v"))
    stream = torch.cuda.current_stream()
    # quantizer: one pass over each of the three tensors (bf16 in, codes +
    # scales out) into preallocated outputs, each launch timed on its own
    q8, qd = fa.quantize_fp8(q)
    k8, kd = fa.quantize_fp8(k)
    v8, vd = fa.quantize_fp8(v)
    torch.cuda.synchronize()
    quant_ms = 0.0
    for src, c8, cd in ((q, q8, qd), (k, k8, kd), (v, v8, vd)):
        qa = torch.cuda.Event(enable_timing=True)
        qb = torch.cuda.Event(enable_timing=True)
        qa.record(stream)
        fa.quantize_fp8(src, codes=c8, descale=cd)
        qb.record(stream)
        torch.cuda.synchronize()
        quant_ms += qa.elapsed_time(qb)
    qbytes = 3 * (q.numel() * 3) + 4 * (qd.numel() + kd.numel() + vd.numel())
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H_q, w.N_q), dtype=torch.float32, device="cuda")
    t0 = time.perf_counter()
    n = 0
    while n < 5 or time.perf_counter() - t0 < 1.0:
        fa.fwd_fp8(q8, qd, k8, kd, v8, vd, causal=w.causal, scale=w.scale, out=o, lse=lse)
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in per:
        a.record(stream)
        fa.fwd_fp8(q8, qd, k8, kd, v8, vd, causal=w.causal, scale=w.scale, out=o, lse=lse)
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in per]
    avg = float(np.mean(ms))
    tf = w.fwd_flop / (avg * 1e-3) / 1e12
    o_ref, lse_ref = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    diff = o.float() - o_ref.float()
    rel_rms = float(diff.square().mean().sqrt() / o_ref.float().square().mean().sqrt())
    return {
        "workload": w.name + "_fp8",
        "entry_point": "fa_fwd_fp8",
        "dtype": "e4m3 inputs (128-row block scales), f32 scores, e4m3 P, bf16 O",
        "avg_launch_ms": round(avg, 4),
        "median_launch_ms": round(float(np.median(ms)), 4),
        "min_launch_ms": round(float(np.min(ms)), 4),
        "tflops": round(tf, 2),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4), "kernel": "fwd_fp8_kernel"},
        "vs_bf16_path": {"o_rel_rms": round(rel_rms, 6), "o_max_abs": round(float(diff.abs().max()), 5),
                         "lse_max_abs": round(float((lse - lse_ref).abs().max()), 5)},
        "quantize": {"ms_three_tensors": round(quant_ms, 4), "bytes": qbytes,
                     "gbs": round(qbytes / (quant_ms * 1e-3) / 1e9, 1)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--warmup-seconds", type=float, default=1.5,
                    help="keep warming up (untimed) until this much wall time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward measurement on c5")
    ap.add_argument("--no-decode", action="store_true", help="skip the split-KV decode measurement")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed variable-length measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward measurement")
    ap.add_argument("--no-clock-sample", action="store_true",
                    help="do not query amd-smi for the clock and power under load")
    ap.add_argument("--no-other-fwd", action="store_true",
                    help="skip the forward on the other bf16 configurations (c2, c4, c4x)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times (HBM "
                         "counter calibration for the traffic figure) and exit")
    args = ap.parse_args()
    global _NO_CLOCK_SAMPLE
    _NO_CLOCK_SAMPLE = args.no_clock_sample

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the attention path runs on "
              "one GPU (across GPUs it would shard over (batch, key/value head) pairs with no communication, "
              "each GPU running the same kernels on its share).", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_109_amd as fa

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.load_library()

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}))
        return

    w = WORKLOADS[args.workload]
    print(f"# workload {w}", file=sys.stderr, flush=True)
    inp = make_inputs(w)
    q, k, v = (inp.torch(n, "cuda") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H_q, w.N_q), dtype=torch.float32, device="cuda")

    # W untimed warm-up steps, continued until the GPU has been busy for at
    # least --warmup-seconds: clocks ramp up under load, and a few
    # millisecond-long launches would otherwise be timed at idle clocks.
    # The GPU holds its socket power at the board limit under this load and
    # lowers the gfx clock to stay there; one amd-smi sample taken during the
    # warm-up records the clock the timed launches run at.
    import threading
    load_sample = {}

    def _sampler():
        # after 1.2 s of back-to-back launches (the power reading is averaged)
        time.sleep(1.2)
        load_sample["v"] = sample_clock_power()
        time.sleep(0.6)  # launches continue a while after the query before timing

    sampler = threading.Thread(target=_sampler, daemon=True)
    t_warm = time.perf_counter()
    n_warm = 0
    while (n_warm < args.warmup or time.perf_counter() - t_warm < args.warmup_seconds
           or sampler.is_alive() or n_warm <= 16):
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        n_warm += 1
        if n_warm % 16 == 0:
            torch.cuda.synchronize()
            if n_warm == 16:
                sampler.start()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_warm

    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        per[i][0].record(stream)
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        per[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    launch_ms = [a.elapsed_time(b) for a, b in per]
    ms_per_step = total_ms / args.steps
    avg_launch_ms = float(np.mean(launch_ms))
    tflops = w.fwd_flop / (ms_per_step * 1e-3) / 1e12
    achieved = w.fwd_flop / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == 1 else PEAK_F32_TFLOPS

    props = torch.cuda.get_device_properties(0)
    clock_khz = device_clock_khz(torch)
    result = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d, causal halved) and fraction of MI355X dense-bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == 1 else "f32",
        "data": "synthetic: i.i.d. N(0,1) from PCG64(seed), rounded to bf16",
        "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "N_q": w.N_q, "N_kv": w.N_kv,
                   "d": w.d, "causal": w.causal, "scale": w.scale, "seed": w.seed},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(w.name),
            "kernel": "fwd_bf16_kernel" if w.dtype == 1 else "fwd_f32_kernel",
            "avg_launch_ms": round(avg_launch_ms, 4),
            "median_launch_ms": round(float(np.median(launch_ms)), 4),
            "min_launch_ms": round(float(np.min(launch_ms)), 4),
            "flop_per_launch": w.fwd_flop,
        },
        "under_load": None if load_sample.get("v") is None else dict(
            load_sample["v"],
            # MFMA busy fraction at the clock actually sustained: achieved over
            # 4096 FLOP/clk/CU x CUs x the mean gfx clock of the 8 XCDs
            mfma_frac_at_sustained_clock=round(achieved / (4096 * props.multi_processor_count
                                                           * load_sample["v"]["gfx_clock_mhz_mean"] * 1e6 / 1e12), 4)),
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""),
                   "peak_clock_mhz": None if clock_khz is None else clock_khz / 1000,
                   # dense bf16: 4096 FLOP per clock per CU (32x32x16 MFMA, 4 SIMDs)
                   "bf16_peak_tflops_from_device": None if clock_khz is None else
                   round(4096 * props.multi_processor_count * clock_khz * 1e3 / 1e12, 1)},
        "wall_s_timed_region": round(wall, 3),
    }
    if not args.no_other_fwd:
        print("# timing the forward on the other bf16 configurations", file=sys.stderr, flush=True)
        result["fwd_other_configs"] = time_other_forward(fa, torch, max(10, args.steps), w.name.split("_")[0])
    if not args.no_bwd:
        print("# timing the backward on c5", file=sys.stderr, flush=True)
        result["bwd"] = time_backward(fa, torch, max(30, args.steps), 2)
    if not args.no_varlen:
        print("# timing the packed variable-length forward", file=sys.stderr, flush=True)
        result["varlen"] = time_varlen(fa, torch, max(5, args.steps // 2))
    if not args.no_fp8:
        print("# timing the FP8 forward", file=sys.stderr, flush=True)
        result["fp8"] = time_fp8(fa, torch, max(5, args.steps))
    if not args.no_decode:
        print("# timing the split-KV forward on the decode workload", file=sys.stderr, flush=True)
        result["decode"] = time_decode(fa, torch, max(5, args.steps))
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
