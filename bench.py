#!/usr/bin/env python3
"""Benchmark of Parallax attention on one MI355X.

One JSON line on stdout.  The headline (`value`) is decode KV HBM throughput
on the decode workload (B=64, Hq=16, Hkv=8, d=128, 4096 cached keys per
sequence, bf16): one step is one call of parallax_fwd_decode over the whole
batch (split-KV kernel + merge kernel).  The second half of the metric, the
causal prefill (B=8, T=4096, Hq=16, Hkv=8, d=128, bf16), is timed the same way
and reported under "prefill" with its MFMA roofline; the prefill backward
(parallax_bwd_prefill on the same tensors) under "prefill"/"backward", and the
fused q/k/v/probe projection of the same layer under "prefill"/"projection"
(with torch's library GEMM time for the same product as context).  As context
only (skipped with --no-context), "prefill"/"longer_sequence" times the same heads and token count at a
4x longer sequence (B=2, T=16384), and "decode_other_workloads" the two decode
extremes (2048 x 128 keys, 256 x 32768 keys) and the ragged batch (2048
sequences of 128..32768 keys, Hq=32, Hkv=16, d=64).  "prefill_f32" times the
fp32 causal prefill (B=1, Hq=Hkv=2, T=256, d=64) and checks every row against
the oracle.  "sweep" (skipped with --no-sweep) is the decode sweep of Parallax
against the library's softmax-only path over batch 1..2048 x context
128..32768, I/O-matched (same d) and compute-matched (Parallax at d=64).

Inputs are seeded synthetic tensors resident in HBM before timing starts.
Several input sets are rotated so that no step finds its K/V in the 256 MB
Infinity Cache.  Kernel time is measured with HIP events recorded on the
stream the kernels run on (torch's current stream, which the binding passes
to the C ABI).  The CPU baseline is the fp64 oracle, as it stands, on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published

DECODE_WL = "decode_bf16_b64_hq16_hkv8_l4096_d128"
PREFILL_WL = "prefill_bf16_b8_hq16_hkv8_t4096_d128"

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_kernel_b64_l4096_traffic.md")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_kernel_b8_t4096_traffic.md")
DECODE_SOURCES = ["transformer_attention_flash_amd/csrc/plx_decode.hip",
                  "transformer_attention_flash_amd/csrc/plx_device.h"]
PREFILL_SOURCES = ["transformer_attention_flash_amd/csrc/plx_prefill.hip",
                   "transformer_attention_flash_amd/csrc/plx_device.h"]
BACKWARD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "backward_b8_t4096_traffic.md")
BACKWARD_SOURCES = ["transformer_attention_flash_amd/csrc/plx_backward.hip",
                    "transformer_attention_flash_amd/csrc/plx_device.h"]
PROJECTION_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "projection_t32768_dm2048_traffic.md")
PROJECTION_SOURCES = ["transformer_attention_flash_amd/csrc/plx_projection.hip",
                      "transformer_attention_flash_amd/csrc/plx_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu() -> dict:
    """The host's CPU model and the threads this process may run on."""
    model = None
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
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def build_info() -> dict:
    """Git revision the library was built from (written by the build step)."""
    path = os.path.join(ROOT, "transformer_attention_flash_amd", "_build_info.json")
    try:
        with open(path) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {"git_sha": None}


def parity_errors(got, ref) -> dict:
    """max-abs and relative L2 of the GPU rows against the oracle's."""
    import numpy as np
    diff = got - ref
    return {"rows": int(got.reshape(-1, got.shape[-1]).shape[0]), "max_abs": float(np.abs(diff).max()),
            "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(ref))}


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(digest: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch from a committed counter summary, or None when it
    is missing or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    f = re.search(r"fetch_bytes_per_launch:\s*([0-9.eE+]+)", text)
    w = re.search(r"write_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m and f and w) or m.group(1) != digest:
        return None
    return float(f.group(1)) + float(w.group(1))


def time_steps(fn_for_step, steps, warmup, torch):
    """Run warmup steps, then time `steps` steps with HIP events on the current
    stream; returns (total seconds by events, per-step list of ms)."""
    for i in range(warmup):
        fn_for_step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        fn_for_step(warmup + i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / 1e3, per


def cpu_baseline_decode(x, w, budget_s: float, gpu_out=None):
    """Oracle (expanded form) on whole sequences of the decode workload, in
    passes over the batch, until about budget_s seconds of CPU work; returns
    the oracle's KV GB/s, and (given the GPU output on the same inputs) the
    GPU's errors against the oracle rows of the first pass."""
    import numpy as np
    import oracle  # the CPU baseline leg of the benchmark

    tau = 1.0 / math.sqrt(w.d)
    per_seq_bytes = 2 * 2 * w.Hkv * w.L * w.d
    chunks = []
    for b in range(0, w.B, 8):  # host fp64 copies, 8 sequences per oracle call
        sl = slice(b, min(b + 8, w.B))
        chunks.append(tuple(x[n][sl].float().cpu().numpy().astype(np.float64) for n in ("q", "rho", "k", "v")))
    done_bytes, spent, nseq, passes = 0, 0.0, 0, 0
    first = []
    while spent < budget_s:
        for q, r, k, v in chunks:
            t0 = time.perf_counter()
            o = oracle.decode(q, r, k, v, tau, form=oracle.EXPANDED)
            spent += time.perf_counter() - t0
            nseq += q.shape[0]
            done_bytes += q.shape[0] * per_seq_bytes
            if passes == 0:
                first.append(o)
        passes += 1
    # The explicit form (a d x d covariance per row, O(L d^2)) on its own,
    # smaller sample: whole sequences until about a quarter of the budget.
    e_bytes, e_spent, e_seq = 0, 0.0, 0
    for q, r, k, v in chunks:
        for i in range(q.shape[0]):
            if e_spent >= budget_s / 4:
                break
            t0 = time.perf_counter()
            oracle.decode(q[i:i + 1], r[i:i + 1], k[i:i + 1], v[i:i + 1], tau, form=oracle.EXPLICIT)
            e_spent += time.perf_counter() - t0
            e_seq += 1
            e_bytes += per_seq_bytes
    res = {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{passes} pass(es) over all {w.B} sequences ({w.Hq} heads, {w.L} keys each; {nseq} "
                     f"sequence evaluations), fp64 expanded form, {spent:.1f} s",
           "host": host_cpu(),
           "explicit_form": {"value": e_bytes / e_spent / 1e9, "unit": "GB/s",
                             "sample": f"{e_seq} whole sequence(s), fp64 explicit covariance form, {e_spent:.1f} s"}}
    if gpu_out is not None:
        res["gpu_parity_vs_oracle"] = parity_errors(gpu_out.float().cpu().numpy().astype(np.float64),
                                                    np.concatenate(first))
    return res


def cpu_baseline_prefill(x, w, budget_s: float, gpu_out=None):
    """Oracle on query rows of the prefill workload (whole sequences, all
    heads, positions visited in a strided order) until about budget_s seconds;
    returns the oracle's TFLOP/s under the GPU's flop count (8 d flops per
    causal pair), and (given the GPU output on the same inputs) the GPU's
    errors against every oracle row evaluated."""
    import numpy as np
    import oracle

    tau = 1.0 / math.sqrt(w.d)
    flops, spent, nrows, nseq = 0.0, 0.0, 0, 0
    got_rows, ref_rows = [], []
    step = 64
    for b in range(w.B):
        if spent >= budget_s:
            break
        q, r, k, v = (x[n][b:b + 1].float().cpu().numpy().astype(np.float64) for n in ("q", "rho", "k", "v"))
        ob = None if gpu_out is None else gpu_out[b].float().cpu().numpy().astype(np.float64)
        nseq += 1
        for off in range(step):
            if spent >= budget_s:
                break
            ts = np.arange(off, w.T, step)
            rows = np.array([(0, h, t) for h in range(w.Hq) for t in ts], dtype=np.int64)
            t0 = time.perf_counter()
            o = oracle.prefill(q, k, v, r, tau, form=oracle.EXPANDED, rows=rows)
            spent += time.perf_counter() - t0
            nrows += len(rows)
            flops += float(8 * w.d * (rows[:, 2] + 1).sum())
            if ob is not None:
                ref_rows.append(o)
                got_rows.append(ob[rows[:, 1], rows[:, 2]])
    res = {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{nrows} query rows from {nseq} sequence(s) (all {w.Hq} heads, positions over "
                     f"0..{w.T - 1}), fp64 expanded form, {spent:.1f} s",
           "host": host_cpu()}
    if got_rows:
        res["gpu_parity_vs_oracle"] = parity_errors(np.concatenate(got_rows), np.concatenate(ref_rows))
    return res


def cpu_baseline_backward(x, dout, w):
    """The backward oracle (closed form, numpy fp64 on the host's BLAS) on one
    whole KV-head group of the prefill workload; returns its TFLOP/s on the
    same 8-GEMM count as the GPU figure."""
    import numpy as np
    from oracle import grad as ograd

    G = w.Hq // w.Hkv
    b, g = 0, 0
    hs = slice(g * G, (g + 1) * G)
    h = {n: x[n][b:b + 1, hs].double().cpu().numpy() for n in ("q", "rho")}
    kk = x["k"][b:b + 1, g:g + 1].double().cpu().numpy()
    vv = x["v"][b:b + 1, g:g + 1].double().cpu().numpy()
    do = dout[b:b + 1, hs].double().cpu().numpy()
    t0 = time.perf_counter()
    ograd.grad_expanded(h["q"], kk, vv, h["rho"], do, 1.0 / np.sqrt(w.d), groups=[(0, 0)])
    dt = time.perf_counter() - t0
    flops = 8 * 2 * w.d * G * w.T * (w.T + 1) // 2
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except ImportError:
        cores = os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"one KV-head group ({G} query heads x {w.T} positions, batch 0, kv head 0), "
                      f"closed-form fp64 gradients with numpy, {dt:.1f} s"}


def measure_device(torch):
    """The device's own ceilings beside the datasheet figures: the bf16 MFMA
    peak implied by its compute units and maximum clock, and measured rates of
    a plain streaming read (cached and non-temporal 16-byte loads over 2 GiB,
    far beyond the caches) and of a kernel doing nothing but bf16 MFMAs at
    two wavefronts per SIMD."""
    from transformer_attention_flash_amd import diag

    info = diag.device_info()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def best_seconds(fn, reps, rounds=3):
        best = None
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / reps
            best = t if best is None or t < best else best
        return best

    measured = {}
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    for nt in (False, True):
        fn = lambda: diag.stream_read(buf, nontemporal=nt, sink=sink)  # noqa: E731
        for _ in range(3):
            fn()
        key = "stream_read_nontemporal_GBs" if nt else "stream_read_cached_GBs"
        measured[key] = round(nbytes / best_seconds(fn, 10) / 1e9, 1)
    del buf
    n_blocks, iters = 2 * info["compute_units"], 16000
    flops = n_blocks * 4 * 8 * iters * diag.MFMA_FLOP
    fn = lambda: diag.mfma_bf16(n_blocks, iters, sink=sink)  # noqa: E731
    for _ in range(20):  # ~40 ms: lets the clock settle under matrix load
        fn()
    measured["bf16_mfma_tflops"] = round(flops / best_seconds(fn, 10) / 1e12, 1)
    torch.cuda.synchronize()
    return {"name": torch.cuda.get_device_properties(0).gcnArchName,
            "compute_units": info["compute_units"], "max_clock_mhz": info["max_clock_mhz"],
            "bf16_mfma_peak_tflops_from_clock": round(info["bf16_mfma_peak_tflops"], 1),
            "datasheet": {"hbm_GBs": HBM_PEAK_GBS, "bf16_mfma_tflops": BF16_MFMA_PEAK_TFLOPS},
            "measured": measured}


SWEEP_BATCHES = (1, 16, 128, 1024, 2048)
SWEEP_CONTEXTS = (128, 1024, 8192, 32768)
FLUSH_BYTES = 512 << 20
SWEEP_MAX_KV_BYTES = 160 * 10 ** 9  # one input set of K/V beside the rest of the bench in 288 GB of HBM


def run_sweep(torch, plx, synth, diag, budget_s: float):
    """Decode sweep, Parallax against the softmax-only path (rho = NULL) of the
    same library, over the pages' range: batch 1..2048 x context 128..32768
    (every point), Hq = 16, Hkv = 8, bf16.  Two settings:
      I/O-matched:     Parallax and softmax-only at the same d = 128;
      compute-matched: Parallax at d = 64 against softmax-only at d = 128
                       (equal matrix flops per key: Parallax has two scoring
                       and two value products, softmax attention one each).
    No timed call finds its K/V in the caches (4 MB L2 per XCD, 256 MB
    Infinity Cache): points with at least 128 MB of K/V rotate enough input
    sets to cover 512 MB; smaller points time each call alone, after a
    cached streaming read of a 512 MB buffer that evicts them.  Points are
    visited small to large; once budget_s is spent, the remaining points are
    listed as skipped, as is a point whose d = 128 K/V exceeds 160 GB (2048 x
    32768 keys: 275 GB).  Returns {"points": [...], ...}."""
    dev = "cuda"
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    t_start = time.time()
    points, skipped = [], []

    def time_point(B, L, d, with_rho, xs_cache):
        kv = 4 * B * 8 * L * d
        key = (B, L, d)
        if key not in xs_cache:
            xs_cache.clear()
            torch.cuda.empty_cache()
            n_sets = 1 if kv >= FLUSH_BYTES else (-(-FLUSH_BYTES // kv) if kv >= (128 << 20) else 1)
            xs_cache[key] = [synth.make_decode(B, 16, 8, L, d, torch.bfloat16, dev, seed=s) for s in range(n_sets)]
        xs = xs_cache[key]
        out = torch.empty_like(xs[0]["q"])
        ws_n = plx.decode_workspace_size(B, 16, 8, d, L)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

        def call(i):
            x = xs[i % len(xs)]
            plx.decode(x["q"], x["k"], x["v"], x["rho"] if with_rho else None, out=out, workspace=ws)

        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        if kv >= (128 << 20):  # rotated sets, back-to-back calls between two events
            iters = max(4 * len(xs), min(60, int(0.05 / (kv / 5e12))))
            secs, _ = time_steps(call, iters, 0, torch)
            return secs / iters * 1e6, len(xs), "rotated input sets"
        per = []
        for i in range(15):  # one call at a time after a cache-evicting read
            diag.stream_read(flush, nontemporal=False, sink=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call(i)
            e1.record()
            per.append((e0, e1))
        torch.cuda.synchronize()
        us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in per)
        return us[len(us) // 2], 1, "cache evicted before each call (median of 15)"

    xs_cache = {}
    for L in SWEEP_CONTEXTS:
        for B in SWEEP_BATCHES:
            if time.time() - t_start > budget_s:
                skipped.append({"B": B, "context": L, "reason": "time budget spent"})
                continue
            if 4 * B * 8 * L * 128 > SWEEP_MAX_KV_BYTES:
                skipped.append({"B": B, "context": L, "reason": f"K/V of {4 * B * 8 * L * 128 / 1e9:.0f} GB at "
                                                                 f"d = 128 does not fit beside the rest in HBM"})
                continue
            row = {"B": B, "context": L}
            for name, d, with_rho in (("parallax_d128", 128, True), ("softmax_d128", 128, False),
                                      ("parallax_d64", 64, True)):
                us, n_sets, how = time_point(B, L, d, with_rho, xs_cache)
                row[name + "_us"] = round(us, 2)
                row[name + "_GBs"] = round(4 * B * 8 * L * d / us / 1e3, 1)
                row["timing_" + str(d)] = how
            row["io_matched_speedup"] = round(row["softmax_d128_us"] / row["parallax_d128_us"], 3)
            row["compute_matched_speedup"] = round(row["softmax_d128_us"] / row["parallax_d64_us"], 3)
            points.append(row)
            log(f"  sweep B={B} L={L}: parallax d128 {row['parallax_d128_us']} us, softmax {row['softmax_d128_us']} "
                f"us, parallax d64 {row['parallax_d64_us']} us")
    xs_cache.clear()
    del flush, sink
    torch.cuda.empty_cache()
    io = [p["io_matched_speedup"] for p in points]
    cm = [p["compute_matched_speedup"] for p in points]
    big = [p for p in points if 4 * p["B"] * 8 * p["context"] * 128 >= (128 << 20)]
    return {"heads": {"Hq": 16, "Hkv": 8}, "dtype": "bf16", "points": points, "skipped_for_time": skipped,
            "seconds": round(time.time() - t_start, 1),
            "io_matched_speedup_range": [min(io), max(io)] if io else None,
            "compute_matched_speedup_range": [min(cm), max(cm)] if cm else None,
            "bandwidth_bound_points": {"n": len(big),
                                       "io_matched_geomean": _geomean([p["io_matched_speedup"] for p in big]),
                                       "compute_matched_geomean": _geomean([p["compute_matched_speedup"]
                                                                            for p in big])}}


def _geomean(xs):
    return round(math.exp(sum(math.log(x) for x in xs) / len(xs)), 3) if xs else None


def prefill_f32_leg(torch, plx, synth, steps=50):
    """The fp32 causal prefill (B=1, Hq=Hkv=2, T=256, d=64): microseconds per
    call, and every output row against the oracle."""
    import oracle

    w = synth.WORKLOADS["prefill_f32_b1_h2_t256_d64"]
    x = synth.make_workload(w, "cuda")
    out = torch.empty_like(x["q"])
    secs, per = time_steps(lambda i: plx.prefill(x["q"], x["k"], x["v"], x["rho"], out=out), steps, 20, torch)
    h = {n: x[n].double().cpu().numpy() for n in ("q", "k", "v", "rho")}
    ref = oracle.prefill(h["q"], h["k"], h["v"], h["rho"], 1 / math.sqrt(w.d))
    flops = 4 * 2 * w.d * w.B * w.Hq * w.T * (w.T + 1) // 2
    return {"workload": w.name, "us_per_call": round(secs / steps * 1e6, 2),
            "us_per_call_median": round(sorted(per)[len(per) // 2] * 1e3, 2), "steps": steps,
            "tflops": round(flops / (secs / steps) / 1e12, 3), "bound": "launch latency (3.4e7 flop)",
            "gpu_parity_vs_oracle": parity_errors(out.double().cpu().numpy(), ref)}


def io_contract(torch, plx, synth, copy_mib: int):
    """Decode workload calls for the counter runs that show the probe branch
    adds no K/V traffic and no matrix instructions: a plain device copy of
    copy_mib MiB (calibration), then three calls with rho and three with
    rho = NULL on the same two input sets, in that order."""
    dev = "cuda"
    w = synth.WORKLOADS[DECODE_WL]
    n = copy_mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    sets = [synth.make_decode(w.B, w.Hq, w.Hkv, w.L, w.d, w.dtype, dev, seed=s) for s in range(2)]
    out = torch.empty_like(sets[0]["q"])
    order = []
    for with_rho in (True, False):
        for i in range(3):
            x = sets[i % 2]
            plx.decode(x["q"], x["k"], x["v"], x["rho"] if with_rho else None, out=out)
            order.append("rho" if with_rho else "rho=NULL")
    torch.cuda.synchronize()
    print(json.dumps({"io_contract": {"workload": w.name, "copy_bytes": n, "decode_calls_in_order": order,
                                      "rho_bytes_per_call": 2 * w.B * w.Hq * w.d,
                                      "kv_bytes_per_call": 2 * 2 * w.B * w.Hkv * w.L * w.d}}), flush=True)


def other_decode_workloads(plx, synth, dev, torch):
    """The two decode extremes and the ragged batch, timed like the headline
    (one call over the whole batch is one step), as context: GB/s of K/V and
    its fraction of the HBM peak.  Small caches rotate 4 input sets; the
    large ones (34 GB, 138 GB of K/V) are far beyond the Infinity Cache with
    one."""
    res = {}
    for name, n_sets, steps, warmup in (("decode_bf16_b2048_hq16_hkv8_l128_d128", 4, 50, 20),
                                        ("decode_bf16_b256_hq16_hkv8_l32768_d128", 1, 10, 3),
                                        ("decode_ragged_bf16_b2048_hq32_hkv16_d64_l128to32768", 1, 5, 2)):
        w = synth.WORKLOADS[name]
        log(f"decode workload {name}")
        if w.kind == "decode_ragged":
            xs = [synth.make_workload(w, dev)]
            kv = 2 * 2 * w.Hkv * w.d * int(xs[0]["cu_host"][-1])
            kw = dict(cu_seqlens=xs[0]["cu_seqlens"], max_ctx=xs[0]["max_ctx"], num_kv_heads=w.Hkv)
        else:
            xs = [synth.make_decode(w.B, w.Hq, w.Hkv, w.L, w.d, w.dtype, dev, seed=s) for s in range(n_sets)]
            kv = 2 * 2 * w.B * w.Hkv * w.L * w.d
            kw = {}
        out = torch.empty_like(xs[0]["q"])

        def step(i, xs=xs, kw=kw, out=out):
            x = xs[i % len(xs)]
            plx.decode(x["q"], x["k"], x["v"], x["rho"], out=out, **kw)

        secs, _ = time_steps(step, steps, warmup, torch)
        gbs = kv / (secs / steps) / 1e9
        res[name] = {"value": round(gbs, 2), "unit": "GB/s", "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "ms_per_step": round(secs / steps * 1e3, 4), "steps": steps, "kv_bytes": kv,
                     "input_sets_rotated": len(xs)}
        log(f"  {secs / steps * 1e3:.3f} ms/step, {gbs:.0f} GB/s")
        del xs, out, kw
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The clocks take a few dozen prefill calls (~50 ms of work) to settle
    # after an idle spell; the warm-up covers that.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--prefill-warmup", type=int, default=60)
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated across steps")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-projection", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context-only legs (longer-sequence prefill, other decode workloads)")
    ap.add_argument("--no-device", action="store_true", help="skip the device ceiling measurements")
    ap.add_argument("--backward-steps", type=int, default=20)
    ap.add_argument("--backward-warmup", type=int, default=20)
    ap.add_argument("--sweep", action="store_true",
                    help="run only the decode sweep (Parallax vs softmax-only over batch x context)")
    ap.add_argument("--no-sweep", action="store_true", help="leave the decode sweep out of the default run")
    ap.add_argument("--sweep-budget", type=float, default=60.0, help="seconds the decode sweep may take")
    ap.add_argument("--io-contract", action="store_true",
                    help="only the decode calls of the probe-traffic counter runs (with rho, then rho = NULL)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Parallax forward here runs on a single MI355X with no "
              "cross-GPU sharding; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_attention_flash_amd as plx
    from transformer_attention_flash_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    plx.load_library()
    dev = "cuda"

    from transformer_attention_flash_amd import diag

    if args.io_contract:
        io_contract(torch, plx, synth, args.copy_probe_mib or 1024)
        return
    if args.sweep:
        print(json.dumps({"sweep": run_sweep(torch, plx, synth, diag, args.sweep_budget)}), flush=True)
        return

    if args.copy_probe_mib:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters
        # calibrate the per-kernel HBM traffic of the same profiling run.
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read, {n} bytes written")
        del src, dst

    # ---------------- decode (headline) ----------------
    w = synth.WORKLOADS[DECODE_WL]
    log(f"decode workload {w.name}: generating {args.sets} input sets")
    sets = [synth.make_decode(w.B, w.Hq, w.Hkv, w.L, w.d, w.dtype, dev, seed=s) for s in range(args.sets)]
    out = torch.empty_like(sets[0]["q"])
    ks = plx.decode_auto_split(w.B, w.Hq, w.Hkv, w.d, w.L)
    ws = torch.empty(max(plx.decode_workspace_size(w.B, w.Hq, w.Hkv, w.d, w.L), 1), dtype=torch.uint8,
                     device=dev)

    def decode_step(i):
        x = sets[i % len(sets)]
        plx.decode(x["q"], x["k"], x["v"], x["rho"], out=out, workspace=ws)

    secs, per = time_steps(decode_step, args.steps, args.warmup, torch)
    kv_bytes = 2 * 2 * w.B * w.Hkv * w.L * w.d
    qro_bytes = 3 * 2 * w.B * w.Hq * w.d
    step_s = secs / args.steps
    gbs = kv_bytes / step_s / 1e9
    flops = 4 * 2 * w.d * w.B * w.Hq * w.L
    digest = source_digest(DECODE_SOURCES)
    traffic = read_traffic(digest)
    log(f"decode: {step_s * 1e6:.1f} us/step, {gbs:.0f} GB/s KV, keys_per_split={ks}")

    result = {
        "metric": "decode KV HBM GB/s (% peak) + prefill TFLOP/s (% MFMA peak)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "context": w.L,
                   "keys_per_split": ks, "input_sets_rotated": args.sets, "accumulate": "fp32"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": "decode_split_kernel + decode_combine_kernel (one parallax_fwd_decode call)",
                     "algorithmic_bytes_per_launch": kv_bytes,
                     "kernel_source_digest": digest},
        "decode_detail": {"us_per_step_median": round(sorted(per)[len(per) // 2] * 1e3, 2),
                          "us_per_step_p10": round(sorted(per)[len(per) // 10] * 1e3, 2),
                          "us_per_step_p90": round(sorted(per)[(9 * len(per)) // 10] * 1e3, 2),
                          "tokens_per_s": round(w.B / step_s, 1),
                          "kv_plus_q_rho_out_GBs": round((kv_bytes + qro_bytes) / step_s / 1e9, 2),
                          "tflops": round(flops / step_s / 1e12, 3)},
    }

    result["build"] = build_info()
    if not args.no_cpu_baseline:
        log("decode CPU baseline (oracle)")
        x0 = sets[0]
        out0 = plx.decode(x0["q"], x0["k"], x0["v"], x0["rho"])
        result["cpu_baseline"] = cpu_baseline_decode(x0, w, args.cpu_budget, gpu_out=out0)
        del out0
    del sets
    torch.cuda.empty_cache()
    if not args.no_context:
        result["decode_other_workloads"] = other_decode_workloads(plx, synth, dev, torch)

    # ---------------- prefill ----------------
    if not args.no_prefill:
        pw = synth.WORKLOADS[PREFILL_WL]
        log(f"prefill workload {pw.name}")
        psets = [synth.make_prefill(pw.B, pw.Hq, pw.Hkv, pw.T, pw.d, pw.dtype, dev, seed=s) for s in range(2)]
        pout = torch.empty_like(psets[0]["q"])

        def prefill_step(i):
            x = psets[i % len(psets)]
            plx.prefill(x["q"], x["k"], x["v"], x["rho"], out=pout)

        def softmax_only_step(i):
            x = psets[i % len(psets)]
            plx.prefill(x["q"], x["k"], x["v"], None, out=pout)

        psecs, pper = time_steps(prefill_step, args.prefill_steps, args.prefill_warmup, torch)
        ptraffic = read_traffic(source_digest(PREFILL_SOURCES), PREFILL_TRAFFIC_FILE)
        pairs = pw.B * pw.Hq * pw.T * (pw.T + 1) // 2
        pflops = 4 * 2 * pw.d * pairs
        tf = pflops / (psecs / args.prefill_steps) / 1e12
        ssecs, _ = time_steps(softmax_only_step, args.prefill_steps, args.prefill_warmup, torch)
        stf = 2 * 2 * pw.d * pairs / (ssecs / args.prefill_steps) / 1e12
        log(f"prefill: {psecs / args.prefill_steps * 1e3:.3f} ms/step, {tf:.1f} TFLOP/s; softmax-only "
            f"{ssecs / args.prefill_steps * 1e3:.3f} ms, {stf:.1f} TFLOP/s")
        result["prefill"] = {
            "workload": pw.name, "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_step": round(psecs / args.prefill_steps * 1e3, 4), "steps": args.prefill_steps,
            "warmup": args.prefill_warmup,
            "us_per_step_median": round(sorted(pper)[len(pper) // 2] * 1e3, 2),
            "us_per_step_p10": round(sorted(pper)[len(pper) // 10] * 1e3, 2),
            "us_per_step_p90": round(sorted(pper)[(9 * len(pper)) // 10] * 1e3, 2),
            "tokens_per_s": round(pw.B * pw.T / (psecs / args.prefill_steps), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": None if ptraffic is None else round(ptraffic),
                         "kernel": "prefill_kernel<bf16, 128, 2, rho>",
                         "algorithmic_flops_per_launch": pflops},
            "softmax_only": {"value": round(stf, 2), "unit": "TFLOP/s",
                             "ms_per_step": round(ssecs / args.prefill_steps * 1e3, 4)},
        }
        if not args.no_context:
            # Context only: the same heads and token count (B * T = 32768) at a longer sequence, where
            # a workgroup's fixed start-up cost is spread over 4x as many key tiles.
            lb, lt = max(1, pw.B // 4), pw.T * 4
            lx = synth.make_prefill(lb, pw.Hq, pw.Hkv, lt, pw.d, pw.dtype, dev, seed=7)
            lout = torch.empty_like(lx["q"])
            lsecs, _ = time_steps(lambda i: plx.prefill(lx["q"], lx["k"], lx["v"], lx["rho"], out=lout),
                                  max(2, args.prefill_steps // 5), max(2, args.prefill_warmup // 5), torch)
            lsteps = max(2, args.prefill_steps // 5)
            ltf = 4 * 2 * pw.d * lb * pw.Hq * lt * (lt + 1) // 2 / (lsecs / lsteps) / 1e12
            log(f"prefill B={lb} T={lt}: {lsecs / lsteps * 1e3:.3f} ms/step, {ltf:.1f} TFLOP/s")
            result["prefill"]["longer_sequence"] = {
                "B": lb, "T": lt, "value": round(ltf, 2), "unit": "TFLOP/s",
                "ms_per_step": round(lsecs / lsteps * 1e3, 4), "frac_of_peak": round(ltf / BF16_MFMA_PEAK_TFLOPS, 4)}
            del lx, lout
        if not args.no_cpu_baseline:
            log("prefill CPU baseline (oracle)")
            x0 = psets[0]
            out0 = plx.prefill(x0["q"], x0["k"], x0["v"], x0["rho"])
            result["prefill"]["cpu_baseline"] = cpu_baseline_prefill(x0, pw, args.cpu_budget, gpu_out=out0)
            del out0

        # ---------------- fused q/k/v/probe projection of the same layer ----------------
        if not args.no_projection:
            dm = pw.Hq * pw.d
            px, pwt = synth.make_projection(pw.B, pw.T, dm, pw.Hq, pw.Hkv, pw.d, pw.dtype, dev)

            def projection_step(i):
                plx.qkvr_projection(px, pwt, pw.Hq, pw.Hkv, pw.d)

            x2 = px.reshape(pw.B * pw.T, dm)
            wt_t = pwt.t()

            def library_gemm_step(i):
                torch.matmul(x2, wt_t)

            jsecs, _ = time_steps(projection_step, args.prefill_steps, args.prefill_warmup, torch)
            lsecs, _ = time_steps(library_gemm_step, args.prefill_steps, args.prefill_warmup, torch)
            jflops = 2 * pw.B * pw.T * (2 * pw.Hq + 2 * pw.Hkv) * pw.d * dm
            jtraffic = read_traffic(source_digest(PROJECTION_SOURCES), PROJECTION_TRAFFIC_FILE)
            jtf = jflops / (jsecs / args.prefill_steps) / 1e12
            log(f"projection: {jsecs / args.prefill_steps * 1e3:.3f} ms, {jtf:.1f} TFLOP/s; library GEMM alone "
                f"{lsecs / args.prefill_steps * 1e3:.3f} ms")
            result["prefill"]["projection"] = {
                "value": round(jtf, 2), "unit": "TFLOP/s", "ms_per_step": round(jsecs / args.prefill_steps * 1e3, 4),
                "shape": {"tokens": pw.B * pw.T, "d_model": dm, "features": (2 * pw.Hq + 2 * pw.Hkv) * pw.d},
                "roofline": {"bound": "mfma", "achieved": round(jtf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(jtf / BF16_MFMA_PEAK_TFLOPS, 4),
                             "traffic": jtraffic if jtraffic is None else round(jtraffic),
                             "kernel": "projection_kernel (one parallax_qkvr_projection call)"},
                "context_library_gemm_ms": round(lsecs / args.prefill_steps * 1e3, 4),
            }
            del px, pwt, x2, wt_t

        # ---------------- prefill backward (training step of the layer) ----------------
        if not args.no_backward:
            x = psets[0]
            dout = synth.make_upstream_grad(tuple(x["q"].shape), pw.dtype, dev)
            fw = plx.prefill_train(x["q"], x["k"], x["v"], x["rho"])
            ws = torch.empty(max(16, pw.B * pw.Hq * pw.T * 16), dtype=torch.uint8, device=dev)

            def backward_step(i):
                plx.prefill_backward(x["q"], x["k"], x["v"], x["rho"], *fw, dout, workspace=ws)

            def train_forward_step(i):
                plx.prefill_train(x["q"], x["k"], x["v"], x["rho"])

            bsecs, bper = time_steps(backward_step, args.backward_steps, args.backward_warmup, torch)
            fsecs, _ = time_steps(train_forward_step, args.backward_steps, args.backward_warmup, torch)
            # Algorithmic work: 8 GEMM-equivalents of 2d flops per causal pair
            # (recomputed S and R, g = dO.v, dV, dQ, dK from dS and from dR,
            # dRho); the kernels execute 11, since dq and dk/dv each recompute
            # S, R and g.
            bflops = 8 * 2 * pw.d * pairs
            btraffic = read_traffic(source_digest(BACKWARD_SOURCES), BACKWARD_TRAFFIC_FILE)
            btf = bflops / (bsecs / args.backward_steps) / 1e12
            log(f"backward: {bsecs / args.backward_steps * 1e3:.3f} ms/step, {btf:.1f} TFLOP/s; training forward "
                f"{fsecs / args.backward_steps * 1e3:.3f} ms")
            result["prefill"]["backward"] = {
                "value": round(btf, 2), "unit": "TFLOP/s", "ms_per_step": round(bsecs / args.backward_steps * 1e3, 4),
                "steps": args.backward_steps, "warmup": args.backward_warmup,
                "us_per_step_median": round(sorted(bper)[len(bper) // 2] * 1e3, 2),
                "algorithmic_flops_per_step": bflops, "executed_gemm_equivalents": 11,
                "roofline": {"bound": "mfma", "achieved": round(btf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(btf / BF16_MFMA_PEAK_TFLOPS, 4),
                             "traffic": btraffic if btraffic is None else round(btraffic),
                             "kernel": "bwd_dq + bwd_dkdv (one parallax_bwd_prefill call)"},
                "training_forward_ms": round(fsecs / args.backward_steps * 1e3, 4),
            }
            if not args.no_cpu_baseline:
                log("backward CPU baseline (oracle)")
                result["prefill"]["backward"]["cpu_baseline"] = cpu_baseline_backward(x, dout, pw)

    if not args.no_prefill:
        log("fp32 prefill (B=1, Hq=Hkv=2, T=256, d=64)")
        result["prefill_f32"] = prefill_f32_leg(torch, plx, synth)
    if not args.no_sweep:
        log(f"decode sweep (budget {args.sweep_budget:.0f} s)")
        result["sweep"] = run_sweep(torch, plx, synth, diag, args.sweep_budget)

    if not args.no_device:
        log("device ceilings: streaming read, MFMA-only kernel")
        dv = measure_device(torch)
        result["device"] = dv
        m = dv["measured"]
        result["roofline"]["frac_of_measured_stream_read"] = round(gbs / m["stream_read_nontemporal_GBs"], 4)
        if "prefill" in result:
            pr = result["prefill"]
            for part in (pr, pr.get("projection"), pr.get("backward")):
                if part is not None:
                    part["roofline"]["frac_of_measured_mfma"] = round(part["value"] / m["bf16_mfma_tflops"], 4)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
