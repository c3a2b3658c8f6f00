"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one synthetic batch:
fa_fwd (O and LSE) followed by fa_bwd (dQ, dK, dV by recomputation), at
B=1, H=8, N=16384, d=128, bf16, non-causal -- the shape of the pages'
sequence-length benchmark at its largest N (FlashAttention-2 principle and
deployment page, benchmark section).  Inputs are resident in HBM before the
timed region.  The forward and backward calls are bracketed by HIP events on
the stream they run on, so their per-call durations are measured live.

Prints ONE JSON line.  `value` is the forward's algorithmic TFLOP/s
(4*B*H*N^2*d over the median HIP-event time of fa_fwd), the metric's first
figure; the backward (10*B*H*N^2*d) and the whole step are reported beside it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from aware_exact_attention_amd import fa  # noqa: E402
from aware_exact_attention_amd.inputs import WORKLOADS, make_inputs, to_f64  # noqa: E402

METRIC = "attn fwd TFLOP/s & % bf16 MFMA peak at B1 H8 N16K d128; bwd TFLOP/s"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 vector (the f32 path runs on the vector ALUs)
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "aware_exact_attention_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_traffic_B1H8N16384d128.txt")
COPY_BYTES = 1 << 30          # size of the calibration copy (read and written once each)
# kernels of one step, as named in rocprofv3 output
FWD_KERNELS = ("fwd_kernel",)
BWD_KERNELS = ("bwd_pre_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel")


def kernel_source_hash() -> str:
    """Hash of the HIP sources; traffic counters are only valid for the kernels they were taken on."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="bwd_16k", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-next-rows", action="store_true", help="skip the split-KV / merge measurements")
    p.add_argument("--cpu-heads", type=int, default=1, help="heads of the workload the oracle is timed on")
    p.add_argument("--traffic-json", default=TRAFFIC_FILE,
                   help="HBM bytes per launch measured with rocprofv3 counters (written by --traffic-from)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain device copy of COPY_BYTES (for the FETCH_SIZE / WRITE_SIZE calibration)")
    p.add_argument("--trace-summary", metavar="TRACE_DIR",
                   help="summarise a rocprofv3 --kernel-trace run of this benchmark (the last --steps dispatches "
                        "of each kernel) as a markdown table, then exit")
    p.add_argument("--traffic-from", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                   help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output of the bench and of --copy-calibration "
                        "into the traffic summary, then exit")
    return p.parse_args()


def _counter_means(d: str, counter: str):
    """Mean per-dispatch value of `counter` for every kernel in a rocprofv3 counter_collection CSV."""
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def traffic_from(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out_path):
    """HBM bytes per launch = FETCH_SIZE + WRITE_SIZE (KiB per dispatch), each scaled by
    the factor that makes the same counter read COPY_BYTES for a plain copy of COPY_BYTES."""
    def per_kernel(d, counter):
        m = _counter_means(d, counter)
        return {n: sum(v for k, v in m.items() if n in k) * 1024 for n in FWD_KERNELS + BWD_KERNELS}

    def copy_bytes_raw(d, counter):
        m = _counter_means(d, counter)
        big = [v for k, v in m.items() if "copy" in k.lower() or "elementwise" in k.lower()]
        return max(big) * 1024 if big else None

    cf, cw = copy_bytes_raw(copy_fetch_dir, "FETCH_SIZE"), copy_bytes_raw(copy_write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / cf if cf else None
    w_scale = COPY_BYTES / cw if cw else None
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    res = {"source_hash": kernel_source_hash(), "copy_bytes": COPY_BYTES,
           "copy_fetch_bytes_raw": cf, "copy_write_bytes_raw": cw, "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": {}}
    for group, names in (("fwd", FWD_KERNELS), ("bwd", BWD_KERNELS)):
        tot = 0.0
        for n in names:
            fb, wb = fetch[n] * (f_scale or 1.0), write[n] * (w_scale or 1.0)
            res["kernels"][n] = {"fetch_bytes": round(fb), "write_bytes": round(wb)}
            tot += fb + wb
        res[group] = round(tot)
    with open(out_path, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res))


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES bytes, five times."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "calls": 5}))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, do, heads: int):
    """Time the fp64 oracle (as it stands) on `heads` heads of the workload on the host cores,
    and single-threaded on the two smallest workloads (tiny fp32, one GPT-2-shaped head)."""
    import numpy as np  # noqa: F401
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))
    sl = (slice(0, 1), slice(0, heads))
    args = [to_f64(t[sl]) for t in (q, k, v, do)]
    t0 = time.perf_counter()
    oracle.ref_fwd(*args[:3], w.scale, w.causal)
    t1 = time.perf_counter()
    oracle.ref_bwd(*args, w.scale, w.causal)
    t2 = time.perf_counter()
    frac = heads / (w.B * w.H)
    flop = (w.fwd_flop + w.bwd_flop) * frac
    single = {}
    for name, nheads in (("tiny_f32", 1), ("gpt2", 1)):
        wl = WORKLOADS[name]
        ins = make_inputs(wl.B, wl.H, wl.N, wl.d, wl.dtype, wl.seed, wl.qk_std)
        a = [to_f64(t[:1, :nheads]) for t in ins]
        reps = 20 if name == "tiny_f32" else 3
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                s0 = time.perf_counter()
                for _ in range(reps):
                    oracle.ref_fwd(*a, wl.scale, wl.causal)
                dt = (time.perf_counter() - s0) / reps
        else:  # pragma: no cover
            dt = float("nan")
        fl = wl.fwd_flop * nheads / (wl.B * wl.H)
        single[name] = {"s_per_head_fwd": round(dt, 6), "gflops": round(fl / dt / 1e9, 3), "threads": 1,
                        "sample": f"ref_fwd on {nheads} of {wl.B * wl.H} heads, mean of {reps} calls"}
    return {
        "value": round(flop / (t2 - t0) / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"fp64 oracle ref_fwd + ref_bwd on {heads} of {w.B * w.H} heads of the benchmark workload "
                  f"(N={w.N}, d={w.d}); fwd {t1 - t0:.2f} s, bwd {t2 - t1:.2f} s; TFLOP/s of that sample",
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "single_thread": single,
    }


def mfma_ceiling():
    """The bf16 MFMA rate the GPU sustains (fa_probe_mfma_bf16: four independent
    chains per wave, two waves per SIMD, register operands), next to the spec."""
    wgs, iters = 2048, 4000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    fa.probe_mfma_bf16(wgs, iters, sink)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fa.probe_mfma_bf16(wgs, iters, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = statistics.median(ts)
    flop = wgs * 4 * iters * 4 * 32768
    tf = flop / (ms * 1e-3) / 1e12
    return {"measured_tflops": round(tf, 1), "spec_tflops": PEAK_BF16_TFLOPS,
            "frac_of_spec": round(tf / PEAK_BF16_TFLOPS, 4),
            "clock_ghz_at_full_mfma_rate": round(tf * 1e12 / (256 * 4096) / 1e9, 3),
            "probe": f"fa_probe_mfma_bf16: {wgs} workgroups x 4 waves x {iters} x 4 chains of "
                     f"v_mfma_f32_32x32x16_bf16, median of 5 calls ({ms:.3f} ms)"}


def trace_summary(trace_dir: str, steps: int):
    """Markdown table of a rocprofv3 kernel trace of this benchmark: per kernel of the
    step, mean and median duration over its last `steps` dispatches (the timed steps;
    warm-up calls excluded) and the fraction of the bf16 peak at the algorithmic FLOP."""
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    w = WORKLOADS["bwd_16k"]
    per = {}
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        name = r["Kernel_Name"]
        for n in FWD_KERNELS + BWD_KERNELS:
            if n in name:
                per.setdefault(n, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| Kernel | Dispatches in trace | Mean of last %d (us) | Median of last %d (us) |" % (steps, steps),
           "|---|---|---|---|"]
    means = {}
    for n in FWD_KERNELS + BWD_KERNELS:
        ds = per.get(n, [])[-steps:]
        if not ds:
            continue
        means[n] = (statistics.mean(ds), statistics.median(ds))
        out.append(f"| `{n}` | {len(per[n])} | {means[n][0]:.1f} | {means[n][1]:.1f} |")
    f_us = means.get("fwd_kernel", (float("nan"),) * 2)
    b_us = [sum(means[n][i] for n in BWD_KERNELS if n in means) for i in (0, 1)]
    out.append("")
    for label, flop, us in (("forward (fwd_kernel)", w.fwd_flop, f_us),
                            ("backward (sum of the three kernels)", w.bwd_flop, b_us)):
        tf = [flop / (u * 1e-6) / 1e12 for u in us]
        out.append(f"- {label}: mean {us[0]:.1f} us -> {tf[0]:.1f} TFLOP/s = {tf[0] / PEAK_BF16_TFLOPS:.4f} of "
                   f"{PEAK_BF16_TFLOPS}; median {us[1]:.1f} us -> {tf[1]:.1f} TFLOP/s = "
                   f"{tf[1] / PEAK_BF16_TFLOPS:.4f}")
    print("\n".join(out))


def _graph_ms(fn, calls: int, warmup: int = 3) -> float:
    """GPU time per call of `fn`: `calls` back-to-back calls captured in one HIP
    graph, replayed 5 times between HIP events (median), so that host-side call
    overhead does not show in the times of kernels of a few microseconds.  The
    library's calls allocate nothing and only launch kernels, so they capture."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    rounds = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        rounds.append(e0.elapsed_time(e1) / calls)
    return sorted(rounds)[len(rounds) // 2]


def config_rows():
    """Every configuration of the task at its own shape: forward (and, for the
    forward+backward config, backward) time, TFLOP/s and fraction of the bf16
    peak; the sequence-length sweep per N.  Graph-replayed calls."""
    res = {}
    for name in ("tiny_f32", "gpt2", "gpt2_causal", "sweep_2k", "sweep_4k", "sweep_8k", "sweep_16k",
                 "stress_causal", "fwd_bwd_causal"):
        w = WORKLOADS[name]
        ts = make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_std, backward=w.backward)
        q, k, v = (t.cuda() for t in ts[:3])
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        # enough calls per replay (about 20 ms of work at the large shapes) that
        # the clock has settled after the host-side input generation
        calls = max(3, min(50, int(2e13 / max(w.fwd_flop, 1))))
        t_f = _graph_ms(lambda: fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse), calls)
        # peak device memory of one call: the library allocates nothing, so it is the
        # caller's q, k, v, o and lse (the pages' second benchmark column)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        peak_bytes = torch.cuda.max_memory_allocated()
        extra = peak_bytes - base
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        r = {"shape": [w.B, w.H, w.N, w.d], "dtype": w.dtype, "causal": w.causal,
             "peak_tflops": peak,
             "fwd_ms": round(t_f, 5), "fwd_tflops": round(w.fwd_flop / (t_f * 1e-3) / 1e12, 1),
             "fwd_frac_peak": round(w.fwd_flop / (t_f * 1e-3) / 1e12 / peak, 4),
             "peak_mem_gb": round(peak_bytes / 1e9, 4), "fwd_extra_alloc_bytes": int(extra)}
        if w.backward:
            do = ts[3].cuda()
            grads = tuple(torch.empty_like(q) for _ in range(3))
            ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
            t_b = _graph_ms(lambda: fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, workspace=ws,
                                           out=grads), max(3, min(50, int(2e13 / w.bwd_flop))))
            r.update({"bwd_ms": round(t_b, 5), "bwd_tflops": round(w.bwd_flop / (t_b * 1e-3) / 1e12, 1),
                      "bwd_frac_peak": round(w.bwd_flop / (t_b * 1e-3) / 1e12 / peak, 4)})
        res[name] = r
    return res


def next_rows():
    """Key-split forward (fa_fwd_splitkv) against fa_fwd, and fa_bwd, on grids too
    small to fill the GPU, the sliding-window and block-sparse forwards, fp16 inputs, dropout,
    and the Eq. (2) merge kernel (fa_lse_merge) against the HBM roof."""
    res = {}
    for name, (B, H, N, d, causal) in {"B1H8N2048d128": (1, 8, 2048, 128, False),
                                       "B1H4N4096d128_causal": (1, 4, 4096, 128, True),
                                       "B1H2N8192d64": (1, 2, 8192, 64, False)}.items():
        q, k, v, do = (t.cuda() for t in make_inputs(B, H, N, d, "bf16", 9, 1.0, backward=True))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        parts = fa.splitkv_parts(B, H, N, d, 0)
        ws = torch.empty(max(fa.splitkv_workspace_bytes(B, H, N, d, 0), 16), dtype=torch.uint8, device="cuda")
        flop = 4 * B * H * N * N * d / (2 if causal else 1)
        t_f = _graph_ms(lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse), 20)
        t_s = _graph_ms(lambda: fa.fwd_splitkv(q, k, v, causal=causal, workspace=ws, out=o, lse=lse), 20)
        assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
        # the backward of these small grids runs its dK/dV and dQ passes in one launch
        wsb = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
        grads = tuple(torch.empty_like(q) for _ in range(3))
        t_b = _graph_ms(lambda: fa.bwd(q, k, v, o, lse, do, causal=causal, workspace=wsb, out=grads), 20)
        res[name] = {"parts": parts, "fa_fwd_ms": round(t_f, 5), "fa_fwd_splitkv_ms": round(t_s, 5),
                     "speedup": round(t_f / t_s, 3), "splitkv_tflops": round(flop / (t_s * 1e-3) / 1e12, 1),
                     "splitkv_frac_peak": round(flop / (t_s * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "fa_bwd_ms": round(t_b, 5), "bwd_tflops": round(2.5 * flop / (t_b * 1e-3) / 1e12, 1)}
    # tile-skipping masks at the benchmark shape: FLOP counted on the visible (query, key) pairs only
    B, H, N, d = 1, 8, 16384, 128
    q, k, v = (t.cuda() for t in make_inputs(B, H, N, d, "bf16", 9, 1.0))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    t_d = _graph_ms(lambda: fa.fwd(q, k, v, out=o, lse=lse), 5)
    pairs = sum(min(N - 1, i + 512) - max(0, i - 512) + 1 for i in range(N))
    t_w = _graph_ms(lambda: fa.fwd_window(q, k, v, 512, 512, out=o, lse=lse), 10)
    fl_w = 4 * B * H * pairs * d
    dob = torch.randn(q.shape, generator=torch.Generator().manual_seed(10)).to(torch.bfloat16).cuda()
    grads = tuple(torch.empty_like(q) for _ in range(3))
    wsb = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    fa.fwd_window(q, k, v, 512, 512, out=o, lse=lse)
    t_wb = _graph_ms(lambda: fa.bwd_window(q, k, v, o, lse, dob, 512, 512, workspace=wsb, out=grads), 10)
    res["window_512_512_B1H8N16384d128"] = {
        "ms": round(t_w, 5), "visible_fraction": round(pairs / N / N, 4), "dense_fa_fwd_ms": round(t_d, 5),
        "tflops_visible": round(fl_w / (t_w * 1e-3) / 1e12, 1),
        "frac_peak": round(fl_w / (t_w * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_ms": round(t_wb, 5), "bwd_tflops_visible": round(2.5 * fl_w / (t_wb * 1e-3) / 1e12, 1),
        "bwd_frac_peak": round(2.5 * fl_w / (t_wb * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    nb = N // 64
    g = torch.Generator().manual_seed(9)
    bm = (torch.rand((nb, nb), generator=g) < 0.5).to(torch.uint8)
    kept = int(bm.sum())
    bmd = bm.cuda()
    t_b = _graph_ms(lambda: fa.fwd_blocksparse(q, k, v, bmd, out=o, lse=lse), 5)
    fl_b = 4 * B * H * kept * 64 * 64 * d
    fa.fwd_blocksparse(q, k, v, bmd, out=o, lse=lse)
    t_bb = _graph_ms(lambda: fa.bwd_blocksparse(q, k, v, o, lse, dob, bmd, workspace=wsb, out=grads), 5)
    res["blocksparse_half_B1H8N16384d128"] = {
        "ms": round(t_b, 5), "kept_blocks": round(kept / nb / nb, 4), "dense_fa_fwd_ms": round(t_d, 5),
        "tflops_visible": round(fl_b / (t_b * 1e-3) / 1e12, 1),
        "frac_peak": round(fl_b / (t_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_ms": round(t_bb, 5), "bwd_tflops_visible": round(2.5 * fl_b / (t_bb * 1e-3) / 1e12, 1),
        "bwd_frac_peak": round(2.5 * fl_b / (t_bb * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    # fp16 inputs at the benchmark shape (fa_fwd_fp16, fa_bwd_fp16)
    q16, k16, v16, do16 = (t.cuda() for t in make_inputs(B, H, N, d, "fp16", 9, 1.0, backward=True))
    o16 = torch.empty_like(q16)
    grads16 = tuple(torch.empty_like(q16) for _ in range(3))
    ws16 = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    t_f16 = _graph_ms(lambda: fa.fwd(q16, k16, v16, out=o16, lse=lse), 3)
    t_b16 = _graph_ms(lambda: fa.bwd(q16, k16, v16, o16, lse, do16, workspace=ws16, out=grads16), 3)
    fl_f = 4 * B * H * N * N * d
    res["fp16_B1H8N16384d128"] = {
        "fwd_ms": round(t_f16, 5), "fwd_tflops": round(fl_f / (t_f16 * 1e-3) / 1e12, 1),
        "fwd_frac_peak": round(fl_f / (t_f16 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_ms": round(t_b16, 5), "bwd_tflops": round(2.5 * fl_f / (t_b16 * 1e-3) / 1e12, 1),
        "bwd_frac_peak": round(2.5 * fl_f / (t_b16 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "peak_note": "fp16 dense MFMA peak equals bf16's (2516.6 TFLOP/s)"}
    # head dimension 96 (LDS rows padded to 256 bytes) at B1 H8 N16384, bf16
    q96, k96, v96, do96 = (t.cuda() for t in make_inputs(B, H, N, 96, "bf16", 9, 1.0, backward=True))
    o96 = torch.empty_like(q96)
    g96 = tuple(torch.empty_like(q96) for _ in range(3))
    ws96 = torch.empty(fa.bwd_workspace_bytes(B, H, N, 96), dtype=torch.uint8, device="cuda")
    t_f96 = _graph_ms(lambda: fa.fwd(q96, k96, v96, out=o96, lse=lse), 3)
    t_b96 = _graph_ms(lambda: fa.bwd(q96, k96, v96, o96, lse, do96, workspace=ws96, out=g96), 3)
    fl_96 = 4 * B * H * N * N * 96
    res["d96_B1H8N16384"] = {
        "fwd_ms": round(t_f96, 5), "fwd_tflops": round(fl_96 / (t_f96 * 1e-3) / 1e12, 1),
        "fwd_frac_peak": round(fl_96 / (t_f96 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_ms": round(t_b96, 5), "bwd_tflops": round(2.5 * fl_96 / (t_b96 * 1e-3) / 1e12, 1),
        "bwd_frac_peak": round(2.5 * fl_96 / (t_b96 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q96, k96, v96, do96, o96, g96, ws96
    # head dimension 256 (one wave per SIMD) at B1 H8 N16384, bf16
    q256, k256, v256, do256 = (t.cuda() for t in make_inputs(B, H, N, 256, "bf16", 9, 1.0, backward=True))
    o256 = torch.empty_like(q256)
    g256 = tuple(torch.empty_like(q256) for _ in range(3))
    ws256 = torch.empty(fa.bwd_workspace_bytes(B, H, N, 256), dtype=torch.uint8, device="cuda")
    t_f256 = _graph_ms(lambda: fa.fwd(q256, k256, v256, out=o256, lse=lse), 3)
    t_b256 = _graph_ms(lambda: fa.bwd(q256, k256, v256, o256, lse, do256, workspace=ws256, out=g256), 2)
    fl_256 = 4 * B * H * N * N * 256
    res["d256_B1H8N16384"] = {
        "fwd_ms": round(t_f256, 5), "fwd_tflops": round(fl_256 / (t_f256 * 1e-3) / 1e12, 1),
        "fwd_frac_peak": round(fl_256 / (t_f256 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_ms": round(t_b256, 5), "bwd_tflops": round(2.5 * fl_256 / (t_b256 * 1e-3) / 1e12, 1),
        "bwd_frac_peak": round(2.5 * fl_256 / (t_b256 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q256, k256, v256, do256, o256, g256, ws256
    # dropout p = 0.1 at the benchmark shape (fa_fwd_dropout, fa_bwd_dropout)
    t_fd = _graph_ms(lambda: fa.fwd_dropout(q, k, v, 0.1, 1234, out=o, lse=lse), 3)
    t_bd = _graph_ms(lambda: fa.bwd_dropout(q, k, v, o, lse, dob, 0.1, 1234, workspace=ws16, out=grads), 3)
    res["dropout_p0.1_B1H8N16384d128"] = {
        "fwd_ms": round(t_fd, 5), "fwd_tflops": round(fl_f / (t_fd * 1e-3) / 1e12, 1),
        "bwd_ms": round(t_bd, 5), "bwd_tflops": round(2.5 * fl_f / (t_bd * 1e-3) / 1e12, 1),
        "note": "FLOP of the attention products only; the mask's Philox draws are VALU work on top"}
    # merge kernel alone: S = 4 parts of B1 H8 N2048 d128
    S, B, H, N, d = 4, 1, 8, 2048, 128
    g = torch.Generator().manual_seed(9)
    op = torch.randn((S, B, H, N, d), generator=g).cuda()
    lp = torch.randn((S, B, H, N), generator=g).cuda()
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    t_m = _graph_ms(lambda: fa.lse_merge(op, lp, out=o, lse=lse), 50)
    rows = B * H * N
    mbytes = S * rows * d * 4 + S * rows * 4 + rows * d * 2 + rows * 4
    gbs = mbytes / (t_m * 1e-3) / 1e9
    res["lse_merge_S4_B1H8N2048d128"] = {"ms": round(t_m, 5), "algorithmic_bytes": mbytes,
                                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                                      "frac": round(gbs / PEAK_HBM_GBS, 4)}}
    return res


def main():
    a = parse()
    if a.trace_summary:
        trace_summary(a.trace_summary, a.steps)
        return
    if a.traffic_from:
        traffic_from(*a.traffic_from, a.traffic_json)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": a.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    fa.load()
    w = WORKLOADS[a.workload]
    q, k, v, do = make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_std, backward=True)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, workspace=ws, out=grads)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    for t in (o, lse) + grads:
        assert torch.isfinite(t).all().item(), "non-finite output"

    ms_step = (t1 - t0) * 1e3 / a.steps

    def stats(ms):
        return {"ms_mean": round(statistics.mean(ms), 4), "ms_median": round(statistics.median(ms), 4),
                "ms_min": round(min(ms), 4)}

    f_ms = statistics.median(fwd_ms)
    b_ms = statistics.median(bwd_ms)
    f_tf = w.fwd_flop / (f_ms * 1e-3) / 1e12
    b_tf = w.bwd_flop / (b_ms * 1e-3) / 1e12
    step_tf = (w.fwd_flop + w.bwd_flop) / (ms_step * 1e-3) / 1e12

    # measured HBM bytes per launch, valid only for the kernel sources they were taken on
    traffic = {}
    if a.workload == "bwd_16k" and a.traffic_json and os.path.exists(a.traffic_json):
        t = json.load(open(a.traffic_json))
        if t.get("source_hash") == kernel_source_hash():
            traffic = t

    def roof(flop, ms, key):
        ach = flop / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic.get(key)}

    # The backward call (2.5x the forward's algorithmic FLOPs) dominates the step.
    r_bwd = roof(w.bwd_flop, b_ms, "bwd")
    r_bwd["kernel"] = ("fa_bwd: bwd_pre_kernel + bwd_dkdv_kernel + bwd_dq_kernel (one HIP event pair around the "
                       "call, median over the timed steps); FLOP = 10*B*H*N^2*d algorithmic (the dQ pass's "
                       "recompute of S and dP not counted)")
    r_fwd = roof(w.fwd_flop, f_ms, "fwd")
    r_fwd["kernel"] = "fa_fwd: fwd_kernel (bf16, 8 waves; median over the timed steps); FLOP = 4*B*H*N^2*d"
    bytes_fwd = w.B * w.H * w.N * (8 * w.d + 4)
    bytes_bwd = w.B * w.H * w.N * (16 * w.d + 12)

    out = {
        "metric": METRIC,
        "value": round(f_tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"attention fwd+bwd B{w.B} H{w.H} N{w.N} d{w.d} bf16 "
                               f"{'causal' if w.causal else 'non-causal'}, seeded N(0,1) inputs",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal, "seed": w.seed},
        "value_is": "forward TFLOP/s (4*B*H*N^2*d over the median event time of fa_fwd)",
        "fwd": {"ms": round(f_ms, 4), **stats(fwd_ms), "tflops": round(f_tf, 2),
                "frac_peak": round(f_tf / PEAK_BF16_TFLOPS, 4), "algorithmic_bytes": bytes_fwd,
                "pages_a100_context": "pages: 28.5 ms (38.6 TFLOP/s derived) on an A100 at this shape, forward only"},
        "bwd": {"ms": round(b_ms, 4), **stats(bwd_ms), "tflops": round(b_tf, 2),
                "frac_peak": round(b_tf / PEAK_BF16_TFLOPS, 4), "algorithmic_bytes": bytes_bwd},
        "step": {"ms": round(ms_step, 4), "tflops": round(step_tf, 2),
                 "note": "fa_fwd + fa_bwd per step, host wall clock around the timed steps"},
        "roofline": r_bwd,
        "roofline_fwd": r_fwd,
    }
    out["mfma_ceiling"] = mfma_ceiling()
    if not a.no_next_rows:
        out["configs"] = config_rows()
        out["next_rows"] = next_rows()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, do, a.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
