"""Benchmark of the LVSA hot path on one MI355X.

One step = one denoising step of the attention hot path over the whole
workload: build the step's CSR mask on the host (C++), copy it to the device,
run the frame-block-sparse attention on [B, H, T·P, d] bf16 (by default
through lvsa_attention_ws: a key-norm pass, then the attention kernel
with a fixed softmax reference where the norm bound allows; --no-workspace times
lvsa_attention, the running-max path).  The
default workload is the Wan-2.1-1.3B-shaped 6× horizon: B=1, H=12, d=128,
T=121 latent frames × 1560 tokens (480×832 video), C=21, W=9, anchors
rotating with the step (seeded synthetic N(0,1) inputs, resident in HBM before
the timed region).

Prints ONE JSON line on stdout (everything else goes to stderr):
  value         effective TFLOP/s = algorithmic FLOPs 4·B·H·T·min(C,T)·P²·d
                per step ÷ time per step (padding and softmax not counted)
  roofline      the attention kernel: HIP events around each launch on its
                stream, against the vendor bf16 peak and against the peak a
                matrix-core microbenchmark measures on this GPU
                (libmfma_peak.so); the L2-to-fabric bytes per launch from the
                committed rocprofv3 counter summary (null once the kernel
                source differs from the one the counters were taken on)
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same step,
                and the pure-Python oracle mask builder per step
  also          per-call kernel median/p10/p90, host mask build and mask H2D
                times, dense comparator (same kernel, C = T mask) and speedup,
                peak device memory; an outside reference (torch SDPA, flash
                backend, dense, same tensors); the same steps with every mask built
                ahead of time (one launch per step, and one HIP-graph replay
                of the whole sequence); for workloads at the training horizon
                (T <= C) the full-step / dense-kernel time ratios.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload wan13b_6x]
    python bench.py --sweep [--sweep-out FILE]   # every workload, table on stderr
    python bench.py --library OTHER/liblvsa.so   # time another build (A/B)
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure (2.4 GHz engine clock)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, vendor figure
METRIC = "LVSA attention effective TFLOP/s + ms/call, T=121×1560 tok, H=12 d=128 bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_wan13b_6x.json")
KERNEL_SOURCES = [os.path.join(ROOT, "block_sparse_attention_lvsa_amd", "csrc", "attention.hip")]
SWEEP = ["wan13b_1x", "syn_1p5x", "syn_2x", "wan13b_6x", "wan14b_6x", "wan22_720p_6x_h5", "wan13b_720p_6x"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """sha256[:16] of the kernel source's code: line comments, trailing
    spaces and blank lines are dropped, so that a comment edit does not void
    counter records taken on the same code."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def algorithmic_flops(w) -> float:
    return 4.0 * w.B * w.H * w.T * min(w.C, w.T) * w.P * w.P * w.D


def measured_traffic(w):
    """The committed rocprofv3 counter record of the attention kernel
    (L2-to-fabric bytes per launch and their spread over launches), or None
    when it is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_hash() or rec.get("workload") != w.name:
        return None
    return rec


def mfma_peak_probe(seconds=0.5):
    """Sustained dense bf16 MFMA rate of this GPU (TFLOP/s) and its engine
    clock (MHz), from libmfma_peak.so; (None, None) if it is not built."""
    path = os.path.join(ROOT, "block_sparse_attention_lvsa_amd", "libmfma_peak.so")
    if not os.path.exists(path):
        return None, None
    lib = ctypes.CDLL(path)
    lib.lvsa_probe_mfma_peak.restype = ctypes.c_int
    lib.lvsa_probe_mfma_peak.argtypes = [ctypes.c_double, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double)]
    tf, mhz = ctypes.c_double(0), ctypes.c_double(0)
    if lib.lvsa_probe_mfma_peak(seconds, ctypes.byref(tf), ctypes.byref(mhz)) != 0:
        return None, None
    return tf.value, mhz.value


def cpu_baseline(w, q, k, v, budget_s: float):
    """The float64 oracle on a bounded sample: query frames of head 0 at step
    0, taken in order until ``budget_s`` of CPU time is used.  Also times the
    pure-Python oracle mask builder per step (steps 0..49), beside the C++
    builder's time the GPU leg reports."""
    import torch
    import oracle

    m0 = time.perf_counter()
    for s in range(50):
        oracle.build_mask(w.T, w.C, w.W, s)
    mask_us = (time.perf_counter() - m0) / 50 * 1e6
    rows = oracle.key_frames(w.T, w.C, w.W, 0)
    qh, kh, vh = (x[:, :1].cpu() for x in (q, k, v))
    threads = torch.get_num_threads()
    per_frame = 4.0 * min(w.C, w.T) * w.P * w.P * w.D
    done = 0
    t0 = time.perf_counter()
    while done < w.T and time.perf_counter() - t0 < budget_s:
        oracle.block_attention(qh, kh, vh, rows, frames=[done])
        done += 1
    dt = time.perf_counter() - t0
    return {
        "value": per_frame * done / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{w.name}: head 0, step 0, query frames 0..{done - 1} ({done} of {w.T} frames × {w.H} heads), "
                  f"float64 torch-CPU, {dt:.1f} s, {threads} threads of {os.cpu_count()} host CPUs",
        "oracle_mask_us_per_step": round(mask_us, 1),
    }


def sdpa_flash_dense_ms(q, k, v, reps=2):
    """Outside reference, not on the LVSA path: torch's scaled_dot_product_attention
    on the same tensors, dense (no mask), restricted to its flash backend (an
    error instead of a fallback to the score-materialising math path).
    Returns (ms per call, None) or (None, reason)."""
    import torch
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            torch.nn.functional.scaled_dot_product_attention(q, k, v)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                torch.nn.functional.scaled_dot_product_attention(q, k, v)
            e1.record()
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, None
    except Exception as ex:  # backend unavailable for this build or shape
        return None, f"{type(ex).__name__}: {str(ex)[:160]}"


def pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(p * len(xs)))]


def run_workload(w, steps, warmup, dense, calib_copy=False, keep_inputs=False, modes=True, workspace=True):
    """Times `steps` full hot-path steps of workload `w`; returns a dict."""
    import torch
    import block_sparse_attention_lvsa_amd as L
    from block_sparse_attention_lvsa_amd.synth import make_qkv

    dev = torch.device("cuda:0")
    lib = L.library()
    torch.cuda.synchronize(dev)  # initialises the device before the memory statistics are reset
    torch.cuda.reset_peak_memory_stats(dev)
    q, k, v = make_qkv(w, device=dev)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    if calib_copy:
        # Reads exactly 2^30 bytes and writes 2^30 bytes per launch: the
        # reference that scales rocprofv3's FETCH_SIZE / WRITE_SIZE readings.
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    T, C, W = w.T, w.C, w.W
    nnz = L.lvsa_mask_nnz(T, C, W)
    total = warmup + steps
    # One pinned host buffer pair per step (the host never rewrites a buffer
    # whose copy may still be pending) and one device pair (same stream, so
    # copy s+1 runs after kernel s).
    h_rp = [torch.empty(T + 1, dtype=torch.int32, pin_memory=True) for _ in range(total)]
    h_ci = [torch.empty(nnz, dtype=torch.int32, pin_memory=True) for _ in range(total)]
    d_rp = torch.empty(T + 1, dtype=torch.int32, device=dev)
    d_ci = torch.empty(nnz, dtype=torch.int32, device=dev)
    info = L.LvsaMaskInfo()
    recs = [L._tensor_record(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
    # With a workspace the call is lvsa_attention_ws: a key-norm pass, then
    # the attention with a fixed softmax reference where the bound allows.
    ws_bytes = L.lvsa_attention_workspace_bytes(w.B, w.H, T * w.P, w.D, T) if workspace else 0
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def attention(rp_ptr, ci_ptr, sptr):
        if workspace:
            return lib.lvsa_attention_ws(ctypes.byref(recs[0]), ctypes.byref(recs[1]), ctypes.byref(recs[2]),
                                         ctypes.c_void_p(rp_ptr), ctypes.c_void_p(ci_ptr), T, nnz,
                                         ctypes.byref(recs[3]), 0.0, ctypes.c_void_p(ws.data_ptr()), ws_bytes, sptr)
        return lib.lvsa_attention(ctypes.byref(recs[0]), ctypes.byref(recs[1]), ctypes.byref(recs[2]),
                                  ctypes.c_void_p(rp_ptr), ctypes.c_void_p(ci_ptr), T, nnz,
                                  ctypes.byref(recs[3]), 0.0, sptr)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    I32P = ctypes.POINTER(ctypes.c_int32)

    def step(i, s, ev=None, mask_times=None):
        t0 = time.perf_counter()
        rc = lib.lvsa_build_mask(T, C, W, s, L.LVSA_ROT_MOD_TPER,
                                 ctypes.cast(ctypes.c_void_p(h_rp[i].data_ptr()), I32P),
                                 ctypes.cast(ctypes.c_void_p(h_ci[i].data_ptr()), I32P), nnz, ctypes.byref(info))
        if mask_times is not None:
            mask_times.append(time.perf_counter() - t0)
        if rc:
            raise RuntimeError(L.lvsa_last_error())
        if ev is not None:
            ev[0].record(stream)
        d_rp.copy_(h_rp[i], non_blocking=True)
        d_ci.copy_(h_ci[i], non_blocking=True)
        if ev is not None:
            ev[1].record(stream)
        rc = attention(d_rp.data_ptr(), d_ci.data_ptr(), sp)
        if ev is not None:
            ev[2].record(stream)
        if rc:
            raise RuntimeError(L.lvsa_last_error())

    for i in range(warmup):
        step(i, i)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    mask_times = []
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    g0.record(stream)
    for j in range(steps):
        step(warmup + j, j, ev[j], mask_times)
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = max(g0.elapsed_time(g1), wall * 1e3) / steps
    kms = [e[1].elapsed_time(e[2]) for e in ev]
    h2d = [e[0].elapsed_time(e[1]) for e in ev]
    flops = algorithmic_flops(w)
    k_avg = sum(kms) / len(kms)
    res = {
        "workload": w.name,
        "ms_per_step": ms_per_step,
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "kernel_ms": {"avg": k_avg, "median": statistics.median(kms), "p10": pct(kms, 0.1), "p90": pct(kms, 0.9)},
        "kernel_tflops": flops / (k_avg * 1e-3) / 1e12,
        "mask_build_us_median": statistics.median(mask_times) * 1e6,
        "mask_h2d_ms_median": statistics.median(h2d),
        "flops_per_step": flops,
        "path": "lvsa_attention_ws (key-norm pass + fixed softmax reference where the bound allows)" if workspace
                else "lvsa_attention (running-max softmax)",
    }
    if modes:
        # The same steps with no per-step host work: all masks built ahead of
        # time and copied once (outside the timed region), then (a) one launch
        # per step, (b) the whole step sequence replayed from a HIP graph.
        ms = L.lvsa_build_mask_steps(T, C, W, 0, steps).to(dev)
        torch.cuda.synchronize()

        def launch_all():
            sptr = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
            for j in range(steps):
                rc = attention(ms.row_ptr.data_ptr(), ms.col_idx[j].data_ptr(), sptr)
                if rc:
                    raise RuntimeError(L.lvsa_last_error())

        def timed(fn):
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            g0.record(stream)
            fn()
            g1.record(stream)
            torch.cuda.synchronize()
            return max(g0.elapsed_time(g1), (time.perf_counter() - w0) * 1e3) / steps

        launch_all()
        prebuilt_ms = timed(launch_all)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            launch_all()
        graph.replay()
        graph_ms = timed(graph.replay)
        res["step_modes_ms"] = {"host_mask_each_step": ms_per_step, "prebuilt_masks": prebuilt_ms,
                                "graph_replay": graph_ms, "kernel_only_avg": k_avg}
        del graph
    if dense:
        # Dense comparator: the same kernel with a C = T mask (one run of N keys).
        dm = L.lvsa_build_mask(T, max(T, 2), 1, 0).to(dev)
        dws = ws if workspace else None
        L.lvsa_attention(q, k, v, dm, out=out, workspace=dws)
        torch.cuda.synchronize()
        reps = 3
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            L.lvsa_attention(q, k, v, dm, out=out, workspace=dws)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / reps
        res["dense_ms_per_call"] = dense_ms
        res["speedup_vs_dense_kernel"] = dense_ms / k_avg
        res["ideal_speedup_T_over_C"] = T / min(C, T)
        # Outside reference (labelled as such): torch SDPA, flash backend, dense.
        sdpa_ms, why = sdpa_flash_dense_ms(q, k, v)
        res["outside_reference_torch_sdpa_flash_dense_ms"] = sdpa_ms
        if sdpa_ms is None:
            res["outside_reference_unavailable"] = why
        else:
            res["speedup_vs_torch_sdpa_flash_dense"] = sdpa_ms / k_avg
        torch.cuda.empty_cache()
        if T <= C:
            # At the training horizon the method is the dense model: the full
            # step (host mask + H2D + kernel) against the dense kernel alone.
            res["full_step_over_dense_kernel"] = ms_per_step / dense_ms
            if modes:
                res["graph_step_over_dense_kernel"] = res["step_modes_ms"]["graph_replay"] / dense_ms
    res["max_memory_allocated_gb"] = torch.cuda.max_memory_allocated(dev) / 1e9
    if keep_inputs:
        res["_inputs"] = (q, k, v)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan13b_6x")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-workspace", action="store_true",
                    help="time lvsa_attention (running-max softmax) instead of lvsa_attention_ws")
    ap.add_argument("--no-step-modes", action="store_true",
                    help="skip the prebuilt-mask and graph-replay timings of the same steps")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run a plain 1 GiB device-to-device copy first (reference for HBM byte counters)")
    ap.add_argument("--sweep", action="store_true", help="time every workload (table on stderr)")
    ap.add_argument("--sweep-out", default=None, help="also write the sweep table (markdown) here")
    ap.add_argument("--library", default=None, help="time this build of liblvsa.so instead of the package's (A/B)")
    ap.add_argument("--no-peak-probe", action="store_true", help="skip the matrix-core peak microbenchmark")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              f"multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_lvsa_amd as L
    from block_sparse_attention_lvsa_amd.synth import WORKLOADS

    if args.library:
        L.LIB_PATH = os.path.abspath(args.library)
    if args.sweep:
        lines = ["| workload | B·H, T×P, C/W | ms/call (median) | effective TFLOP/s | % of 2.5 PF | dense (C=T) ms | "
                 "speedup | ideal T/C | torch SDPA flash, dense ms (outside reference) | "
                 "ms/step: host mask each step / prebuilt / graph | "
                 "full step / dense (T≤C): host mask / graph | peak mem GB |",
                 "|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for name in SWEEP:
            w = WORKLOADS[name]
            r = run_workload(w, args.steps, args.warmup, dense=True, workspace=not args.no_workspace)
            log(json.dumps(r))
            ov = r.get("full_step_over_dense_kernel")
            og = r.get("graph_step_over_dense_kernel")
            sm = r["step_modes_ms"]
            lines.append(f"| {name} | {w.B * w.H}, {w.T}×{w.P}, {w.C}/{w.W} | {r['kernel_ms']['median']:.3f} | "
                         f"{r['kernel_tflops']:.1f} | {100 * r['kernel_tflops'] / PEAK_BF16_TFLOPS:.1f} | "
                         f"{r['dense_ms_per_call']:.3f} | {r['speedup_vs_dense_kernel']:.2f} | "
                         f"{r['ideal_speedup_T_over_C']:.2f} | "
                         f"{'%.1f' % r['outside_reference_torch_sdpa_flash_dense_ms'] if r.get('outside_reference_torch_sdpa_flash_dense_ms') else 'n/a'} | "
                         f"{sm['host_mask_each_step']:.3f} / "
                         f"{sm['prebuilt_masks']:.3f} / {sm['graph_replay']:.3f} | "
                         f"{'%.3f / %.3f' % (ov, og) if ov else '—'} | {r['max_memory_allocated_gb']:.1f} |")
            torch.cuda.empty_cache()
        table = "\n".join(lines)
        log(table)
        if args.sweep_out:
            with open(args.sweep_out, "w") as f:
                f.write(table + "\n")
        return

    w = WORKLOADS[args.workload]
    log(f"workload {w}")
    r = run_workload(w, args.steps, args.warmup, dense=not args.no_dense, calib_copy=args.calib_copy,
                     keep_inputs=not args.no_cpu_baseline, modes=not args.no_step_modes,
                     workspace=not args.no_workspace)
    log(f"step: {r['ms_per_step']:.3f} ms  kernel avg {r['kernel_ms']['avg']:.3f} ms (median "
        f"{r['kernel_ms']['median']:.3f}, p10 {r['kernel_ms']['p10']:.3f}, p90 {r['kernel_ms']['p90']:.3f})  "
        f"{r['value']:.1f} TFLOP/s effective, kernel {r['kernel_tflops']:.1f} TFLOP/s")
    log(f"host mask build: median {r['mask_build_us_median']:.1f} us/step; mask H2D median "
        f"{r['mask_h2d_ms_median'] * 1e3:.1f} us/step")
    if "step_modes_ms" in r:
        sm = r["step_modes_ms"]
        log(f"ms/step: host mask each step {sm['host_mask_each_step']:.3f}, masks prebuilt {sm['prebuilt_masks']:.3f}, "
            f"graph replay {sm['graph_replay']:.3f} (kernel alone {sm['kernel_only_avg']:.3f})")
    if "dense_ms_per_call" in r:
        log(f"dense (C=T) kernel: {r['dense_ms_per_call']:.3f} ms -> speedup {r['speedup_vs_dense_kernel']:.2f}x "
            f"(ideal {r['ideal_speedup_T_over_C']:.2f}x)")
        if r.get("outside_reference_torch_sdpa_flash_dense_ms"):
            log(f"outside reference, torch SDPA (flash backend, dense): "
                f"{r['outside_reference_torch_sdpa_flash_dense_ms']:.2f} ms -> LVSA kernel "
                f"{r['speedup_vs_torch_sdpa_flash_dense']:.2f}x faster")

    achieved = r["kernel_tflops"]
    k_ms = r["kernel_ms"]["avg"]
    alg_bytes = 8.0 * w.B * w.H * w.N * w.D  # Q, K, V read once, O written once (bf16)
    span = w.P >= 384
    kname = ("lvsa_attn_span<%d>" if span else "lvsa_attn_frame<%d>") % w.D
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
            "kernel": kname + (" (+ lvsa_key_norms and the merge of split items, in the timed call)" if not args.no_workspace
                               else ""),
            "kernel_ms_avg": round(k_ms, 4),
            "achieved_is": "algorithmic FLOPs 4·B·H·T·min(C,T)·P²·d per call / HIP-event time of the whole call"}
    if not args.no_peak_probe:
        ptf, pmhz = mfma_peak_probe()
        if ptf:
            log(f"measured bf16 MFMA peak: {ptf:.0f} TFLOP/s at {pmhz:.0f} MHz (vendor {PEAK_BF16_TFLOPS:.0f})")
            roof["peak_measured"] = {"value": round(ptf, 1), "unit": "TFLOP/s", "clock_mhz": round(pmhz),
                                     "what": "libmfma_peak.so: independent v_mfma_f32_32x32x16_bf16 chains on "
                                             "every SIMD at 3 waves/SIMD, no memory traffic, after a warm-up"}
            roof["frac_of_measured_peak"] = round(achieved / ptf, 4)
    tr = measured_traffic(w)
    if tr:
        b = tr["bytes_per_launch"]
        roof["traffic"] = b
        roof["traffic_what"] = ("L2-to-fabric bytes per launch of the attention kernel (rocprofv3 FETCH_SIZE + "
                                "WRITE_SIZE, scaled by a plain 1 GiB copy): what left the L2s for the memory "
                                "side, served by the MALL or by HBM (no counter here tells the two apart)")
        roof["traffic_spread"] = tr.get("spread")
        roof["traffic_over_algorithmic"] = round(b / alg_bytes, 2)
        roof["traffic_gbs"] = round(b / (k_ms * 1e-3) / 1e9, 1)
        roof["traffic_frac_of_hbm_peak"] = round(b / (k_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        roof["traffic_profile"] = tr.get("profile")

    cpu = None
    if not args.no_cpu_baseline:
        q, k, v = r.pop("_inputs")
        cpu = cpu_baseline(w, q, k, v, args.cpu_budget)
        log(f"cpu oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads ({cpu['sample']})")

    extra = {key: (round(val, 4) if isinstance(val, float) else val) for key, val in r.items()
             if key in ("dense_ms_per_call", "speedup_vs_dense_kernel", "ideal_speedup_T_over_C",
                        "full_step_over_dense_kernel", "graph_step_over_dense_kernel",
                        "outside_reference_torch_sdpa_flash_dense_ms", "speedup_vs_torch_sdpa_flash_dense",
                        "outside_reference_unavailable", "mask_build_us_median",
                        "mask_h2d_ms_median", "max_memory_allocated_gb", "path")}
    if "step_modes_ms" in r:
        extra["step_modes_ms"] = {key: round(val, 4) for key, val in r["step_modes_ms"].items()}
    extra["kernel_ms"] = {key: round(val, 4) for key, val in r["kernel_ms"].items()}
    rec = {
        "metric": METRIC,
        "value": round(r["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "P": w.P, "d": w.D, "C": w.C, "W": w.W,
                   "tokens": w.N, "rotation": "mod_tper", "denoising_steps": f"0..{args.steps - 1}",
                   "flops_per_step": r["flops_per_step"], "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
