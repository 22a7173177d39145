#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input: the fused
forward (O and LSE) followed by the recompute backward (D, dK/dV, dQ) at
B=2, H=12, N=8192, d=64, fp16, non-causal (the A100 table's shape at its
largest N).  Inputs are resident in HBM before timing starts.

Credited flops (the metric's convention): forward 4*B*H*N^2*d, backward 2.5x
that (both halved for causal).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F16_TFLOPS = 2500.0  # MI355X published dense fp16/bf16 MFMA peak
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic_B2H12N8192d64_f16.json")
# every HIP source and header of the library (a stored counter summary counts
# only for the sources it was taken on)
KERNEL_SOURCES = sorted(os.path.join("io_aware_exact_08_amd", "csrc", f)
                        for f in os.listdir(os.path.join(ROOT, "io_aware_exact_08_amd", "csrc"))
                        if f.endswith((".hip", ".hpp")))
# host worker processes for the CPU oracle: at most the host cores a single-GPU node gives each GPU
MAX_CPU_WORKERS = 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The clocks take roughly 0.2 s of sustained load to settle: whatever
    # --warmup says, warm-up runs at least --warmup-s seconds of wall time
    # (outside the timed region), so the timed steps see steady state.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--warmup-s", type=float, default=0.25)
    ap.add_argument("--N", type=int, default=8192)
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time only the forward (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="worker processes for the CPU oracle (0: the usable cores, at most "
                         f"{MAX_CPU_WORKERS})")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB before the "
                         "timed loop (reference dispatch for HBM byte counters)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the untimed-by-the-step per-configuration report")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 counter_collection.csv files (a "
                         "FETCH_SIZE run and a WRITE_SIZE run of this script with "
                         "--copy-calibration-mib) into the per-kernel HBM traffic summary")
    ap.add_argument("--traffic-out", default=PROFILE_TRAFFIC)
    return ap.parse_args()


def sources_digest():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel):
    """HBM bytes per launch of `kernel` (fetch + write, copy-calibrated) from the
    committed rocprofv3 counter summary, or None when it is missing or was
    taken on different kernel sources."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256_16") != sources_digest():
        return None
    return rec.get("hbm_bytes_per_launch", {}).get(kernel)


KERNEL_KEYS = ("fwd_kernel", "bwd_pre_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel")


def _counter_rows(path, counter):
    import csv
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def traffic_summary(fetch_csv, write_csv, out_path, calib_mib):
    """Copy-calibrated HBM bytes per launch, per kernel of the step.

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  Each is scaled by
    (bytes a plain copy of `calib_mib` MiB moves) / (what the same counter read
    for that copy's dispatch), the copy being the largest-reading dispatch whose
    kernel name contains "copy"."""
    calib_kib = calib_mib * 1024.0
    rec = {"sources_sha256_16": sources_digest(), "copy_calibration_mib": calib_mib,
           "commands": [
               f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- python3 bench.py "
               f"--no-cpu-baseline --steps 3 --warmup 1 --copy-calibration-mib {calib_mib}"
               for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
               f"python3 bench.py --traffic-summary {fetch_csv} {write_csv}"],
           "counter_kib_per_launch": {}, "hbm_bytes_per_launch": {}}
    per = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, name)
        copies = [v for kn, v in rows if "copy" in kn.lower()]
        if not copies:
            raise SystemExit(f"{path}: no copy dispatch to calibrate {name} against")
        factor = calib_kib / max(copies)
        rec[f"{name}_factor"] = round(factor, 4)
        for key in KERNEL_KEYS:
            vals = [v for kn, v in rows if f"::{key}<" in kn]
            if vals:
                kib = sum(vals) / len(vals)
                rec["counter_kib_per_launch"].setdefault(key, {})[name] = round(kib, 1)
                per.setdefault(key, 0.0)
                per[key] += kib * 1024.0 * factor
    rec["hbm_bytes_per_launch"] = {k_: int(round(v)) for k_, v in per.items()}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def config_sweep(fa, si, torch, np, dev):
    """Event-timed forward (and backward where the configuration has one) of the
    other synthetic configurations, as graph replays (see `timed`); reported
    beside the headline step, outside its timed region."""
    out = {}

    def tensors(w):
        dt = torch.float16 if w.fmt == "f16" else torch.bfloat16
        conv = lambda b: torch.from_numpy(b.view(np.int16)).view(dt).to(dev)  # noqa: E731
        return conv(w.q), conv(w.k), conv(w.v), (conv(w.do) if w.do is not None else None)

    how = {}

    def timed(fn, reps, outs=()):
        # the clocks need about 0.2 s of sustained load to settle
        t0 = time.perf_counter()
        n = 0
        while n < 3 or time.perf_counter() - t0 < 0.25:
            fn()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # The calls go through the Python binding, whose host time per call
        # (several microseconds) would show in the small shapes' kernel time:
        # time replays of a captured graph of `reps` calls instead (the same
        # launches, no host work between them).  Eager calls if capture fails
        # or a replay's outputs differ from the eager call's.
        ref = [t.clone() for t in outs]
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            replays = 3
            e0.record()
            for _ in range(replays):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            if all(torch.equal(t, r) for t, r in zip(outs, ref)):
                how["timing"] = "graph"
                return e0.elapsed_time(e1) / (reps * replays)
        except Exception:
            torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        how["timing"] = "eager"
        return e0.elapsed_time(e1) / reps

    def run(name, w, out_f32=False, bwd=False, reps=20, splits=None, bias_bits=None):
        q, k, v, do = tensors(w)
        B, H, N, d = w.shape
        fl = 4.0 * B * H * N * N * d * (0.5 if w.causal else 1.0)
        o, lse = fa.flash_attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out_f32=out_f32)
        if bias_bits is not None:
            dt = torch.float16 if w.fmt == "f16" else torch.bfloat16
            bias = torch.from_numpy(bias_bits.view(np.int16)).view(dt).to(dev)
            ms = timed(lambda: fa.flash_attn_fwd_bias(q, k, v, bias, causal=w.causal, scale=w.scale,
                                                      out_f32=out_f32, o=o, lse=lse), reps, (o, lse))
            rec = {"shape": [B, H, N, d], "dtype": w.fmt, "causal": w.causal, "bias": list(bias.shape),
                   "timing": how.get("timing"),
                   "fwd_ms": round(ms, 4), "fwd_tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                   "fwd_frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)}
            if bwd:
                ws = torch.empty(fa.workspace_bytes(B, H, N, d) // 4 + 4, dtype=torch.float32,
                                 device=dev)
                dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                ms_b = timed(lambda: fa.flash_attn_bwd_bias(q, k, v, bias, o, lse, do,
                                                            causal=w.causal, scale=w.scale, dq=dq,
                                                            dk=dk, dv=dv, workspace=ws), reps, (dq, dk, dv))
                rec["bwd_ms"] = round(ms_b, 4)
                rec["bwd_tflops_credited"] = round(2.5 * fl / (ms_b * 1e-3) / 1e12, 1)
                # executed work: dK/dV 8 and dQ 6 BHN^2d products = 3.5x the forward's
                rec["bwd_frac_of_peak"] = round(3.5 * fl / (ms_b * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)
            out[name] = rec
            return
        if splits is None:
            ms = timed(lambda: fa.flash_attn_fwd(q, k, v, causal=w.causal, scale=w.scale,
                                                 out_f32=out_f32, o=o, lse=lse), reps, (o, lse))
        else:
            # splits == 0: the library's automatic plan
            ws = torch.empty(max(fa._lib.flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, splits) // 4, 1),
                             dtype=torch.float32, device=dev)
            ms = timed(lambda: fa.flash_attn_fwd_splitkv(q, k, v, causal=w.causal, scale=w.scale,
                                                         out_f32=out_f32, num_splits=splits,
                                                         o=o, lse=lse, workspace=ws), reps, (o, lse))
        rec = {"shape": [B, H, N, d], "dtype": w.fmt, "causal": w.causal, "timing": how.get("timing"),
               "fwd_ms": round(ms, 4), "fwd_tflops": round(fl / (ms * 1e-3) / 1e12, 1),
               "fwd_frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)}
        if splits is not None:
            rec["splits"] = splits if splits else "automatic"
        if bwd:
            ws = torch.empty(fa.workspace_bytes(B, H, N, d) // 4 + 4, dtype=torch.float32,
                             device=dev)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ms_b = timed(lambda: fa.flash_attn_bwd(q, k, v, o, lse, do, causal=w.causal,
                                                   scale=w.scale, dq=dq, dk=dk, dv=dv,
                                                   workspace=ws), reps, (dq, dk, dv))
            rec["bwd_ms"] = round(ms_b, 4)
            rec["bwd_tflops_credited"] = round(2.5 * fl / (ms_b * 1e-3) / 1e12, 1)
            rec["bwd_frac_of_peak"] = round(3.5 * fl / (ms_b * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)
        out[name] = rec

    for n in (1024, 2048, 4096, 8192):
        run(f"fwd_B2H12N{n}d64_f16", si.a100_sweep(n))
        # the same through the split-KV entry point's automatic plan (it splits
        # the key range only where rounds of workgroups would be partly idle)
        run(f"fwd_splitkv_auto_B2H12N{n}d64_f16", si.a100_sweep(n), splits=0)
    run("fwd_causal_B2H16N4096d128_bf16_spiked_f32out", si.spiked_causal(), out_f32=True)
    run("fwdbwd_causal_B1H8N32768d64_bf16", si.long_causal(with_do=True), bwd=True, reps=3)
    few = si.random_case(1, 4, 8192, 128, "bf16", False, seed=11)
    run("fwd_B1H4N8192d128_bf16", few, out_f32=True)
    run("fwd_splitkv_B1H4N8192d128_bf16", few, out_f32=True, splits=0)
    run("fwdbwd_B2H12N4096d64_f16", si.fwd_bwd(False), bwd=True)
    run("fwdbwd_bias_B2H12N4096d64_f16", si.fwd_bwd(False), bwd=True,
        bias_bits=si.attn_bias((2, 12, 4096, 4096), "f16", [5, 4096], "random", hole=0.1))
    run("fwdbwd_causal_B2H12N4096d64_f16", si.fwd_bwd(True), bwd=True)
    # d=128 backward at the spiked workload's shape (without the spikes)
    run("fwdbwd_causal_B2H16N4096d128_bf16",
        si.random_case(2, 16, 4096, 128, "bf16", True, seed=3, with_do=True), bwd=True)
    run("fwdbwd_B2H12N4096d128_f16", si.random_case(2, 12, 4096, 128, "f16", False, seed=4,
                                                      with_do=True), bwd=True)
    # ragged sequence lengths around the A100 shape's largest N
    for n in (8000, 8200):
        run(f"fwdbwd_B2H12N{n}d64_f16", si.random_case(2, 12, n, 64, "f16", False, seed=n,
                                                        with_do=True), bwd=True)
        run(f"fwd_splitkv_auto_B2H12N{n}d64_f16", si.random_case(2, 12, n, 64, "f16", False, seed=n),
            splits=0)
    run("fwdbwd_B2H8N4096d256_f16", si.random_case(2, 8, 4096, 256, "f16", False, seed=257,
                                                     with_do=True), bwd=True)
    run("fwdbwd_causal_B2H8N4096d256_bf16_f32out",
        si.random_case(2, 8, 4096, 256, "bf16", True, seed=257, with_do=True), out_f32=True, bwd=True)
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, timed on the host cores
# ---------------------------------------------------------------------------
def _cpu_worker_init():
    # one BLAS thread per worker: the pool, not BLAS, spreads the heads
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_job(job):
    """One head (or a head's sampled rows) of the oracle, in a worker process."""
    import oracle
    kind, a = job
    if kind == "fwd":
        oracle.forward_head(*a)
    elif kind == "fwdbwd":
        q, k, v, do, scale, causal = a
        oracle.forward_head(q, k, v, scale, causal)
        oracle.backward_head(q, k, v, do, scale, causal)
    else:
        oracle.forward_rows(*a)
    return 0


def _head_jobs(w, kind):
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    do = w.f64("do") if kind == "fwdbwd" else None
    jobs = []
    for b in range(w.B):
        for h in range(w.H):
            if kind == "fwd":
                jobs.append(("fwd", (q[b, h], k[b, h], v[b, h], w.scale, w.causal)))
            else:
                jobs.append(("fwdbwd", (q[b, h], k[b, h], v[b, h], do[b, h], w.scale, w.causal)))
    return jobs


def cpu_baseline(workers=0):
    """The fp64 oracle as it stands (never tuned for timing), spread over a pool of
    worker processes with one BLAS thread each, on every synthetic configuration:
    the forward of the small, A100-shape, spiked and long causal workloads, and
    forward+backward of the fwd+bwd workload and of the benchmarked step's own
    workload (which gives `value`).  Credited flops as for the GPU (forward
    4*N^2*d per head, backward 2.5x that, halved for causal).  Runs before the
    GPU is touched, so the pool can fork."""
    import multiprocessing as mp

    import numpy as np
    from synth import inputs as si

    usable = len(os.sched_getaffinity(0))
    k = workers or min(MAX_CPU_WORKERS, usable)
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    per = {}
    with mp.get_context("fork").Pool(k, initializer=_cpu_worker_init) as pool:
        def timed(jobs):
            t0 = time.perf_counter()
            pool.map(_oracle_job, jobs, chunksize=1)
            return time.perf_counter() - t0

        def heads(name, w, kind):
            dt = timed(_head_jobs(w, kind))
            fl = 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
            fl *= 3.5 if kind == "fwdbwd" else 1.0
            per[name] = {"seconds": round(dt, 3), "tflops": round(fl / dt / 1e12, 5),
                         "sample": f"all {w.B * w.H} heads, {'forward+backward' if kind == 'fwdbwd' else 'forward'}"}
            return dt, fl

        heads("fwd_B1H4N128d64_f16", si.tiny_fwd(), "fwd")
        for n in (1024, 2048, 4096, 8192):
            heads(f"fwd_B2H12N{n}d64_f16", si.a100_sweep(n), "fwd")
        heads("fwd_causal_B2H16N4096d128_bf16_spiked", si.spiked_causal(), "fwd")
        # long causal: the sampled rows, then every row at N=2048
        w = si.long_causal()
        pairs = si.long_causal_sample_rows(w.H, w.N)
        q, kk, v = w.f64("q"), w.f64("k"), w.f64("v")
        jobs = []
        for h in sorted({int(h) for h, _ in pairs}):
            rows = [(0, 0, int(i)) for hh, i in pairs if hh == h]
            jobs.append(("rows", (q[:, h:h + 1], kk[:, h:h + 1], v[:, h:h + 1], rows, w.scale, True)))
        dt = timed(jobs)
        fl_rows = sum(4.0 * (int(i) + 1) * w.d for _, i in pairs)
        full = 4.0 * w.H * w.N * w.N * w.d * 0.5
        per["fwd_causal_B1H8N32768d64_bf16_rows"] = {
            "seconds": round(dt, 3), "rows": int(len(pairs)), "rows_per_s": round(len(pairs) / dt, 1),
            "tflops": round(fl_rows / dt / 1e12, 5),
            "full_forward_s_extrapolated": round(full / (fl_rows / dt), 1),
            "sample": f"{len(pairs)} sampled query rows over 8 heads at N=32768 (the full "
                      "forward's time is extrapolated from their flop rate)"}
        heads("fwd_causal_B1H8N2048d64_bf16", si.long_causal(N=2048), "fwd")
        heads("fwdbwd_B2H12N4096d64_f16", si.fwd_bwd(False), "fwdbwd")
        heads("fwdbwd_causal_B2H12N4096d64_f16", si.fwd_bwd(True), "fwdbwd")
        dt, fl = heads("fwdbwd_B2H12N8192d64_f16", si.a100_sweep(8192, with_do=True), "fwdbwd")
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": k, "kind": "oracle",
            "sample": f"the benchmarked step's workload (B2 H12 N8192 d64 fp16), all 24 heads, "
                      f"forward+backward in float64 ({dt:.1f} s), credited flops as for the GPU",
            "workers": k, "usable_cores": usable, "blas_threads_per_worker": 1,
            "blas_threads_default": blas, "per_config": per}


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.traffic_out,
                        args.copy_calibration_mib or 256)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the path shards by heads with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    # The CPU oracle runs first, before anything touches the GPU, so that its
    # worker pool can fork.
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_workers)

    import numpy as np
    import torch

    import io_aware_exact_08_amd as fa
    from synth import inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = si.a100_sweep(args.N, with_do=True)
    if args.causal:
        w.causal = True

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(dev)

    q, k, v, do = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.do)
    B, H, N, d = w.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.workspace_bytes(B, H, N, d) // 4 + 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    # One step: forward, then the backward's three stages (exactly what
    # flash_attn_bwd enqueues), with events between the kernels.
    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        fa.flash_attn_fwd(q, k, v, causal=w.causal, scale=w.scale, o=o, lse=lse)
        mark(1)
        if not args.fwd_only:
            fa.flash_attn_bwd_preprocess(o, lse, do, ws)
            mark(2)
            fa.flash_attn_bwd_dkdv(q, k, v, do, ws, causal=w.causal, scale=w.scale, dk=dk, dv=dv)
            mark(3)
            fa.flash_attn_bwd_dq(q, k, v, do, ws, causal=w.causal, scale=w.scale, dq=dq)
            mark(4)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Warm-up: at least --warmup steps and at least --warmup-s seconds of wall
    # time (the clocks settle after about 0.2 s of sustained load).
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_s:
        step()
        n_warm += 1
        if n_warm % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def avg_ms(i, j):
        return float(np.mean([e[i].elapsed_time(e[j]) for e in events]))

    last = 1 if args.fwd_only else 4
    per_step = np.array([e[0].elapsed_time(e[last]) for e in events])
    q25, med, q75 = (float(x) for x in np.percentile(per_step, [25, 50, 75]))

    ms_per_step = wall * 1e3 / args.steps
    causal_f = 0.5 if w.causal else 1.0
    unit = B * H * N * N * d * causal_f  # N^2 d per head, summed over heads
    fwd_flops = 4.0 * unit
    bwd_flops = 2.5 * fwd_flops  # the metric's credit for the backward
    step_flops = fwd_flops + (0.0 if args.fwd_only else bwd_flops)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    fwd_avg = avg_ms(0, 1)
    fwd_tflops = fwd_flops / (fwd_avg * 1e-3) / 1e12
    res = {
        "metric": "attention fwd(+bwd) TFLOP/s on 1 MI355X and % of MFMA peak, B=2 H=12 d=64",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": ("forward" if args.fwd_only else "forward+backward")
                        + f" exact attention B={B} H={H} N={N} d={d} fp16 "
                        + ("causal" if w.causal else "non-causal"),
            "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
            "accumulate": "f32", "parallelism": "single GPU",
        },
        "frac_of_peak": round(value / PEAK_MFMA_F16_TFLOPS, 4),
        "step_ms_events": {"median": round(med, 4), "q25": round(q25, 4), "q75": round(q75, 4),
                           "iqr": round(q75 - q25, 4), "mean": round(float(per_step.mean()), 4)},
        "tflops_at_median_step": round(step_flops / (med * 1e-3) / 1e12, 2),
        "warmup_done": {"steps": n_warm, "seconds": round(warm_s, 3)},
        "fwd": {"ms": round(fwd_avg, 4), "tflops": round(fwd_tflops, 2),
                "frac_of_peak": round(fwd_tflops / PEAK_MFMA_F16_TFLOPS, 4)},
    }
    # Per-kernel event timings; algorithmic flops per launch are 2*N^2*d per
    # head for every product the kernel computes (forward 2, dK/dV 4, dQ 3).
    kernels = {"fwd_kernel": (fwd_avg, 4.0 * unit)}
    if not args.fwd_only:
        pre_ms, dkdv_ms, dq_ms = avg_ms(1, 2), avg_ms(2, 3), avg_ms(3, 4)
        bwd_avg = pre_ms + dkdv_ms + dq_ms
        res["bwd"] = {"ms": round(bwd_avg, 4),
                      "tflops_credited": round(bwd_flops / (bwd_avg * 1e-3) / 1e12, 2),
                      "kernels": "bwd_pre + bwd_dkdv + bwd_dq"}
        kernels.update({"bwd_dkdv_kernel": (dkdv_ms, 8.0 * unit),
                        "bwd_dq_kernel": (dq_ms, 6.0 * unit)})
        pre_bytes = B * H * N * (2 * d * 2 + 4 + 8)  # read O, dO, LSE; write D, LSE2
        res["bwd_pre"] = {"ms": round(pre_ms, 4),
                          "GB_per_s": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1)}
    res["kernels"] = {k_: {"ms": round(t, 4), "algorithmic_tflops": round(fl / (t * 1e-3) / 1e12, 2),
                           "frac_of_peak": round(fl / (t * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)}
                      for k_, (t, fl) in kernels.items()}
    # Roofline of the dominant (longest) kernel.
    dom = max(kernels, key=lambda k_: kernels[k_][0])
    t_dom, fl_dom = kernels[dom]
    ach = fl_dom / (t_dom * 1e-3) / 1e12
    res["roofline"] = {
        "kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
        "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(ach / PEAK_MFMA_F16_TFLOPS, 4),
        "traffic": traffic_from_profile(dom),
    }
    if not args.no_sweep:
        res["configs"] = config_sweep(fa, si, torch, np, dev)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
