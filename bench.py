#!/usr/bin/env python3
"""Benchmark: chunkwise gated linear attention forward on one MI355X.

Default workload: B=8, H=16, T=2048, K=V=128, bf16 q/k/v, fp32 gates, chunk 64,
final state stored (synthetic seeded inputs, recipe in gla_inputs.py).

A step is one full forward (every kernel of the path) over the whole batch,
with inputs resident in device memory.  Untimed steps for --settle-ms (the GPU
clock ramps up over the first tens of milliseconds of load), W untimed warmup
steps, then exactly K timed steps between two device synchronisations; one JSON
line is printed.

Also reported:
  roofline      the dominant kernel's algorithmic bytes per launch divided by its
                average launch time, measured with HIP events on the launch stream
                inside the timed region, against the 8 TB/s HBM peak; `traffic`
                is the HBM bytes per launch measured by rocprofv3 counters for the
                current kernel source (null when no matching measurement exists).
  cpu_baseline  the fp64 CPU oracle (test infrastructure) on the host cores, on the
                whole workload, in tokens/s.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


import gla_inputs as gi  # noqa: E402

METRIC = "GLA chunked fwd tokens/s + TFLOP/s, fraction of MFMA/HBM roofline (1 GPU)"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
KERNEL_SRCS = [os.path.join(ROOT, "chunkwise_gated_linear_amd", "csrc", f)
               for f in ("gla_kernels.hip", "gla_walk_bf16.hip", "gla_device.h", "gla_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def kernel_source_hash() -> str:
    """Hash of every device source: counters measured on other kernel code are not reused."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(w, n_tokens, n_seqs):
    """Bytes (inputs read once + outputs written once) and flops of the method."""
    e = 2 if w.dtype == "bf16" else 4
    H, K, V = w.H, w.K, w.V
    th = n_tokens * H
    nbytes = th * (2 * K * e + V * e + 4 * K) + th * V * e + 4 * n_seqs * H * K * V * (int(w.h0) + int(w.ht))
    flops = th * (4 * K * V + (64 + 1) * (K + V))
    return nbytes, flops


def describe(w, lengths):
    if w.varlen:
        return (f"varlen {w.n_seqs} seqs lengths U[{w.len_lo},{w.len_hi}] total {sum(lengths)}, "
                f"H={w.H} K={w.K} V={w.V} {w.dtype}, chunk {w.chunk}")
    return (f"B={w.B},H={w.H},T={w.T},K={w.K},V={w.V} {w.dtype} q/k/v, g fp32 logsigmoid(N(0,1))/16, "
            f"chunk {w.chunk}, h0={'yes' if w.h0 else 'no'}, ht={'stored' if w.ht else 'no'}")


def load_traffic(workload: str):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def _counter_per_dispatch(run_dir, counter, name_filter=None):
    """Mean per-dispatch value of `counter` in a rocprofv3 --pmc CSV run directory,
    for the kernel matching name_filter (default: the kernel with the largest value)."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")))
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    per_kernel = {}
    for (name, _), v in vals.items():
        per_kernel.setdefault(name, []).append(v)
    if not per_kernel:
        raise SystemExit(f"no {counter} rows under {run_dir}")
    if name_filter is not None:
        names = [n for n in per_kernel if name_filter in n]
        if not names:
            raise SystemExit(f"no kernel matching {name_filter!r} under {run_dir}")
    else:
        names = list(per_kernel)
    means = {n: sum(per_kernel[n]) / len(per_kernel[n]) for n in names}
    best = max(means, key=means.get)
    return best, means[best]


def record_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dominant kernel by what the
    same counters read for a plain device copy of known size, and store the HBM bytes per
    launch in profiles/traffic.json for the current device sources."""
    copy_bytes = 512 << 20
    _, cf = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE")
    _, cw = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE")
    f_factor, w_factor = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    kname, kf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", "gla_chunk_output")
    _, kw = _counter_per_dispatch(write_dir, "WRITE_SIZE", "gla_chunk_output")
    fetch_b, write_b = kf * 1024.0 * f_factor, kw * 1024.0 * w_factor
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[workload] = {
        "kernel": kname.rsplit("(", 1)[0],
        "bytes_per_launch": fetch_b + write_b,
        "fetch_bytes": fetch_b, "write_bytes": write_b,
        "fetch_kib_counter": kf, "write_kib_counter": kw,
        "copy_fetch_factor": f_factor, "copy_write_factor": w_factor,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(table[workload], indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the W warmup steps, run untimed steps for this long so the GPU "
                         "reaches its sustained clock (short runs otherwise measure the ramp)")
    ap.add_argument("--workload", default="c2048", choices=sorted(gi.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single", type=int, default=21,
                    help="launches timed one by one after the timed steps, warm and with L2/MALL evicted")
    ap.add_argument("--segment-chunks", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the forward, run a plain device copy of a known size "
                         "(used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="(no GPU) store HBM bytes per launch of --workload from rocprofv3 --pmc runs of "
                         "FETCH_SIZE and WRITE_SIZE on this benchmark and on --copy-calibration")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build is a single-GPU kernel library; run it with --gpus 1 "
              "(multi-GPU sharding is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunkwise_gated_linear_amd as gla

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    gla.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        nbytes = 512 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                          "launches": args.steps}), flush=True)
        return

    w = gi.WORKLOADS[args.workload]
    d = gi.make_inputs(w)
    lengths = d.get("lengths")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(d[x]).to(tdt).to(dev) for x in ("q", "k", "v"))
    g = torch.from_numpy(d["g"]).to(dev)
    h0 = None if d["h0"] is None else torch.from_numpy(d["h0"]).to(dev)
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(d["cu_seqlens"]).to(dev)
    n_tokens = int(q.shape[0] * q.shape[1])
    n_seqs = w.n_seqs if w.varlen else w.B
    call = gla.GlaCall(q, k, v, g, h0=h0, cu_seqlens=cu, output_final_state=w.ht,
                       segment_chunks=args.segment_chunks)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            call(sptr)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        call(sptr)
    torch.cuda.synchronize()

    # One event pair on the launch stream brackets the K back-to-back steps; the
    # average launch duration is their span / K (per-step event records would
    # add their own gaps between launches).
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call(sptr)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = ev0.elapsed_time(ev1) / args.steps

    # After the timed steps (not part of `value`): single launches, each between
    # its own event pair: back to back (warm); cold, after writing one 512 MiB
    # buffer and reading another, so that L2 and the MALL hold neither inputs nor
    # dirty lines; and after the write alone, whose dirty lines are written back
    # while the launch runs.  Then the bandwidth of a plain 512 MiB device copy
    # on this GPU, as a measured counterpart of the HBM peak.
    def single_launches(n, prep=None):
        ts = []
        for _ in range(n):
            if prep is not None:
                prep()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(sptr)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        return ts[len(ts) // 2], ts[0]
    launch_us = None
    copy_gbs = None
    if args.single > 0:
        warm_med, warm_min = single_launches(args.single)
        wbuf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        rbuf = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        cold_med, cold_min = single_launches(args.single, lambda: (wbuf.fill_(1), rbuf.sum(dtype=torch.int64)))
        dirty_med, _ = single_launches(args.single, lambda: wbuf.fill_(1))
        del wbuf, rbuf
        launch_us = {"warm_median": warm_med, "warm_min": warm_min, "cold_median": cold_med,
                     "cold_min": cold_min, "after_write_median": dirty_med, "launches": args.single}
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbs = 2 * src.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del src, dst

    nbytes, flops = algorithmic(w, n_tokens, n_seqs)
    tokens_per_s = n_tokens / (ms_per_step * 1e-3)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved_gbs = nbytes / (launch_ms * 1e-3) / 1e9
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_MFMA_PEAK_TFLOPS * 1e12))
    traffic = load_traffic(args.workload)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        threads = len(os.sched_getaffinity(0))
        # the whole workload, repeated until about 10 s of wall time (bounded at 100 runs)
        runs, c0 = 0, time.perf_counter()
        while True:
            oracle.gla_reference(d["q"], d["k"], d["v"], d["g"], h0=d["h0"], cu_seqlens=d["cu_seqlens"],
                                 output_final_state=w.ht, threads=threads)
            runs += 1
            if time.perf_counter() - c0 >= 10.0 or runs >= 100:
                break
        c1 = time.perf_counter()
        cpu = {"value": runs * n_tokens / (c1 - c0), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole workload ({n_tokens} tokens x {w.H} heads), fp64 token recurrence, "
                         f"{runs} runs in {c1 - c0:.2f} s on {cpu_model()}"}

    segmented = call.ws_bytes > 0
    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": describe(w, lengths), "tokens": n_tokens, "heads": w.H,
                   "segmented_state_scan": segmented},
        "tflops_algorithmic": tflops,
        "roofline_time_us": t_roof * 1e6,
        "roofline": {
            "bound": "hbm",
            "kernel": "gla_chunk_output" if not segmented else "gla_fwd (chunk_local + state_scan + chunk_output)",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": nbytes,
            "launch_ms_avg": launch_ms,
            "measured_copy_GBs": copy_gbs,
            "frac_of_measured_copy": None if copy_gbs is None else achieved_gbs / copy_gbs,
        },
        "single_launch_us": launch_us,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
