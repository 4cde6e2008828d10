#!/usr/bin/env python3
"""Benchmark: chunkwise gated linear attention forward on one MI355X.

Default workload ("long"): B=1, H=32, T=65536, K=V=128, bf16 q/k/v, fp32 gates
logsigmoid(N(0,1))/16, chunk 64, final state stored -- the largest of the five
measured configurations (synthetic seeded inputs, recipe in gla_inputs.py).
``--workload`` selects another one (small, c2048, c4096, varlen).

``--pass wy`` measures the WY-representation forward of the gated delta rule
(gla_wy_fwd: w = A (beta 2^g k), u = A (beta v) per chunk) on inputs of the
workload's shape (k, v, A bf16 or fp32, beta and g fp32, seed 1006), with the
numpy fp64 oracle as the CPU baseline.

``--pass bwd`` measures the backward instead (gla_bwd: dq, dk, dv, dg and, with
an initial state, dh0, for seeded gradients do of o and dht of ht), with the
same line format, the backward's own algorithmic bytes and flops, and the fp64
backward oracle as the CPU baseline.

A step is one full forward (every kernel of the path as the library schedules
it: for segmented sequences the segment plan or a table clear and the single
pass, or with --schedule 1 segment summaries, state scan and output walk) over
the whole batch, with inputs resident in device memory.  Untimed steps for
--settle-ms (the GPU clock ramps up over the first tens of milliseconds of
load), W untimed warmup steps, then exactly K timed steps between two device
synchronisations; one JSON line is printed.

Also reported:
  roofline      algorithmic bytes (and flops) of one forward divided by its
                average duration, measured with HIP events on the launch stream
                over the timed region, against the 8 TB/s HBM peak or the dense
                MFMA peak, whichever bound gives the longer ideal time; `traffic`
                is the HBM bytes one forward moves (FETCH_SIZE + WRITE_SIZE of all
                its kernels, from rocprofv3 counter runs of the current device
                code), null when no matching measurement exists.
  cpu_baseline  the fp64 CPU oracle (test infrastructure) on the host cores, on a
                bounded sample of the same workload (whole sequences of the first
                heads), in tokens/s of the full workload's head count.
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
METRIC_BWD = "GLA chunked bwd tokens/s + TFLOP/s, fraction of MFMA/HBM roofline (1 GPU)"
METRIC_WY = "WY forward (gated delta rule) tokens/s + TFLOP/s, fraction of MFMA/HBM roofline (1 GPU)"
WY_SEED = 1006
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
_CSRC = os.path.join(ROOT, "chunkwise_gated_linear_amd", "csrc")
# the sources each pass's kernels and launches are built from
KERNEL_SRCS = {
    "fwd": [os.path.join(_CSRC, f) for f in ("gla_kernels.hip", "gla_walk_bf16.hip", "gla_device.h",
                                            "gla_internal.h", "gla_host.hip")],
    "bwd": [os.path.join(_CSRC, f) for f in ("gla_bwd.hip", "gla_kernels.hip", "gla_device.h",
                                            "gla_internal.h", "gla_host.hip")],
    "wy": [os.path.join(_CSRC, f) for f in ("gla_wy.hip", "gla_kernels.hip", "gla_device.h",
                                           "gla_internal.h", "gla_host.hip")],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CALIB_BYTES = 512 << 20


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def code_only(text: str) -> str:
    """C++ source without its comments, blank lines and indentation: what the
    compiler sees of it (string and character literals are kept whole)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.strip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def kernel_source_hash(which: str = "fwd") -> str:
    """Hash of the code (comments aside) of the device and launch sources of one
    pass: counters measured on other code are not reused."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS[which]:
        with open(path, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
            h.update(b"\0")
    return h.hexdigest()[:16]


def algorithmic(w, n_tokens, n_seqs):
    """Bytes (inputs read once + outputs written once) and flops of the method.

    Flops per token-head: 4KV (the state contribution k^T v and the read q S)
    plus (C+1)(K+V) (the causal halves of the in-chunk scores and of A v)."""
    e = 2 if w.dtype == "bf16" else 4
    H, K, V = w.H, w.K, w.V
    th = n_tokens * H
    nbytes = th * (2 * K * e + V * e + 4 * K) + th * V * e + 4 * n_seqs * H * K * V * (int(w.h0) + int(w.ht))
    flops = th * (4 * K * V + (w.chunk + 1) * (K + V))
    return nbytes, flops


def algorithmic_bwd(w, n_tokens, n_seqs):
    """Bytes (q, k, v, g, do, h0, dht read once; dq, dk, dv, dg, dh0 written once)
    and flops of the backward.

    Flops per token-head: 10KV (the two chunk summaries k~^T v and (q e^G)^T do,
    do S^T, v E^T and k~ E) plus (C+1)(3K+2V) (the causal halves of the in-chunk
    scores A and dA', of A^T do, dA' k and dA'^T q)."""
    e = 2 if w.dtype == "bf16" else 4
    H, K, V = w.H, w.K, w.V
    th = n_tokens * H
    state = 4 * n_seqs * H * K * V
    nbytes = (th * (2 * K * e + 2 * V * e + 4 * K)           # q, k, v, do, g
              + th * (2 * K * e + V * e + 4 * K)             # dq, dk, dv, dg
              + state * (2 * int(w.h0) + int(w.ht)))         # h0 and dh0, dht
    flops = th * (10 * K * V + (w.chunk + 1) * (3 * K + 2 * V))
    return nbytes, flops


def algorithmic_wy(w, n_tokens, n_seqs):
    """Bytes (k, v, beta, A, g read once; w, u written once) and flops (the full
    64-wide rows of A times the K + V scaled columns) of the WY forward."""
    e = 2 if w.dtype == "bf16" else 4
    th = n_tokens * w.H
    nbytes = th * (w.K * e + w.V * e + 4 + 64 * e + 4) + th * (w.K + w.V) * e
    flops = th * 2 * 64 * (w.K + w.V)
    return nbytes, flops


def cpu_baseline_wy(d, w, n_tokens, target_s=10.0):
    """The numpy fp64 WY oracle on the first heads, grown until about target_s
    seconds; reported as tokens/s of the full head count."""
    import numpy as np
    import oracle
    H = w.H

    def run(nh, reps=1):
        sl = lambda a: None if a is None else np.ascontiguousarray(a[:, :, :nh])
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.wy_reference(sl(d["k"]), sl(d["v"]), sl(d["beta"]), sl(d["A"]), sl(d["g"]),
                                cu_seqlens=d["cu_seqlens"])
        return (time.perf_counter() - t0) / reps

    nh = 1
    dt = run(nh)
    while dt < target_s / 2 and nh < H:
        nh = min(H, 2 * nh)
        dt = run(nh)
    reps = 1
    while dt * reps < 0.8 * target_s:
        reps = max(2 * reps, int(target_s / max(dt, 1e-5)))
        dt = run(nh, reps)
    return {"value": n_tokens * (nh / H) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{nh} of {H} heads, all {n_tokens} tokens, fp64 numpy matrix product per chunk "
                      f"(one thread), {dt * reps:.2f} s for {reps} run(s) on {cpu_model()}; tokens/s "
                      f"scaled to {H} heads"}


def describe(w, lengths):
    if w.varlen:
        return (f"varlen {w.n_seqs} seqs lengths U[{w.len_lo},{w.len_hi}] total {sum(lengths)}, "
                f"H={w.H} K={w.K} V={w.V} {w.dtype}, chunk {w.chunk}")
    return (f"B={w.B},H={w.H},T={w.T},K={w.K},V={w.V} {w.dtype} q/k/v, g fp32 logsigmoid(N(0,1))/16, "
            f"chunk {w.chunk}, h0={'yes' if w.h0 else 'no'}, ht={'stored' if w.ht else 'no'}")


def load_traffic(workload: str):
    """HBM bytes per launch recorded for `workload` (forward) or "bwd:<workload>"."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    which = workload.split(":")[0] if ":" in workload else "fwd"
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash(which):
        return None
    return entry.get("bytes_per_launch")


def _counter_means(run_dir, counter):
    """Mean per-dispatch value of `counter` per kernel name in a rocprofv3 --pmc CSV
    run directory (values of one dispatch are summed over the counter's instances)."""
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
    return {n: sum(v) / len(v) for n, v in per_kernel.items()}


def _largest(means):
    name = max(means, key=means.get)
    return name, means[name]


def record_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, read_fetch_dir=None):
    """HBM bytes of one forward: FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every kernel
    of the library, each scaled by what the same counter reads for a plain device copy of
    known size, summed over the kernels one forward launches.  Stored in
    profiles/traffic.json under the workload name and the hash of the current sources."""
    _, cf = _largest(_counter_means(copy_fetch_dir, "FETCH_SIZE"))
    _, cw = _largest(_counter_means(copy_write_dir, "WRITE_SIZE"))
    f_factor, w_factor = CALIB_BYTES / (cf * 1024.0), CALIB_BYTES / (cw * 1024.0)
    read_factor = None
    if read_fetch_dir:
        _, rf = _largest(_counter_means(read_fetch_dir, "FETCH_SIZE"))
        read_factor = CALIB_BYTES / (rf * 1024.0)
    fetch = {n: v for n, v in _counter_means(fetch_dir, "FETCH_SIZE").items() if "gla" in n}
    write = {n: v for n, v in _counter_means(write_dir, "WRITE_SIZE").items() if "gla" in n}
    kernels = {}
    for n in sorted(set(fetch) | set(write)):
        short = n.rsplit("(", 1)[0]
        kernels[short] = {"fetch_kib_counter": fetch.get(n, 0.0), "write_kib_counter": write.get(n, 0.0),
                          "fetch_bytes": fetch.get(n, 0.0) * 1024.0 * f_factor,
                          "write_bytes": write.get(n, 0.0) * 1024.0 * w_factor}
    total_f = sum(k["fetch_bytes"] for k in kernels.values())
    total_w = sum(k["write_bytes"] for k in kernels.values())
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[workload] = {
        "bytes_per_launch": total_f + total_w,
        "fetch_bytes": total_f, "write_bytes": total_w,
        "kernels": kernels,
        "copy_fetch_factor": f_factor, "copy_write_factor": w_factor,
        "read_only_fetch_factor": read_factor,
        "kernel_source_sha256_16": kernel_source_hash(workload.split(":")[0] if ":" in workload else "fwd"),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(table[workload], indent=1))


def cpu_baseline(d, w, n_tokens, target_s=10.0):
    """The fp64 oracle on whole sequences of the first heads, grown until about
    target_s seconds of wall time; reported as tokens/s of the full head count."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    threads = len(os.sched_getaffinity(0))
    H = w.H

    def run(nh, reps=1):
        sl = lambda a: np.ascontiguousarray(a[:, :, :nh])
        h0 = None if d["h0"] is None else np.ascontiguousarray(d["h0"][:, :nh])
        args = (sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.gla_reference(*args, h0=h0, cu_seqlens=d["cu_seqlens"], output_final_state=w.ht,
                                 threads=threads)
        return (time.perf_counter() - t0) / reps

    # the oracle runs one (sequence, head) per thread: start with enough heads to
    # occupy every core, double until about target_s / 2, then repeat the run
    # until about target_s of wall time in total
    n_seqs = w.n_seqs if w.varlen else w.B
    nh = min(H, max(1, -(-threads // n_seqs)))
    dt = run(nh)
    while dt < target_s / 2 and nh < H:
        nh = min(H, 2 * nh)
        dt = run(nh)
    reps = 1
    while dt * reps < 0.8 * target_s:
        reps = max(2 * reps, int(target_s / max(dt, 1e-5)))
        dt = run(nh, reps)
    used = min(threads, n_seqs * nh)
    return {"value": n_tokens * (nh / H) / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{nh} of {H} heads, all {n_tokens} tokens ({n_seqs} sequences), fp64 token "
                      f"recurrence, {dt * reps:.2f} s for {reps} run(s) on {cpu_model()}; tokens/s "
                      f"scaled to {H} heads"}


def cpu_baseline_bwd(d, w, n_tokens, do, dht, target_s=10.0, max_seq_tokens=4096):
    """The fp64 backward oracle on whole sequences (at most max_seq_tokens of
    each: the oracle keeps every state of a sequence) of the first heads, grown
    until about target_s seconds; reported as tokens/s of the full head count."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    threads = len(os.sched_getaffinity(0))
    H = w.H
    cu = d["cu_seqlens"]
    T = d["q"].shape[1]
    tcut = T if cu is not None else min(T, max_seq_tokens)
    if cu is not None and int(np.max(np.diff(cu))) > max_seq_tokens:
        raise ValueError("backward CPU baseline: packed sequences longer than the sample bound")

    def run(nh, reps=1):
        sl = lambda a: np.ascontiguousarray(a[:, :tcut, :nh])
        h0 = None if d["h0"] is None else np.ascontiguousarray(d["h0"][:, :nh])
        dh = None if dht is None else np.ascontiguousarray(dht[:, :nh])
        args = (sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(do))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.gla_reference_bwd(*args, h0=h0, dht=dh, cu_seqlens=cu, threads=threads)
        return (time.perf_counter() - t0) / reps

    n_seqs = w.n_seqs if w.varlen else w.B
    nh = min(H, max(1, -(-threads // n_seqs)))
    dt = run(nh)
    while dt < target_s / 2 and nh < H:
        nh = min(H, 2 * nh)
        dt = run(nh)
    reps = 1
    while dt * reps < 0.8 * target_s:
        reps = max(2 * reps, int(target_s / max(dt, 1e-5)))
        dt = run(nh, reps)
    used = min(threads, n_seqs * nh)
    sample_tokens = n_tokens if cu is not None else n_seqs * tcut
    return {"value": sample_tokens * (nh / H) / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{nh} of {H} heads, {sample_tokens} tokens ({n_seqs} sequences"
                      f"{'' if tcut == T else f', first {tcut} tokens of each'}), fp64 reverse token "
                      f"recurrence, {dt * reps:.2f} s for {reps} run(s) on {cpu_model()}; tokens/s "
                      f"scaled to {H} heads"}


def run_wy_bench(args, w, d):
    """Timed steps of gla_wy_fwd on inputs d of workload w's shape; prints the JSON line."""
    import torch
    import chunkwise_gated_linear_amd as gla
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    k, v, A = (torch.from_numpy(d[x]).to(tdt).to(dev) for x in ("k", "v", "A"))
    beta = torch.from_numpy(d["beta"]).to(dev)
    g = torch.from_numpy(d["g"]).to(dev)
    call = gla.WyCall(k, v, beta, A, g=g)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(4):
            call(sptr)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        call(sptr)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call(sptr)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = ev0.elapsed_time(ev1) / args.steps
    n_tokens = w.B * w.T
    nbytes, flops = algorithmic_wy(w, n_tokens, w.B)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    mfma_peak = MFMA_PEAK_TFLOPS[w.dtype]
    t_mfma = flops / (mfma_peak * 1e12)
    if t_hbm >= t_mfma:
        bound, achieved, peak, unit = "hbm", nbytes / (launch_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / (launch_ms * 1e-3) / 1e12, mfma_peak, "TFLOP/s"
    cpu = None if args.no_cpu_baseline else cpu_baseline_wy(d, w, n_tokens)
    line = {
        "metric": METRIC_WY, "value": n_tokens / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"WY forward, B={w.B},H={w.H},T={w.T},K={w.K},V={w.V} {w.dtype} k/v/A, "
                               f"beta, g fp32, chunk 64", "name": "wy:" + w.name, "tokens": n_tokens,
                   "heads": w.H, "seed": WY_SEED,
                   "inputs_digest": gi.array_digest(d["k"], d["v"], d["beta"], d["A"], d["g"]),
                   "workspace_bytes": call.ws_bytes},
        "tflops_algorithmic": flops / (ms_per_step * 1e-3) / 1e12,
        "roofline_time_us": max(t_hbm, t_mfma) * 1e6,
        "roofline": {"bound": bound, "kernel": "gla_wy_fwd_kernel", "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak, "traffic": load_traffic("wy:" + w.name),
                     "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                     "launch_ms_avg": launch_ms, "measured_copy_GBs": None},
        "single_launch_us": None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the W warmup steps, run untimed steps for this long so the GPU "
                         "reaches its sustained clock (short runs otherwise measure the ramp)")
    ap.add_argument("--workload", default=None, choices=sorted(gi.WORKLOADS),
                    help="default: long for the forward, c2048 for the backward")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd", "wy"],
                    help="fwd (default): the forward; bwd: the backward (gla_bwd); wy: the WY-representation "
                         "forward of the gated delta rule (gla_wy_fwd)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single", type=int, default=11,
                    help="launches timed one by one after the timed steps, warm and with L2/MALL evicted")
    ap.add_argument("--segment-chunks", type=int, default=0)
    ap.add_argument("--schedule", type=int, default=0, choices=[0, 1, 2, 3],
                    help="segmented sequences: 0 automatic, 1 three passes, 2 one pass; with --pass bwd: "
                         "0 automatic, 1 a separate scan launch, 2 the scan chained into the summary kernel, "
                         "3 the summary kernel walking whole chains")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the forward, run a plain 512 MiB device copy "
                         "(used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--read-calibration", action="store_true",
                    help="instead of the forward, read a 512 MiB buffer once per step (a sum), "
                         "to check the FETCH_SIZE scale on a read-only kernel")
    ap.add_argument("--record-traffic", nargs="+", metavar="DIR",
                    help="(no GPU) FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR [READ_FETCH_DIR]: "
                         "store the HBM bytes per forward of --workload from rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.workload is None:
        args.workload = "long" if args.which == "fwd" else "c2048"
    traffic_key = args.workload if args.which == "fwd" else args.which + ":" + args.workload
    if args.schedule != 0 or args.segment_chunks != 0:
        # counters are recorded for the library's own choices; another
        # schedule runs other kernels and has its own entry (or none)
        traffic_key += f"@schedule={args.schedule},segment_chunks={args.segment_chunks}"
    if args.record_traffic:
        if len(args.record_traffic) not in (4, 5):
            ap.error("--record-traffic takes 4 or 5 directories")
        record_traffic(traffic_key, *args.record_traffic)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; run it with --gpus 1 (how the path would "
              "shard over several GPUs is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunkwise_gated_linear_amd as gla

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    gla.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration or args.read_calibration:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            if args.copy_calibration:
                dst.copy_(src)
            else:
                src.sum()
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy" if args.copy_calibration else "read",
                          "bytes_read": CALIB_BYTES,
                          "bytes_written": CALIB_BYTES if args.copy_calibration else 0,
                          "launches": args.steps}), flush=True)
        return

    w = gi.WORKLOADS[args.workload]
    if args.which == "wy":
        if w.varlen:
            ap.error("--pass wy takes a fixed-length workload")
        d = gi.draw_wy(WY_SEED, w.B, w.T, w.H, w.K, w.V, dtype=w.dtype)
        run_wy_bench(args, w, d)
        return
    d = gi.make_inputs(w)
    lengths = d.get("lengths")
    digest = gi.array_digest(d["q"], d["k"], d["v"], d["g"], d["h0"], d["cu_seqlens"])
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(d[x]).to(tdt).to(dev) for x in ("q", "k", "v"))
    g = torch.from_numpy(d["g"]).to(dev)
    h0 = None if d["h0"] is None else torch.from_numpy(d["h0"]).to(dev)
    cu = None if d["cu_seqlens"] is None else torch.from_numpy(d["cu_seqlens"]).to(dev)
    n_tokens = int(q.shape[0] * q.shape[1])
    n_seqs = w.n_seqs if w.varlen else w.B
    do = dht = None
    if args.which == "fwd":
        call = gla.GlaCall(q, k, v, g, h0=h0, cu_seqlens=cu, output_final_state=w.ht,
                           segment_chunks=args.segment_chunks, schedule=args.schedule)
    else:
        # seeded gradients of the outputs: do like v (rounded to its dtype), dht
        # for a stored final state
        import numpy as np
        rng = np.random.default_rng(w.seed + 1)
        do = rng.standard_normal(d["v"].shape).astype(np.float32)
        dht = (rng.standard_normal(d["h0"].shape if d["h0"] is not None else (n_seqs, w.H, w.K, w.V))
               .astype(np.float32) if w.ht else None)
        tdo = torch.from_numpy(do).to(tdt).to(dev)
        do = tdo.float().cpu().numpy()
        tdht = None if dht is None else torch.from_numpy(dht).to(dev)
        call = gla.GlaBwdCall(q, k, v, g, tdo, h0=h0, dht=tdht, cu_seqlens=cu, schedule=args.schedule)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(4):
            call(sptr)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        call(sptr)
    torch.cuda.synchronize()

    # One event pair on the launch stream brackets the K back-to-back steps; the
    # average forward duration is their span / K (per-step event records would
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

    # After the timed steps (not part of `value`): single forwards, each between
    # its own event pair: back to back (warm); cold, after writing one 512 MiB
    # buffer and reading another, so that L2 and the MALL hold neither inputs nor
    # dirty lines.  Then the bandwidth of a plain 512 MiB device copy on this GPU,
    # as a measured counterpart of the HBM peak.
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
        del wbuf, rbuf
        launch_us = {"warm_median": warm_med, "warm_min": warm_min, "cold_median": cold_med,
                     "cold_min": cold_min, "launches": args.single}
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

    # the workspace's sticky status word: a bounded wait that ran out in any
    # step means that step's results may be wrong, and the line is not printed
    st = call.status()
    if st != 0:
        sys.exit(f"bench.py: status word {st:#x} after the timed steps (a bounded wait between waves ran out)")

    nbytes, flops = (algorithmic if args.which == "fwd" else algorithmic_bwd)(w, n_tokens, n_seqs)
    tokens_per_s = n_tokens / (ms_per_step * 1e-3)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    mfma_peak = MFMA_PEAK_TFLOPS[w.dtype]
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (mfma_peak * 1e12)
    traffic = load_traffic(traffic_key)
    if t_hbm >= t_mfma:
        bound, achieved, peak, unit = "hbm", nbytes / (launch_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / (launch_ms * 1e-3) / 1e12, mfma_peak, "TFLOP/s"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = (cpu_baseline(d, w, n_tokens) if args.which == "fwd"
               else cpu_baseline_bwd(d, w, n_tokens, do, dht))

    ws_bytes = call.ws_bytes
    line = {
        "metric": METRIC if args.which == "fwd" else METRIC_BWD,
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
        "config": {"workload": describe(w, lengths), "name": w.name, "tokens": n_tokens, "heads": w.H,
                   "seed": w.seed, "inputs_digest": digest, "workspace_bytes": ws_bytes},
        "tflops_algorithmic": tflops,
        "roofline_time_us": max(t_hbm, t_mfma) * 1e6,
        "roofline": {
            "bound": bound,
            "kernel": ("gla_fwd (every kernel of one forward)" if args.which == "fwd"
                       else "gla_bwd (every kernel of one backward)"),
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": achieved / peak,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": nbytes,
            "algorithmic_flops_per_launch": flops,
            "launch_ms_avg": launch_ms,
            "measured_copy_GBs": copy_gbs,
        },
        "single_launch_us": launch_us,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
