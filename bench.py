"""Benchmark of the gated bidirectional ReLU linear-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p_60s]
                    [--form workload|token-causal|token-causal-strict]

One step is one full call of the operator (RoPE tables, state partials,
reduce, fused output or token-causal walk) on one seeded synthetic input set
already resident in HBM.  The default form is the workload's own
(bidirectional for 720p_60s); the token-causal forms run the same grid with
token i reading tokens j <= i (or j < i).  Prints ONE JSON line on stdout (progress goes to stderr):
tokens/s for the whole step, achieved HBM GB/s of the step's algorithmic
bytes, the roofline of the dominant kernel (HIP-event durations taken on the
call's stream during the timed steps), and the fp64 CPU oracle timed on a
bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 2500.0, "e5m2": 2500.0, "f32": 157.3}   # dense MFMA of the operand type
# the kernels use (fp8 I/O of either format is widened to bf16 operands; fp32 I/O runs fp32 MFMA)
METRIC = "tokens/s + achieved HBM GB/s (% of peak), gated linear attn fwd, 720p/60s grid"
KERNEL_SOURCES = ["gated_bidirectional_linear_amd/csrc/" + f for f in
                  ("gla_launch.h", "gla_device.h", "gla_common.h", "gla_tables.hip", "gla_state.hip",
                   "gla_output.hip")]
CAUSAL_SOURCES = KERNEL_SOURCES + ["gated_bidirectional_linear_amd/csrc/gla_causal.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(token_causal: bool = False) -> str:
    """Hash of the kernel sources a form's launches are built from."""
    h = hashlib.sha256()
    for p in (CAUSAL_SOURCES if token_causal else KERNEL_SOURCES):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_alg_bytes(w, kernel: str, token_causal: bool = False) -> int:
    """Algorithmic HBM bytes one launch of a kernel must move."""
    s = w.elem_size
    big = w.N * w.heads * w.d * s
    if kernel == "output_kernel" and token_causal:   # read q, k, v, g, beta; write out
        return 5 * big + w.N * w.heads * s
    if kernel == "output_kernel":        # read q, g; write out
        return 3 * big
    if kernel == "state_partial_kernel":  # read k, v, beta
        return 2 * big + w.N * w.heads * s
    return 0


def kernel_alg_flops(w, kernel: str, token_causal: bool = False) -> int:
    """Algorithmic MFMA flops of one launch: the state contraction (pass 1)
    and the numerators (pass 2), 2 N heads d^2 each; the token-causal walk
    does both (its intra-tile products are design overhead, not counted)."""
    one = 2 * w.N * w.heads * w.d * w.d
    if kernel == "output_kernel":
        return 2 * one if token_causal else one
    if kernel == "state_partial_kernel":
        return one
    return 0


def read_traffic(kernel: str, workload: str, token_causal: bool = False):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy-kernel calibration), stored under profiles/.
    None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash(token_causal):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _pmc_means(csv_path: str, counter: str) -> dict:
    """Mean per-dispatch value of one counter, per kernel name, from a
    rocprofv3 counter_collection.csv (values summed over dimensions)."""
    import collections
    import csv
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            per[(r["Dispatch_Id"], r["Kernel_Name"])] += float(r["Counter_Value"])
    sums = collections.defaultdict(list)
    for (d, k), v in per.items():
        sums[k].append(v)
    return {k: sum(v) / len(v) for k, v in sums.items()}


def write_traffic_summary(fetch_csv: str, write_csv: str, calib_mib: int, workload: str, commands: str,
                          token_causal: bool = False) -> None:
    """Turn FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) into HBM bytes per
    launch of the two streaming kernels, each counter scaled by what it reads
    for a device-to-device copy of calib_mib MiB (read calib_mib, write calib_mib)."""
    fetch = _pmc_means(fetch_csv, "FETCH_SIZE")
    write = _pmc_means(write_csv, "WRITE_SIZE")
    # the calibration copy is the only elementwise kernel in these runs
    copy = [k for k in fetch if "elementwise" in k and "neg" in k.lower()] or \
           [k for k in fetch if "elementwise" in k]
    if not copy:
        raise SystemExit("no calibration copy kernel in the counter runs (run bench.py with --calib-copy-mib)")
    ck = max(copy, key=lambda k: fetch[k])
    known_kib = calib_mib * 1024.0
    f_scale = known_kib / fetch[ck]
    w_scale = known_kib / write[ck]
    # every launch of a pass (whichever of its kernel variants ran) is summarised
    # under the timing name of that pass
    for prefix, short in (("gla::output", "output_kernel"), ("gla::token_causal", "output_kernel"),
                          ("gla::state_partial", "state_partial_kernel")):
        names = [k for k in fetch if k.removeprefix("void ").startswith(prefix) and k not in copy]
        if not names:
            continue
        kn = names[0]
        fetched = fetch[kn] * f_scale * 1024
        written = write.get(kn, 0.0) * w_scale * 1024
        path = os.path.join(ROOT, "profiles", f"{short}_{workload}_traffic.txt")
        with open(path, "w") as f:
            f.write(f"# HBM traffic of {short} on the {workload} workload, from rocprofv3 counters\n")
            f.write("# commands:\n")
            for line in commands.strip().splitlines():
                f.write(f"#   {line}\n")
            f.write(f"kernel: {kn.removeprefix('void ').split('(')[0]}\n")
            f.write(f"FETCH_SIZE_kib_per_dispatch: {fetch[kn]:.1f}\n")
            f.write(f"WRITE_SIZE_kib_per_dispatch: {write.get(kn, 0.0):.1f}\n")
            f.write(f"copy_calibration: {ck.split('(')[0]} of {calib_mib} MiB read + {calib_mib} MiB written; "
                    f"FETCH_SIZE {fetch[ck]:.1f} KiB, WRITE_SIZE {write[ck]:.1f} KiB\n")
            f.write(f"fetch_scale: {f_scale:.4f}\n")
            f.write(f"write_scale: {w_scale:.4f}\n")
            f.write(f"read_bytes_per_launch: {fetched:.0f}\n")
            f.write(f"write_bytes_per_launch: {written:.0f}\n")
            f.write(f"traffic_bytes_per_launch: {fetched + written:.0f}\n")
            f.write(f"kernel_source_sha256: {kernel_source_hash(token_causal)}\n")
        print(f"wrote {path}: {(fetched + written) / 1e9:.3f} GB per launch")


SQ_COUNTERS = ("SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_LDS "
               "SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")


def write_sq_summary(pmc_csv: str, workload: str, commands: str, token_causal: bool = False,
                     num_cu: int = 256, num_xcd: int = 8) -> None:
    """Per-kernel issue summary from one rocprofv3 counter run of SQ_COUNTERS.

    cycles = GRBM_GUI_ACTIVE / XCDs (the dispatch's clock cycles; the counter is
    summed over the 8 XCDs).  Per-SIMD fractions divide a chip-wide sum by
    cycles x CUs x 4 SIMDs:
      valu      = 4 SQ_ACTIVE_INST_VALU (quad-cycles that waves spend issuing
                  vector instructions, summed over waves; two waves of one SIMD
                  can count in the same cycle, so this can exceed 1)
      mfma      = SQ_VALU_MFMA_BUSY_CYCLES (32 busy cycles per 32x32x16 MFMA)
      coexec    = SQ_VALU_MFMA_COEXEC_CYCLES (cycles in which a vector
                  instruction issued while the matrix unit was busy)
      lds       = 4 SQ_ACTIVE_INST_LDS, lds_wait = 4 SQ_WAIT_INST_LDS (summed over waves)
    bank_conflicts is SQ_LDS_BANK_CONFLICT per dispatch (cycles, chip-wide);
    clock = cycles / dispatch duration."""
    import collections
    import csv
    names = SQ_COUNTERS.split()
    means = {n: _pmc_means(pmc_csv, n) for n in names}
    dur = collections.defaultdict(list)
    seen = set()
    for r in csv.DictReader(open(pmc_csv)):
        if r["Dispatch_Id"] in seen:
            continue
        seen.add(r["Dispatch_Id"])
        dur[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    path = os.path.join(ROOT, "profiles", f"sq_{workload}.txt")
    with open(path, "w") as f:
        f.write(f"# SQ issue counters per kernel on the {workload} workload, from one rocprofv3 counter run\n")
        f.write("# commands:\n")
        for line in commands.strip().splitlines():
            f.write(f"#   {line}\n")
        f.write(f"# cycles = GRBM_GUI_ACTIVE / {num_xcd}; per-SIMD fractions = chip-wide sum / "
                f"(cycles x {num_cu} CUs x 4 SIMDs):\n")
        f.write("# valu = 4 SQ_ACTIVE_INST_VALU (summed over waves), mfma = SQ_VALU_MFMA_BUSY_CYCLES,\n"
                "# coexec = SQ_VALU_MFMA_COEXEC_CYCLES, lds = 4 SQ_ACTIVE_INST_LDS, lds_wait = 4 SQ_WAIT_INST_LDS;\n"
                "# bank_conflicts = SQ_LDS_BANK_CONFLICT per dispatch; means over dispatches\n")
        f.write(f"{'kernel':56s} {'valu':>6s} {'mfma':>6s} {'coexec':>6s} {'lds':>6s} {'ldswait':>7s} "
                f"{'bankconf':>9s} {'clock':>9s}\n")
        for k in sorted(means["GRBM_GUI_ACTIVE"]):
            if not k.removeprefix("void ").startswith("gla::"):
                continue
            cyc = means["GRBM_GUI_ACTIVE"][k] / num_xcd
            if cyc <= 0:
                continue
            simd = cyc * num_cu * 4
            ns = sum(dur[k]) / len(dur[k]) if dur.get(k) else 0.0
            clock = f"{cyc / ns:5.2f} GHz" if ns > 50_000 else "n/a"
            f.write(f"{k.removeprefix('void ').split('(')[0][:56]:56s} "
                    f"{4 * means['SQ_ACTIVE_INST_VALU'].get(k, 0) / simd:6.3f} "
                    f"{means['SQ_VALU_MFMA_BUSY_CYCLES'].get(k, 0) / simd:6.3f} "
                    f"{means['SQ_VALU_MFMA_COEXEC_CYCLES'].get(k, 0) / simd:6.3f} "
                    f"{4 * means['SQ_ACTIVE_INST_LDS'].get(k, 0) / simd:6.3f} "
                    f"{4 * means['SQ_WAIT_INST_LDS'].get(k, 0) / simd:7.3f} "
                    f"{means['SQ_LDS_BANK_CONFLICT'].get(k, 0):9.3g} {clock:>9s}\n")
        f.write(f"kernel_source_sha256: {kernel_source_hash(token_causal)}\n")
    print(f"wrote {path}")


def write_stats_summary(stats_csv: str, workload: str, commands: str, token_causal: bool = False,
                        warmup: int = 2, bench_log: str = "") -> None:
    """Kernel-trace statistics (rocprofv3 --kernel-trace --stats, kernel_stats.csv)
    as a short text table under profiles/, plus, from the per-dispatch trace
    next to it (kernel_trace.csv), each kernel's mean over the launches after
    the first `warmup` calls (the timed steps of the profiled command), and the
    HIP-event times per launch that the profiled bench.py run itself printed
    (its JSON line in `bench_log`)."""
    import collections
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    trace_csv = stats_csv.replace("kernel_stats.csv", "kernel_trace.csv")
    steady = {}
    if os.path.exists(trace_csv):
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(trace_csv)):
            per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        for k, v in per.items():
            v.sort()
            timed = v[warmup:] if len(v) > warmup else v
            steady[k] = (sum(e - b for b, e in timed) / len(timed) / 1e3, len(timed))
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}_stats.txt")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel-trace statistics, {workload} workload\n")
        f.write("# commands:\n")
        for line in commands.strip().splitlines():
            f.write(f"#   {line}\n")
        f.write(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}\n")
        for r in rows:
            name = r["Name"].split("(")[0].replace("void ", "")
            f.write(f"{name[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                    f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):6.2f}\n")
        if steady:
            f.write(f"# mean over the timed steps (launches after the first {warmup}), from the per-dispatch trace:\n")
            for k, (us, n) in sorted(steady.items(), key=lambda kv: -kv[1][0]):
                if n <= 1:
                    continue
                name = k.split("(")[0].replace("void ", "")
                f.write(f"steady {name[:53]:53s} {n:6d} {us:10.1f}\n")
        if bench_log and os.path.exists(bench_log):
            rec = None
            for line in open(bench_log):
                if line.startswith("{"):
                    rec = json.loads(line)
            if rec is not None:
                f.write("# the same run's own HIP-event times per launch (bench.py JSON line):\n")
                for k, v in rec.get("kernels", {}).items():
                    if v.get("ms_per_launch"):
                        f.write(f"events {k:53s} {v['launches']:6d} {v['ms_per_launch'] * 1e3:10.1f}\n")
        f.write(f"kernel_source_sha256: {kernel_source_hash(token_causal)}\n")
    print(f"wrote {path}")


def host_threads():
    """(usable cores, BLAS description) of this process: the cores in its CPU
    affinity mask, and each BLAS library numpy loaded with its thread count."""
    cores = len(os.sched_getaffinity(0))
    blas = []
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas.append({"library": i.get("internal_api"), "version": i.get("version"),
                             "threads": i.get("num_threads")})
    except Exception:
        pass
    return cores, blas


def timed_oracle(fn):
    """Run fn() with the BLAS threads set to every usable core; returns
    (seconds, cores, blas description)."""
    cores, _ = host_threads()
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limit = None
    try:
        _, blas = host_threads()
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return dt, cores, blas


def cpu_baseline(w, inp, heads_sample: int):
    """Time the fp64 oracle on `heads_sample` heads of the full workload (all
    tokens, complete state and output) and scale to the whole workload."""
    import oracle.gla_oracle as orc
    from workloads import head_slice_f32
    heads = list(range(min(heads_sample, w.heads)))
    sub = head_slice_f32(inp, heads) if w.dtype != "f32" else {
        **inp, **{n: inp[n][:, heads] for n in ("q", "k", "v", "g", "beta")}}
    if w.block_frames is not None:
        run = lambda: orc.gla_block_causal_forward(sub["q"], sub["k"], sub["v"], sub["beta"], sub["g"],  # noqa: E731
                                                   sub["rms_w"], sub["grid"], sub["eps"], w.block_frames)
    else:
        run = lambda: orc.gla_forward(sub["q"], sub["k"], sub["v"], sub["beta"], sub["g"], sub["rms_w"],  # noqa: E731
                                      sub["grid"], sub["eps"])
    dt, cores, blas = timed_oracle(run)
    per_call = dt * w.heads / len(heads)
    return {
        "value": w.N / per_call,
        "unit": "tokens/s",
        "cores": cores,
        "blas": blas,
        "kind": "oracle",
        "sample": f"{len(heads)} of {w.heads} heads at full N={w.N} (whole state and output), "
                  f"{dt:.2f} s, scaled x{w.heads / len(heads):g} to the full workload",
    }


def cpu_baseline_token_causal(w, inp, include_self: bool, heads_sample: int = 2, target_tokens: int = 1 << 30):
    """Time the fp64 oracle's running-sum token-causal evaluation on
    `heads_sample` heads over the first whole frames of the grid (up to
    target_tokens tokens; every output row) and scale to the whole workload."""
    import numpy as np
    import oracle.gla_oracle as orc
    from workloads import head_slice_f32
    hw = w.H * w.W
    frames = max(1, min(w.T, round(target_tokens / hw)))
    n = frames * hw
    heads = list(range(min(heads_sample, w.heads)))
    sub = head_slice_f32(inp, heads) if w.dtype != "f32" else {
        **inp, **{k: inp[k][:, heads] for k in ("q", "k", "v", "g", "beta")}}
    part = {k: sub[k][:n] for k in ("q", "k", "v", "g", "beta")}
    dt, cores, blas = timed_oracle(
        lambda: orc.gla_token_causal_rows(part["q"], part["k"], part["v"], part["beta"], part["g"], sub["rms_w"],
                                          (frames, w.H, w.W), w.eps, np.arange(n), include_self=include_self))
    scale = (w.N / n) * w.heads / len(heads)
    return {
        "value": w.N / (dt * scale),
        "unit": "tokens/s",
        "cores": cores,
        "blas": blas,
        "kind": "oracle",
        "sample": f"token-causal running sums, {len(heads)} of {w.heads} heads, first {frames} of {w.T} frames "
                  f"({n} tokens, every row), {dt:.2f} s, scaled x{scale:.4g} to the full workload",
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 50, or as many as take ~50 ms when a step is shorter than 1 ms)")
    # the clocks settle after ~20 steps (~25 ms) of load: 3 warm-up steps time
    # ~3% slower at 720p/60s, 20 or more time the same
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="720p_60s")
    ap.add_argument("--dtype", choices=("bf16", "fp8", "e5m2", "f32"), default=None,
                    help="operator I/O dtype (default: the workload's own, bf16 for 720p_60s); "
                         "fp8 = OCP FP8 E4M3 q, k, v, g, beta and out; e5m2 = OCP FP8 E5M2")
    ap.add_argument("--form", choices=("workload", "token-causal", "token-causal-strict"), default="workload",
                    help="operator form: the workload's own (bidirectional or block-causal), or the token-level "
                         "causal form with the own token included (token-causal) or excluded (-strict)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--batch", type=int, default=1,
                    help="independent sequences per call ([B, N, heads, d] tensors, items drawn with seeds "
                         "seed, seed + 1, ...); tokens/s and bytes count all items")
    ap.add_argument("--plan", action="append", default=[], metavar="KNOB=VALUE",
                    help="tuning only: set a launch-plan knob of the library (gla_internal.h; names as in "
                         "gated_bidirectional_linear_amd.PLAN_KNOBS) for this run; the line records it in "
                         "config.plan")
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, run 3 elementwise copies (torch.neg, fp32) reading and "
                         "writing this many MiB: a streaming kernel of known size for counter calibration")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="CPU only: write the traffic summaries under profiles/ from two rocprofv3 "
                         "counter_collection.csv files (FETCH_SIZE run, WRITE_SIZE run)")
    ap.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                    help="CPU only: write the kernel-trace summary under profiles/ from a rocprofv3 "
                         "kernel_stats.csv")
    ap.add_argument("--pmc-commands", default="", help="commands recorded in the summaries")
    ap.add_argument("--stats-bench-log", default="", help="output of the profiled bench.py run (its JSON line)")
    ap.add_argument("--stats-name", default="",
                    help="name of the kernel-trace summary (profiles/kernels_NAME_stats.txt) when it is not the "
                         "workload's own, e.g. for a run with another warm-up length")
    ap.add_argument("--sq-summary", metavar="COUNTER_CSV",
                    help="CPU only: write the SQ issue summary under profiles/ from a rocprofv3 "
                         "counter_collection.csv of the counters in SQ_COUNTERS")
    args = ap.parse_args(argv)

    token_causal = args.form != "workload"
    # names the profiles/ summaries: workload, a dtype other than the workload's own, the form
    from workloads import WORKLOADS as _W
    own = _W[args.workload].dtype if args.workload in _W else None
    label = (args.workload + (f"_{args.dtype}" if args.dtype not in (None, own) else "")
             + ("_token_causal" if token_causal else ""))
    if args.sq_summary:
        write_sq_summary(args.sq_summary, label, args.pmc_commands, token_causal)
        return 0
    if args.stats_summary:
        write_stats_summary(args.stats_summary, args.stats_name or label, args.pmc_commands, token_causal,
                            args.warmup, args.stats_bench_log)
        return 0
    if args.pmc_summary:
        write_traffic_summary(args.pmc_summary[0], args.pmc_summary[1], args.calib_copy_mib or 1024,
                              label, args.pmc_commands, token_causal)
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this operator's path is measured per GPU "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        return 2
    from gated_bidirectional_linear_amd import PLAN_KNOBS
    plan = {}
    for kv in args.plan:
        name, _, value = kv.partition("=")
        if name not in PLAN_KNOBS or not value.isdigit():
            print(f"--plan {kv}: expected KNOB=VALUE with KNOB in {sorted(PLAN_KNOBS)}", file=sys.stderr)
            return 2
        plan[name] = int(value)

    import numpy as np
    import torch

    import gated_bidirectional_linear_amd as gla
    from workloads import WORKLOADS, make_workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    for name, value in plan.items():
        gla.plan_override(name, value)
    w = WORKLOADS[args.workload]
    B = args.batch
    if B < 1:
        print("--batch must be at least 1", file=sys.stderr)
        return 2
    # profiles/ hold the default-dtype, single-sequence kernels
    profiled = B == 1 and not plan
    if args.dtype is not None:
        import dataclasses
        w = dataclasses.replace(w, dtype=args.dtype)
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: grid {w.T}x{w.H}x{w.W} N={w.N} heads={w.heads} d={w.d} {w.dtype}")
    t0 = time.time()
    inp = make_workload_inputs(w, seed=args.seed, keep_f32=(w.dtype == "f32"))
    items = [inp] + [make_workload_inputs(w, seed=args.seed + b, keep_f32=(w.dtype == "f32")) for b in range(1, B)]
    log(f"[bench] inputs drawn in {time.time() - t0:.1f} s" + (f" ({B} items)" if B > 1 else ""))

    def upload_one(it, name):
        if w.dtype == "bf16":
            return torch.from_numpy(it[name + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        if w.dtype in ("fp8", "e5m2"):
            tdt = torch.float8_e4m3fn if w.dtype == "fp8" else torch.float8_e5m2
            return torch.from_numpy(it[name + "_bits"]).to(dev).view(tdt)
        return torch.from_numpy(it[name]).to(dev)

    def upload(name):
        if B == 1:
            return upload_one(inp, name)
        return torch.stack([upload_one(it, name) for it in items]).contiguous()

    # Working sets that would sit in the 256 MB Infinity Cache are rotated over
    # enough copies (> 1 GB total) that each step reads from HBM.
    call_bytes = B * w.alg_bytes()
    sets = max(1, -(-1_000_000_000 // call_bytes)) if call_bytes < 1_000_000_000 else 1
    sets = min(sets, 64)   # a grid this small stays in the caches whatever the rotation
    bufs = []
    for i in range(sets):
        t = {n: upload(n) for n in ("q", "k", "v", "g", "beta")}
        t["out"] = torch.empty_like(t["q"])
        bufs.append(t)
    rms_w = torch.from_numpy(inp["rms_w"]).to(dev)
    causal = token_causal or w.block_frames is not None
    # carried state of the causal forms: each step continues the previous one's
    lead = () if B == 1 else (B,)
    state_S = torch.zeros(lead + (w.heads, w.d, w.d), dtype=torch.float32, device=dev) if causal else None
    state_z = torch.zeros(lead + (w.heads, w.d), dtype=torch.float32, device=dev) if causal else None
    torch.cuda.synchronize()
    log(f"[bench] {sets} input set(s) resident on {torch.cuda.get_device_name(dev)}; form {args.form}")

    def step(i):
        b = bufs[i % sets]
        grid = (w.T, w.H, w.W)
        if token_causal:
            gla.token_causal_forward(b["q"], b["k"], b["v"], b["beta"], b["g"], rms_w, grid, state_S, state_z,
                                     include_self=(args.form == "token-causal"), eps=w.eps, out=b["out"])
        elif w.block_frames is not None:
            gla.block_causal_forward(b["q"], b["k"], b["v"], b["beta"], b["g"], rms_w, grid, state_S, state_z,
                                     w.block_frames, eps=w.eps, out=b["out"])
        else:
            gla.forward(b["q"], b["k"], b["v"], b["beta"], b["g"], rms_w, grid, eps=w.eps, out=b["out"])

    torch.cuda.synchronize()
    t_w = time.perf_counter()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    est = (time.perf_counter() - t_w) / max(1, args.warmup)   # seconds per step, roughly
    if args.steps is None:
        args.steps = 50 if est >= 1e-3 else max(50, min(5000, int(0.05 / max(est, 1e-6))))
    # HIP event pairs around one kernel per sampled step, kernels in rotation:
    # every step when steps are long, every 8th step when they are short (a
    # pair adds ~5 us to a 56 us step at 480p, and none measurably to 1 ms)
    period = 1 if est >= 5e-4 else 8
    gla.timing_read()            # discard anything recorded before
    gla.timing_enable(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        gla.timing_select([(i // period) % gla.NUM_KERNELS] if i % period == 0 else [])
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    gla.timing_enable(False)
    gla.timing_select(None)
    kt = gla.timing_read()
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms")

    ms_step = elapsed * 1e3 / args.steps
    tokens_s = B * w.N / (ms_step * 1e-3)
    alg_step = B * (w.alg_bytes() + (2 * w.heads * (w.d * w.d + w.d) * 4 if token_causal else 0))
    step_gbps = alg_step / (ms_step * 1e-3) / 1e9
    kernels = {k: {"ms_per_launch": (ms / n if n else None), "launches": n} for k, (ms, n) in kt.items()}
    dom = max(("state_partial_kernel", "output_kernel"), key=lambda k: kt[k][0] / max(1, kt[k][1]))
    dom_ms = kt[dom][0] / max(1, kt[dom][1])
    achieved = B * kernel_alg_bytes(w, dom, token_causal) / (dom_ms * 1e-3) / 1e9
    traffic = read_traffic(dom, label, token_causal) if profiled else None
    for k, v in kernels.items():
        log(f"[bench]   {k:22s} {v['ms_per_launch'] * 1e3 if v['ms_per_launch'] else 0:9.1f} us/launch")

    warm = None
    if sets > 1:
        # the same steps on one input set, which the 256 MB Infinity Cache can
        # hold between steps: the "warm" figure, reported next to the cold one
        for i in range(3):
            step(0)
        torch.cuda.synchronize()
        t_w = time.perf_counter()
        for i in range(args.steps):
            step(0)
        torch.cuda.synchronize()
        ms_w = (time.perf_counter() - t_w) * 1e3 / args.steps
        warm = {"ms_per_step": ms_w, "tokens_per_s": B * w.N / (ms_w * 1e-3),
                "hbm_gbps": alg_step / (ms_w * 1e-3) / 1e9, "input_sets": 1}
        log(f"[bench] warm (one input set): {ms_w * 1e3:.1f} us/step")

    if args.calib_copy_mib > 0:
        # an elementwise streaming kernel of known size: read and write calib MiB
        src = torch.ones((args.calib_copy_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle on {2 if token_causal else args.cpu_heads} heads ...")
        cpu = (cpu_baseline_token_causal(w, inp, args.form == "token-causal") if token_causal
               else cpu_baseline(w, inp, args.cpu_heads))
        log(f"[bench] oracle: {cpu['value']:.1f} tokens/s ({cpu['sample']})")

    rec = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8_e4m3", "e5m2": "fp8_e5m2"}.get(w.dtype, w.dtype),
        "data": "synthetic (seeded N(0,1) q,k,v,g; beta=sigmoid(N(0,1)); rms_w=1+0.1N(0,1))",
        "config": {
            "workload": w.name,
            **({"plan": plan} if plan else {}),
            "grid": f"{w.T}x{w.H}x{w.W}",
            "tokens": B * w.N,
            "heads": w.heads,
            "head_dim": w.d,
            "eps": w.eps,
            "mode": ({"token-causal": "token-causal (j <= i)", "token-causal-strict": "token-causal (j < i)"}
                     [args.form] if token_causal else
                     "bidirectional" if w.block_frames is None else f"block-causal F={w.block_frames}"),
            "input_sets": sets,
            "batch": B,
        },
        "cache": "cold (inputs rotated over sets larger than the 256 MB Infinity Cache)" if sets > 1 else "cold",
        "warm": warm,
        "hbm_gbps": step_gbps,
        "hbm_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "alg_bytes_per_step": alg_step,
        "kernels": kernels,
        "kernel_timing": ("HIP events around one kernel on " + ("every timed step" if period == 1 else
                          f"every {period}th timed step") + ", the four kernels in rotation; launches timed per "
                          "kernel: "
                          + ", ".join(f"{k} {v[1]}" for k, v in kt.items())),
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
        "mfma": {k: {
            "achieved": B * kernel_alg_flops(w, k, token_causal) / (kt[k][0] / kt[k][1] * 1e-3) / 1e12,
            "peak": MFMA_PEAK_TFLOPS[w.dtype],
            "unit": "TFLOP/s",
            "frac": B * kernel_alg_flops(w, k, token_causal) / (kt[k][0] / kt[k][1] * 1e-3) / 1e12
            / MFMA_PEAK_TFLOPS[w.dtype],
        } for k in ("state_partial_kernel", "output_kernel") if kt[k][1]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
