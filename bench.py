#!/usr/bin/env python3
"""Decode-step benchmark for libpagedattn on one MI355X.

One step = the whole hot path over one batch: store_kvcache of the step's new
token per sequence, then paged_attention_decode (attention kernel plus, when
contexts are split, the merge kernel). Inputs are seeded synthetic data of the
workload's shape, resident in HBM before timing starts.

Each workload is timed twice over K steps: a warm loop (steps back to back,
wall clock around all K) and a cold loop (each step after a 1 GiB read that
evicts the K/V from the L2s and the last-level cache, outside the events).

Prints ONE JSON line:
  value        KV GB/s of the warm loop: logical K+V bytes one decode must read
               (sum over sequences of L * Hkv * D * e * 2) / wall time per step
  tokens_per_s sequences advanced per second (B / time per step)
  roofline     the attention kernel alone, cold: the same KV bytes / the mean
               duration of its cold-loop launches (HIP events on its stream),
               against MI355X's 8 TB/s HBM peak and against the measured
               streaming-read ceiling; the warm figure beside it; traffic from
               committed rocprofv3 counter summaries when they match the
               current kernel source
  cold_step, split_cold_median_us   cold step time and its store / attention /
               merge-and-gaps split
  stream_read_ceiling  best rate of a plain streaming-read kernel on this GPU
  cpu_baseline the float64 CPU oracle timed on this host on a bounded sample
               of the same workload (a reported baseline, not the target)
  workloads    (default run) the same record for each other workload
  prefill      (default run) full-prompt paged prefill, TFLOP/s against the MFMA peak and
               against the measured matrix-core ceiling (a loop of independent 16x16x32
               instructions of the prompt's dtype, two wavefronts per SIMD), on the
               Llama-shaped (fp16) and skewed (bf16) workloads' prompts

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--workload NAME] [--prefill]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "paged-attn decode KV HBM GB/s (% of MI355X peak) and decode tokens/s"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "skewed_prefix_bf16"
# The default run also measures these workloads, each in a record of its own.
RECORD_WORKLOADS = ["tiny_fp32", "qwen3_0p6b_bf16", "llama32_1b_fp16", "long_ctx_bf16"]
# Launch mode a workload is specified with (others: 0, the library's automatic choice).
WORKLOAD_PARTITION = {"long_ctx_bf16": 512}
# Prefix-cache hit length a workload is specified with: the leading tokens its sequences share
# (groups of 8 share their first 512 in the skewed batch). It is passed as cached_prefix_tokens,
# as an engine passes the hit length its block manager reports; others use the library default.
WORKLOAD_CACHED_PREFIX = {"skewed_prefix_bf16": 512}
# Workloads whose CPU baseline is also taken with one BLAS thread.
ONE_THREAD_BASELINE = {"tiny_fp32", "qwen3_0p6b_bf16", "llama32_1b_fp16"}
# Default run: full-prompt prefill records (TFLOP/s) of these workloads' prompts.
PREFILL_RECORDS = ("llama32_1b_fp16", "skewed_prefix_bf16")
PREFILL_RECORD_STEPS, PREFILL_RECORD_WARMUP = 100, 10
KERNEL_SOURCE = ROOT / "paged_attention_decode_amd" / "csrc" / "decode.hip"
PROFILES = ROOT / "profiles"
COPY_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help=f"time this workload only (default: {DEFAULT_WORKLOAD} as the headline, plus a record "
                         "for each other workload)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="0 automatic, -1 one pass, -2 balanced split, -3 workgroup split, >0 fixed ranges of "
                         "that many tokens (default: the workload's own, 512 for the long-context one, else 0)")
    ap.add_argument("--cached-prefix-tokens", type=int, default=None,
                    help="leading tokens per context read with cached loads (0 library default, -1 none; "
                         "default: the workload's shared-prefix length, 512 for the skewed batch, else 0)")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="read the leading blocks that neighbouring sequences share once per group "
                         "(pa_decode_opts.shared_prefix; the sharing is found on the device)")
    ap.add_argument("--fused-step", action="store_true",
                    help="run each step as one pa_decode_step launch (scatter fused into the attention kernel)")
    ap.add_argument("--prefill", action="store_true",
                    help="time pa_paged_prefill instead: every context token of the workload is a prompt token "
                         "(full causal prefill); prints its own JSON line in TFLOP/s")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured into a HIP graph instead of eager launches")
    ap.add_argument("--graph-layers", type=int, default=0,
                    help="time N decode steps, each on its own layer's caches (as one decode pass of an N-layer "
                         "model), captured into one HIP graph, against the same N steps launched eagerly; "
                         "prints its own JSON line")
    ap.add_argument("--comparators", action="store_true",
                    help="also time a PyTorch gather-and-mask decode on the same inputs (benchmark only)")
    ap.add_argument("--no-records", action="store_true",
                    help="default run without the records of the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-timings", action="store_true",
                    help="skip the per-call and per-mode timings (profiled runs: only the timed steps launch)")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0,
                    help="target seconds of oracle work for the headline workload (3 s for each record)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/decode_<workload>_traffic.txt from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, then WRITE_SIZE) of this script, then exit")
    ap.add_argument("--pmc-commands", nargs=2, metavar=("FETCH_CMD", "WRITE_CMD"), default=("", ""),
                    help="the two profiling commands, recorded in the summary")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write profiles/decode_<workload>_kernel_trace.txt from a rocprofv3 --kernel-trace "
                         "--stats run of this script, then exit")
    ap.add_argument("--trace-command", default="", help="the profiling command, recorded in the summary")
    ap.add_argument("--summarize-latency", nargs="+", metavar="PMC_DIR",
                    help="write profiles/decode_<workload>_memory_latency.txt from rocprofv3 --pmc runs of "
                         "TCC/TCP/TA/GRBM counters (read latency and reads in flight), then exit")
    ap.add_argument("--summarize-graph-trace", metavar="TRACE_DIR",
                    help="write profiles/graph_layers_<workload>_kernel_gaps.txt from a rocprofv3 --kernel-trace "
                         "run of --graph-layers (per-pass span, busy time and gaps), then exit")
    ap.add_argument("--summarize-sq", nargs="+", metavar="PMC_DIR",
                    help="write profiles/<kernel>_<workload>_sq_counters.txt from rocprofv3 --pmc runs of SQ_ "
                         "counters (the attention kernel, or the prefill kernel with --prefill), then exit")
    ap.add_argument("--sq-commands", nargs="*", default=[], help="the profiling commands, recorded in the summary")
    args = ap.parse_args()
    args.workload_given = args.workload is not None
    return args


class TimingEvent:
    """A HIP event for timing only, recorded without the system-scope fence.

    torch.cuda.Event's default HIP event writes back and invalidates the caches when it is
    recorded, which on MI355X adds about 11 us to a 240 us decode step and slows the work after
    it. hipEventDisableSystemFence drops that fence; the HIP headers name timing as its use.
    Elapsed times are read only after a device synchronisation. Same interface as the
    torch.cuda.Event calls used here: record(stream), elapsed_time(end), cuda_event.
    """
    _hip = None
    _DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        handle = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(handle), self._DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = handle.value

    def record(self, stream=None):
        import torch
        s = torch.cuda.current_stream() if stream is None else stream
        rc = TimingEvent._hip.hipEventRecord(self.cuda_event, s.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        hip = getattr(type(self), "_hip", None)  # None once the interpreter is tearing down
        if hip is not None and getattr(self, "cuda_event", None):
            hip.hipEventDestroy(self.cuda_event)


def kernel_source_sha(kernel: str = "decode") -> str:
    """sha256 of the source file that holds `kernel` ("decode" or "prefill")."""
    src = KERNEL_SOURCE.with_name(f"{kernel}.hip")
    return hashlib.sha256(src.read_bytes()).hexdigest()


def profile_name(workload: str, shared_prefix: bool = False, fused_step: bool = False) -> str:
    """Workload part of a profile file name (runs with the shared-prefix option or the fused step
    are kept apart)."""
    return workload + ("_shared_prefix" if shared_prefix else "") + ("_fused_step" if fused_step else "")


def traffic_from_profiles(workload: str, launches_bytes: float):
    """HBM bytes per launch of the attention kernel from committed counter summaries, or None."""
    path = PROFILES / f"decode_{workload}_traffic.txt"
    if not path.exists():
        return None
    fields = {}
    for line in path.read_text().splitlines():
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _pmc_rows(directory: str, counter: str):
    import csv
    files = sorted(Path(directory).rglob("*counter_collection.csv"))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize_pmc(workload: str, fetch_dir: str, write_dir: str, commands, shared_prefix: bool = False) -> Path:
    """HBM bytes per attention-kernel launch, with FETCH/WRITE_SIZE scaled by a copy of known size."""
    out = {}
    for key, directory, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _pmc_rows(directory, counter)
        dec = [v for n, v in rows if "decode_kernel" in n]
        # the largest copy kernel in the run is the device-to-device copy of COPY_BYTES
        cpy = [v for n, v in rows if "copy" in n.lower()]
        if not dec or not cpy:
            raise SystemExit(f"{counter}: decode or copy kernel missing in {directory}")
        out[key] = (sum(dec) / len(dec), max(cpy), len(dec))
    known_kib = COPY_BYTES / 1024.0
    f_fetch = known_kib / out["fetch"][1]
    f_write = known_kib / out["write"][1]
    fetch_b = out["fetch"][0] * f_fetch * 1024.0
    write_b = out["write"][0] * f_write * 1024.0
    path = PROFILES / f"decode_{profile_name(workload, shared_prefix)}_traffic.txt"
    PROFILES.mkdir(exist_ok=True)
    opt = " --shared-prefix" if shared_prefix else ""
    path.write_text("\n".join([
        f"# HBM traffic of the attention kernel (decode_kernel) on workload {workload}{opt}",
        "# from two rocprofv3 --pmc runs of bench.py; FETCH_SIZE / WRITE_SIZE are KiB per dispatch,",
        f"# scaled by the same counter on a plain {COPY_BYTES >> 20} MiB copy kernel in the same run",
        f"# fetch command: {commands[0]}",
        f"# write command: {commands[1]}",
        f"# summary command: python bench.py --workload {workload}{opt} --summarize-pmc {fetch_dir} {write_dir}",
        f"kernel_source_sha256: {kernel_source_sha()}",
        f"decode_dispatches: {out['fetch'][2]}",
        f"fetch_kib_per_dispatch_raw: {out['fetch'][0]:.1f}",
        f"write_kib_per_dispatch_raw: {out['write'][0]:.1f}",
        f"copy_fetch_kib_raw: {out['fetch'][1]:.1f}",
        f"copy_write_kib_raw: {out['write'][1]:.1f}",
        f"copy_factor_fetch: {f_fetch:.4f}",
        f"copy_factor_write: {f_write:.4f}",
        f"hbm_fetch_bytes_per_launch: {fetch_b:.0f}",
        f"hbm_write_bytes_per_launch: {write_b:.0f}",
        f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
    ]) + "\n")
    return path


def summarize_sq(workload: str, directories, commands, kernel: str = "decode") -> Path:
    """SQ counters of one kernel, summed over its dispatches in each --pmc run, with derived shares.

    Shares of SQ_WAVE_CYCLES are per wavefront: how much of its life a wavefront spent issuing
    VALU, waiting for an instruction to issue, or waiting on s_waitcnt / a barrier. The MFMA pipe
    busy fraction compares SQ_VALU_MFMA_BUSY_CYCLES with the kernel's SIMD-cycles, taken from the
    run's timestamps at the GPU's 2.4 GHz peak clock, so it is a lower bound."""
    import csv
    name = "prefill" if kernel == "prefill" else "decode_kernel"
    tot, disp, span = {}, {}, {}
    for d in directories:
        files = sorted(Path(d).rglob("*counter_collection.csv"))
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            for r in csv.DictReader(open(f)):
                if name not in r["Kernel_Name"]:
                    continue
                c = r["Counter_Name"]
                tot[c] = tot.get(c, 0.0) + float(r["Counter_Value"])
                disp.setdefault(c, set()).add(r["Dispatch_Id"])
                span[(d, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not tot:
        raise SystemExit(f"no {name} rows")
    lines = [f"# SQ counters of the {name} kernel on workload {workload}, summed over its dispatches",
             *[f"# command: {c}" for c in commands],
             f"# summary command: python bench.py --workload {workload} {'--prefill ' if kernel == 'prefill' else ''}"
             f"--summarize-sq {' '.join(directories)}",
             f"kernel_source_sha256: {kernel_source_sha('prefill' if kernel == 'prefill' else 'decode')}"]
    for c in sorted(tot):
        lines.append(f"{c}: {tot[c]:.6g} ({len(disp[c])} dispatches)")
    def per(c):
        return tot[c] / len(disp[c]) if c in tot else None
    wc = per("SQ_WAVE_CYCLES")
    if wc:
        for c, label in (("SQ_ACTIVE_INST_VALU", "issuing VALU (incl. MFMA)"), ("SQ_WAIT_INST_ANY", "waiting to issue"),
                         ("SQ_WAIT_ANY", "waiting on s_waitcnt or a barrier"), ("SQ_ACTIVE_INST_LDS", "issuing LDS")):
            if per(c) is not None:
                lines.append(f"share_of_wave_cycles {label}: {per(c) / wc:.3f}")
    if per("SQ_INSTS_VALU") and per("SQ_INSTS_MFMA"):
        lines.append(f"valu_instructions_per_mfma: {(per('SQ_INSTS_VALU') - per('SQ_INSTS_MFMA')) / per('SQ_INSTS_MFMA'):.2f}")
    if per("SQ_VALU_MFMA_BUSY_CYCLES") and span:
        mean_ns = sum(span.values()) / len(span)
        simd_cycles = mean_ns * 1e-9 * 2.4e9 * 1024
        lines.append(f"mfma_busy_fraction_at_2.4GHz: {per('SQ_VALU_MFMA_BUSY_CYCLES') / simd_cycles:.3f}")
    path = PROFILES / f"{'prefill' if kernel == 'prefill' else 'decode'}_{workload}_sq_counters.txt"
    PROFILES.mkdir(exist_ok=True)
    path.write_text("\n".join(lines) + "\n")
    return path


def _counter_totals(directories, kernel_substr: str):
    """Per counter: (sum over the kernel's dispatches, dispatch count), and the dispatches' mean duration."""
    import csv
    tot, disp, span = {}, {}, {}
    for d in directories:
        files = sorted(Path(d).rglob("*counter_collection.csv"))
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            for r in csv.DictReader(open(f)):
                if kernel_substr not in r["Kernel_Name"]:
                    continue
                c = r["Counter_Name"]
                tot[c] = tot.get(c, 0.0) + float(r["Counter_Value"])
                disp.setdefault(c, set()).add((d, r["Dispatch_Id"]))
                span[(d, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    per = {c: tot[c] / len(disp[c]) for c in tot}
    mean_ns = sum(span.values()) / len(span) if span else 0.0
    return tot, disp, per, mean_ns


def summarize_latency(workload: str, directories, commands) -> Path:
    """Memory-side view of the attention kernel: average L2->memory read latency (TCC EA read requests
    in flight summed per cycle / requests), average CU->L2 read latency, reads in flight, TA busy."""
    tot, disp, per, mean_ns = _counter_totals(directories, "decode_kernel")
    if not tot:
        raise SystemExit("no decode_kernel rows")
    lines = [f"# memory latency counters of the decode_kernel kernel on workload {workload}, per dispatch",
             *[f"# command: {c}" for c in commands],
             f"# summary command: python bench.py --workload {workload} --summarize-latency {' '.join(directories)}",
             f"kernel_source_sha256: {kernel_source_sha()}",
             f"dispatch_mean_us: {mean_ns / 1e3:.2f}"]
    for c in sorted(per):
        lines.append(f"{c}: {per[c]:.6g} (mean of {len(disp[c])} dispatches)")
    if per.get("TCC_EA0_RDREQ_sum") and per.get("TCC_EA0_RDREQ_LEVEL_sum") is not None:
        lat = per["TCC_EA0_RDREQ_LEVEL_sum"] / per["TCC_EA0_RDREQ_sum"]
        lines.append(f"l2_to_memory_read_latency_cycles: {lat:.0f}")
        if per.get("GRBM_GUI_ACTIVE"):
            lines.append(f"l2_to_memory_reads_in_flight_avg: {per['TCC_EA0_RDREQ_LEVEL_sum'] / per['GRBM_GUI_ACTIVE']:.0f}"
                         " (per GPU cycle of the dispatch)")
    if per.get("TCP_TCC_READ_REQ_sum") and per.get("TCP_TCC_READ_REQ_LATENCY_sum") is not None:
        lines.append(f"cu_to_l2_read_latency_cycles: {per['TCP_TCC_READ_REQ_LATENCY_sum'] / per['TCP_TCC_READ_REQ_sum']:.0f}")
    path = PROFILES / f"decode_{workload}_memory_latency.txt"
    PROFILES.mkdir(exist_ok=True)
    path.write_text("\n".join(lines) + "\n")
    return path


def summarize_graph_trace(workload: str, directory: str, command: str, layers: int, per_step: int) -> Path:
    """Passes of `layers` decode steps (per_step library kernels each) in launch order: span from the
    first kernel's start to the last one's end, summed kernel time, and the gaps between kernels."""
    import csv
    import numpy as np
    traces = sorted(Path(directory).rglob("*kernel_trace.csv"))
    if not traces:
        raise SystemExit(f"no kernel_trace.csv under {directory}")
    ks = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in csv.DictReader(open(traces[0]))
                if "pa::" in r["Kernel_Name"])
    n = layers * per_step
    # graph_layers_bench's launch order: warm-up eager passes, 3 graph replays, then synchronised eager
    # and graph passes, then back-to-back eager and graph passes (reps each)
    import re
    mw, ms = re.search(r"--warmup\s+(\d+)", command), re.search(r"--steps\s+(\d+)", command)
    warm = max(1, int(mw.group(1))) if mw else 10
    reps = max(3, int(ms.group(1))) if ms else 100
    kinds = (["eager warm-up"] * warm + ["graph first replays"] * 3 + ["eager synchronised"] * reps +
             ["graph synchronised"] * reps + ["eager back to back"] * reps + ["graph back to back"] * reps)
    lines = [f"# library kernels of --graph-layers {layers} on workload {workload}, grouped into passes of {n}",
             f"# kernels in launch order; the pass kinds follow the bench's fixed launch order",
             f"# command: {command}",
             f"# summary command: python bench.py --workload {workload} --graph-layers {layers} "
             f"--summarize-graph-trace {directory}",
             f"kernel_source_sha256: {kernel_source_sha()}",
             f"{'pass':>4} {'kind':<20} {'span_us':>9} {'busy_us':>9} {'gap_median_us':>13} {'gap_max_us':>10}"]
    by_kind = {}
    for p in range(len(ks) // n):
        seg = ks[p * n:(p + 1) * n]
        gaps = np.array([seg[i + 1][0] - seg[i][1] for i in range(n - 1)]) / 1e3
        kind = kinds[p] if p < len(kinds) else "?"
        span, busy = (seg[-1][1] - seg[0][0]) / 1e3, sum(e - s for s, e in seg) / 1e3
        by_kind.setdefault(kind, []).append((span, busy, float(np.median(gaps))))
        lines.append(f"{p:>4} {kind:<20} {span:>9.1f} {busy:>9.1f} {float(np.median(gaps)):>13.2f} "
                     f"{float(gaps.max()):>10.2f}")
    for kind, v in by_kind.items():
        a = np.array(v)
        lines.append(f"mean {kind}: span {a[:, 0].mean():.1f} us, busy {a[:, 1].mean():.1f} us, "
                     f"median gap {np.median(a[:, 2]):.2f} us; per layer step {a[:, 0].mean() / layers:.2f} us")
    path = PROFILES / f"graph_layers_{workload}_kernel_gaps.txt"
    PROFILES.mkdir(exist_ok=True)
    path.write_text("\n".join(lines) + "\n")
    return path


def summarize_trace(workload: str, directory: str, command: str, kernel: str = "decode",
                    shared_prefix: bool = False, fused_step: bool = False) -> Path:
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace --stats run, as text."""
    import csv
    files = sorted(Path(directory).rglob("*kernel_stats.csv"))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {directory}")
    opt = (" --shared-prefix" if shared_prefix else "") + (" --fused-step" if fused_step else "")
    lines = [f"# rocprofv3 kernel statistics, workload {workload}{opt}",
             f"# command: {command}",
             f"# summary command: python bench.py --workload {workload}{opt} "
             f"{'--prefill ' if kernel == 'prefill' else ''}--summarize-trace {directory}",
             f"kernel_source_sha256: {kernel_source_sha(kernel)}",
             f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in csv.DictReader(open(files[0])):
        name = r["Name"].replace("(anonymous namespace)::", "")
        name = name if len(name) <= 72 else name[:69] + "..."
        lines.append(f"{name:<72} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                     f"{float(r['Percentage']):>6.2f}")
    # The timed launches alone (the trace's average also counts the warm-up launches): the last
    # --steps launches of the main kernel, in start order.
    import re
    traces = sorted(Path(directory).rglob("*kernel_trace.csv"))
    m = re.search(r"--steps\s+(\d+)", command)
    main_name = "prefill" if kernel == "prefill" else "decode_kernel"
    if traces and m:
        launches = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                          for r in csv.DictReader(open(traces[0])) if main_name in r["Kernel_Name"])
        timed = [d for _, d in launches][-int(m.group(1)):]
        if timed:
            lines.append(f"timed_launches: {len(timed)} (the last --steps launches of the {main_name} kernel)")
            lines.append(f"timed_launches_mean_us: {sum(timed) / len(timed) / 1e3:.2f}")
    path = PROFILES / f"{kernel}_{profile_name(workload, shared_prefix, fused_step)}_kernel_trace.txt"
    PROFILES.mkdir(exist_ok=True)
    path.write_text("\n".join(lines) + "\n")
    return path


def torch_gather_mask_decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_len):
    """Comparator: batched gather through the block tables, masked softmax, in PyTorch (fp32 math).

    The vectorised baseline of the decode benchmark the pages describe (hysenlabs MinivLLM
    review, end of the prefilling-baseline section): gather every sequence's blocks into a
    padded tensor, mask positions past the context, softmax, weighted sum. Used only to time
    it beside the library; never part of the product path.
    """
    import torch
    b, hq, d = q.shape
    nb, hkv, _, bs, x = k_cache.shape
    g = hq // hkv
    mb = -(-max_len // bs)
    tables = block_tables[:, :mb].long()
    # logical [B, Hkv, T, D] views of the gathered pages
    k = k_cache[tables]                                   # [B, MB, Hkv, D/x, bs, x]
    k = k.permute(0, 2, 1, 4, 3, 5).reshape(b, hkv, mb * bs, d).float()
    v = v_cache[tables]                                   # [B, MB, Hkv, bs/4, D, 4]
    v = v.permute(0, 2, 1, 3, 5, 4).reshape(b, hkv, mb * bs, d).float()
    qf = q.float().reshape(b, hkv, g, d)
    scores = torch.matmul(qf, k.transpose(-1, -2).contiguous()) * scale      # [B, Hkv, G, T]
    pos = torch.arange(mb * bs, device=q.device)
    scores = scores.masked_fill(pos[None, None, None, :] >= context_lens[:, None, None, None], float("-inf"))
    w = torch.softmax(scores, dim=-1)
    return torch.matmul(w, v).reshape(b, hq, d)


def describe(cfg) -> dict:
    lens = {"list": f"{list(cfg.len_list)}", "fixed": f"all {cfg.len_hi}",
            "uniform": f"uniform [{cfg.len_lo}, {cfg.len_hi}]",
            "lognormal": f"lognormal median {cfg.len_median:g} sigma {cfg.len_sigma:g} clipped [{cfg.len_lo}, {cfg.len_hi}]"}
    d = {"workload": cfg.name, "batch": cfg.batch, "num_heads": cfg.num_heads, "num_kv_heads": cfg.num_kv_heads,
         "head_dim": cfg.head_dim, "block_size": cfg.block_size, "context_lens": lens[cfg.lengths],
         "scale": cfg.softmax_scale}
    if cfg.prefix_group:
        d["prefix_sharing"] = f"groups of {cfg.prefix_group} sequences share their first {cfg.prefix_tokens} tokens"
    if cfg.q_mult != 1.0:
        d["q_scale"] = cfg.q_mult
    return d


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it, with its family and model numbers (virtual machines
    often report a generic name) and the logical CPUs the system has."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (t.strip() for t in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "vendor_id") and k not in fields:
                    fields[k] = v
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    extra = [f"{k} {fields[k]}" for k in ("vendor_id", "cpu family", "model") if k in fields]
    extra.append(f"{os.cpu_count()} logical CPUs")
    return f"{name} ({', '.join(extra)})"


def cpu_baseline(x, gpu_out, budget_s: float, one_thread_budget_s: float = 0.0) -> dict:
    """Time the float64 oracle on a bounded sample of the batch and compare it with the GPU output.

    Sequences are taken one at a time in a seeded order until the budget is spent or the batch
    is done. With one_thread_budget_s > 0 the same is repeated with the BLAS pool limited to one
    thread."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    c = x.cfg
    geo = oracle.CacheGeometry(x.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.dtype)
    k2, v2 = oracle.store_kvcache(x.k_new, x.v_new, x.slot_mapping, x.k_cache, x.v_cache, geo)
    ref = np.zeros((c.batch, c.num_heads, c.head_dim))

    def timed(budget):
        order = np.random.default_rng(12345).permutation(c.batch).tolist()
        seqs, tokens, dt = [], 0, 0.0
        while order and dt < budget:
            s = order.pop(0)
            t = time.perf_counter()
            part = oracle.decode(x.q, k2, v2, x.block_tables, x.context_lens, x.scale, geo, seqs=[s])
            dt += time.perf_counter() - t
            ref[s] = part[s]
            seqs.append(s)
            tokens += int(x.context_lens[s])
        return seqs, tokens, dt

    seqs, tokens, dt = timed(budget_s)
    kv = tokens * c.num_kv_heads * c.head_dim * c.elem_bytes * 2
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    err = float(np.abs(gpu_out[seqs] - ref[seqs]).max())
    res = {"value": kv / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{len(seqs)} of {c.batch} sequences ({tokens} context tokens) after the step's scatter, "
                     f"float64 numpy, one sequence per call",
           "seconds": dt, "tokens_per_s": len(seqs) / dt, "host_cpus": len(os.sched_getaffinity(0)),
           "cpu_model": cpu_model(), "parity_max_abs_err_vs_gpu": err}
    if one_thread_budget_s > 0:
        with threadpool_limits(limits=1):
            seqs1, tokens1, dt1 = timed(one_thread_budget_s)
        kv1 = tokens1 * c.num_kv_heads * c.head_dim * c.elem_bytes * 2
        res["one_thread"] = {"value": kv1 / dt1 / 1e9, "unit": "GB/s", "cores": 1, "seconds": dt1,
                             "sample": f"{len(seqs1)} of {c.batch} sequences ({tokens1} context tokens)",
                             "tokens_per_s": len(seqs1) / dt1}
    return res


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}


def _pcts(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"p10_us": round(float(np.percentile(a, 10)), 2), "median_us": round(float(np.median(a)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2)}


def extra_timings(calls: dict, reps: int) -> dict:
    """Per-call event timings (p10 / median / p90) of each callable, measured back to back."""
    import torch
    out = {}
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        evs = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
        for b, e in evs:
            b.record()
            fn()
            e.record()
        torch.cuda.synchronize()
        out[name] = _pcts([b.elapsed_time(e) for b, e in evs])
    return out


class StreamRead:
    """The streaming-read kernel of libpa_stream_read.so (measurement only) over one buffer."""

    BYTES = (1 << 31) - (1 << 14)

    def __init__(self, dev):
        import ctypes
        import torch
        lib_path = ROOT / "paged_attention_decode_amd" / "libpa_stream_read.so"
        if not lib_path.exists():
            raise RuntimeError(f"{lib_path} is not built: run `python -m paged_attention_decode_amd.build`")
        self.lib = ctypes.CDLL(str(lib_path))
        self.lib.pa_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        self.lib.pa_bench_stream_read.restype = ctypes.c_int
        self.cus = torch.cuda.get_device_properties(dev).multi_processor_count
        self.buf = torch.empty(self.BYTES, dtype=torch.uint8, device=dev)
        self.sink = torch.empty(self.cus * 16 * 4 * 64, dtype=torch.int32, device=dev)
        self.dev = dev
        self.ceiling_gbs = None  # best rate of ceiling(), once measured
        self.best = None

    def read(self, nbytes, policy=0, unroll=8, groups_per_cu=4):
        import torch
        grid = self.cus * groups_per_cu
        assert grid * 4 * 64 <= self.sink.numel() and nbytes <= self.BYTES
        rc = self.lib.pa_bench_stream_read(self.buf.data_ptr(), nbytes, policy, unroll, grid, self.sink.data_ptr(),
                                           torch.cuda.current_stream(self.dev).cuda_stream)
        if rc != 0:
            raise RuntimeError(f"pa_bench_stream_read failed ({rc})")

    def flush(self):
        """Read 1 GiB with the default policy: afterwards the L2s and the last-level cache hold none
        of the benchmark's K/V (reads leave no dirty lines to write back during the next step)."""
        self.read(1 << 30, 0, 8, 4)

    def same_bytes(self, nbytes: int, reps: int = 10) -> dict:
        """Cold read of as many bytes as a workload's K/V (rounded down to 16 KiB), with the best
        setting of ceiling(): the practical ceiling at that size, launch ramp and tail included."""
        import torch
        n = max(1 << 14, min(self.BYTES, nbytes) // (1 << 14) * (1 << 14))
        b = self.best or {"policy": "nt", "unroll": 8, "groups_per_cu": 4}
        pol = 1 if b["policy"] == "nt" else 0
        self.read(n, pol, b["unroll"], b["groups_per_cu"])
        ms = []
        for _ in range(reps):
            self.flush()
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record()
            self.read(n, pol, b["unroll"], b["groups_per_cu"])
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        med = sorted(ms)[len(ms) // 2]
        return {"bytes": n, "median_us": round(med * 1e3, 2), "gbs": round(n / (med * 1e-3) / 1e9, 1),
                "setting": b, "what": "cold (after a 1 GiB read), median of " + str(reps)}

    def ceiling(self, reps: int = 5) -> dict:
        """Best rate over a small sweep of loads in flight and occupancy, per cache policy."""
        import torch
        rows = []
        for policy in (0, 1):
            for unroll in (8, 16):
                for gpc in (2, 4, 8):
                    self.read(self.BYTES, policy, unroll, gpc)
                    torch.cuda.synchronize()
                    evs = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
                    for b, e in evs:
                        b.record()
                        self.read(self.BYTES, policy, unroll, gpc)
                        e.record()
                    torch.cuda.synchronize()
                    best = min(b.elapsed_time(e) for b, e in evs)
                    rows.append({"policy": "nt" if policy else "default", "unroll": unroll, "groups_per_cu": gpc,
                                 "gbs": round(self.BYTES / (best * 1e-3) / 1e9, 1)})
        top = max(rows, key=lambda r: r["gbs"])
        self.best = top
        by_pol = {p: max(r["gbs"] for r in rows if r["policy"] == p) for p in ("default", "nt")}
        return {"gbs": top["gbs"], "best": top, "best_default_policy_gbs": by_pol["default"],
                "best_nt_policy_gbs": by_pol["nt"], "bytes": self.BYTES,
                "what": "pa_bench_stream_read: 16-byte buffer loads, 1 KiB per wavefront load instruction, "
                        f"one pass over {self.BYTES} bytes, best of {reps} per setting", "sweep": rows}


def prefill_useful_flops(head_dim: int, num_heads: int, new_tokens, context_lens) -> float:
    """Useful flops of a causal paged prefill: 4*D*Hq per visible (query, key) pair. A sequence
    with n new tokens among L sees n*L - n(n-1)/2 pairs (query i, at position L-n+i, sees
    L-n+i+1 keys)."""
    import numpy as np
    n = np.asarray(new_tokens, dtype=np.float64)
    L = np.asarray(context_lens, dtype=np.float64)
    return 4.0 * head_dim * num_heads * float(np.sum(n * L - n * (n - 1) / 2))


def prefill_bench(args) -> None:
    """Full-prompt causal prefill over the workload's paged caches, as its own JSON line."""
    print(json.dumps(measure_prefill(args.workload, args.steps, args.warmup)), flush=True)


class MfmaCeiling:
    """The matrix-core loop of libpa_stream_read.so (measurement only): eight independent chains of
    one matrix-core instruction kind per wavefront, nothing else, two workgroups of four
    wavefronts on every compute unit (two wavefronts per SIMD, as the prefill kernels run)."""

    KINDS = {"bf16": (0, "v_mfma_f32_16x16x32_bf16", 16384), "fp16": (1, "v_mfma_f32_16x16x32_f16", 16384),
             "bf16_16x16x16": (2, "v_mfma_f32_16x16x16_bf16", 8192)}

    def __init__(self, dev):
        import ctypes
        import torch
        lib_path = ROOT / "paged_attention_decode_amd" / "libpa_stream_read.so"
        if not lib_path.exists():
            raise RuntimeError(f"{lib_path} is not built: run `python -m paged_attention_decode_amd.build`")
        self.lib = ctypes.CDLL(str(lib_path))
        self.lib.pa_bench_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p]
        self.lib.pa_bench_mfma.restype = ctypes.c_int
        self.cus = torch.cuda.get_device_properties(dev).multi_processor_count
        self.dev = dev

    def measure(self, kind: str, iters: int = 16000, reps: int = 5) -> dict:
        """Best rate over `reps` launches of 2 * cus workgroups, each asking for 64 KiB of LDS so
        that a compute unit holds exactly two."""
        import torch
        k, name, flops_each = self.KINDS[kind]
        grid = self.cus * 2
        sink = torch.empty(grid * 256, dtype=torch.float32, device=self.dev)
        stream = torch.cuda.current_stream(self.dev).cuda_stream

        def launch():
            if self.lib.pa_bench_mfma(k, iters, grid, 65536, sink.data_ptr(), stream) != 0:
                raise RuntimeError("pa_bench_mfma failed")

        launch()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        flops = float(grid) * 4 * 8 * iters * flops_each
        return {"instruction": name, "waves_per_simd": 2, "tflops": round(flops / (best * 1e-3) / 1e12, 1),
                "ms": round(best, 4), "what": f"best of {reps} launches of the matrix-core loop"}


def measure_prefill(workload: str, steps: int, warmup: int) -> dict:
    """Full-prompt causal prefill over the workload's paged caches; useful flops = 4*D*Hq*sum(n*L - n(n-1)/2)."""
    import numpy as np
    import torch

    import paged_attention_decode_amd as pa
    from workloads import get_config, make_inputs, to_storage

    dev = torch.device("cuda:0")
    cfg = get_config(workload)
    print(f"[bench] prefill: generating {cfg.name}", file=sys.stderr, flush=True)
    x = make_inputs(cfg)
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]

    def up(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    k_cache = up(x.k_cache).view(pa.k_cache_shape(x.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.block_size, tdt))
    v_cache = up(x.v_cache).view(pa.v_cache_shape(x.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.block_size))
    lens = x.context_lens.astype(np.int64)
    qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = up(to_storage(np.random.default_rng(7).standard_normal((int(qs[-1]), cfg.num_heads, cfg.head_dim),
                                                                dtype=np.float32), cfg.dtype))
    bt = torch.from_numpy(x.block_tables).to(dev)
    cl = torch.from_numpy(x.context_lens).to(dev)
    qst = torch.from_numpy(qs).to(dev)
    out = torch.empty((int(qs[-1]), cfg.num_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    flops = prefill_useful_flops(cfg.head_dim, cfg.num_heads, lens, lens)
    for _ in range(max(1, warmup)):
        pa.paged_prefill(q, k_cache, v_cache, bt, cl, qst, x.scale, out)
    torch.cuda.synchronize()
    ev = [TimingEvent() for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(steps):
        pa.paged_prefill(q, k_cache, v_cache, bt, cl, qst, x.scale, out)
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / steps
    tflops = flops / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    ceiling = None
    if cfg.dtype in MfmaCeiling.KINDS:
        ceiling = MfmaCeiling(dev).measure(cfg.dtype)
        ceiling["prefill_frac_of_ceiling"] = round(tflops / ceiling["tflops"], 4)
    return {
        "metric": "paged prefill TFLOP/s (causal, full prompts)", "value": round(tflops, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded, shapes of the workload)",
        "config": dict(describe(cfg), prompt_tokens=int(qs[-1]), useful_flops=flops),
        "tokens_per_s": round(float(qs[-1]) / (ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "kernel": ("prefill_shared_kernel (workgroup-shared K/V)"
                                if cfg.dtype != "fp32" and cfg.head_dim == 128 else "prefill_kernel (per wavefront)"),
                     "kernel_mean_ms": round(ms, 5), "mfma_ceiling": ceiling}}


def _upload(a, dtype, dev):
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _stats_us(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"mean_us": round(float(a.mean()), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "median_us": round(float(np.median(a)), 2), "p90_us": round(float(np.percentile(a, 90)), 2)}


def measure_workload(name: str, args, dev, sr: "StreamRead", headline: bool) -> dict:
    """Time the decode step of one workload: a warm loop of K steps (wall clock and per-launch events
    of the attention kernel), then K cold steps, each after a 1 GiB read (outside the events), with
    events around the store, the attention kernel and the whole step. The roofline is taken on the
    cold attention-kernel launches."""
    import numpy as np
    import torch

    import paged_attention_decode_amd as pa
    from workloads import get_config, make_inputs

    cfg = get_config(name)
    psize = args.partition_size if args.partition_size is not None else WORKLOAD_PARTITION.get(name, 0)
    cpt = args.cached_prefix_tokens if args.cached_prefix_tokens is not None else WORKLOAD_CACHED_PREFIX.get(name, 0)
    print(f"[bench] {name}: generating", file=sys.stderr, flush=True)
    x = make_inputs(cfg)
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    k_cache = _upload(x.k_cache, cfg.dtype, dev).view(
        pa.k_cache_shape(x.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.block_size, tdt))
    v_cache = _upload(x.v_cache, cfg.dtype, dev).view(
        pa.v_cache_shape(x.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.block_size))
    q, k_new, v_new = (_upload(a, cfg.dtype, dev) for a in (x.q, x.k_new, x.v_new))
    block_tables = torch.from_numpy(x.block_tables).to(dev)
    context_lens = torch.from_numpy(x.context_lens).to(dev)
    slots = torch.from_numpy(x.slot_mapping).to(dev)
    out = torch.empty((cfg.batch, cfg.num_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def store():
        pa.store_kvcache(k_new, v_new, slots, k_cache, v_cache)

    def decode(events=None, psz=psize, shared=args.shared_prefix, cpt_=cpt):
        pa.paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, x.scale, out,
                                  partition_size=psz, cached_prefix_tokens=cpt_,
                                  events=events, shared_prefix=shared)

    def step(events=None):
        if args.fused_step:
            pa.decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, x.scale, out,
                           partition_size=psize, cached_prefix_tokens=cpt,
                           events=events, shared_prefix=args.shared_prefix)
            return
        store()
        decode(events)

    if headline:
        # A plain copy of known size (COPY_BYTES read + written): counter runs scale HBM bytes by it.
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The first call allocates the library's workspace; warm-up keeps that out of the timed region.
    print(f"[bench] {name}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    K = args.steps
    kev = [(TimingEvent(), TimingEvent()) for _ in range(K)]
    cev = [[TimingEvent() for _ in range(5)] for _ in range(K)]
    for e in kev + [tuple(c) for c in cev]:  # materialise the HIP events outside the timed region
        for ev in e:
            ev.record(stream)
    torch.cuda.synchronize()

    # Warm loop (the whole-job figure): K steps back to back, wall clock around them.
    print(f"[bench] {name}: timing {K} steps", file=sys.stderr, flush=True)
    if args.graph:
        # One step captured into a HIP graph and replayed K times. Events recorded inside a
        # captured graph do not bracket the kernel, so the attention kernel is timed by an
        # eager loop with library-recorded events afterwards (outside the timed region).
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for i in range(K):
            step(kev[i])
        torch.cuda.synchronize()
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(kev[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    warm_kernel_ms = [b.elapsed_time(e) for b, e in kev]

    # Cold loop: each step after a 1 GiB read, so no K/V is in the L2s or the last-level cache.
    # Events: c0 step start, c1 after the store, (c2, c3) the attention kernel, c4 step end.
    print(f"[bench] {name}: timing {K} cold steps", file=sys.stderr, flush=True)
    for i in range(K):
        sr.flush()
        c = cev[i]
        c[0].record(stream)
        if args.fused_step:
            step((c[2], c[3]))
            c[1] = c[0]
        else:
            store()
            c[1].record(stream)
            decode((c[2], c[3]))
        c[4].record(stream)
    torch.cuda.synchronize()
    cold_kernel_ms = [c[2].elapsed_time(c[3]) for c in cev]
    cold_step_ms = [c[0].elapsed_time(c[4]) for c in cev]
    cold_store_ms = [c[0].elapsed_time(c[1]) for c in cev]
    cold_decode_ms = [c[1].elapsed_time(c[4]) for c in cev]
    gpu_out = out.cpu().numpy()
    same = sr.same_bytes(x.unique_kv_bytes if args.shared_prefix else x.kv_bytes) if sr.best else None
    # A workload specified with its own launch mode is also timed, cold, in the library's automatic one.
    auto_cold_ms = None
    if psize != 0 and not args.no_extra_timings:
        evs = [(TimingEvent(), TimingEvent()) for _ in range(K)]
        for e in evs:
            sr.flush()
            decode(e, 0)
        torch.cuda.synchronize()
        auto_cold_ms = [b.elapsed_time(e) for b, e in evs]

    # A workload specified with its shared-prefix length is also timed, cold, with the library's
    # default cache policy.
    default_policy_cold_ms = None
    if cpt != 0 and not args.no_extra_timings:
        evs = [(TimingEvent(), TimingEvent()) for _ in range(K)]
        for e in evs:
            sr.flush()
            decode(e, psize, args.shared_prefix, 0)
        torch.cuda.synchronize()
        default_policy_cold_ms = [b.elapsed_time(e) for b, e in evs]

    ms_per_step = wall * 1e3 / K
    kv_bytes = x.kv_bytes
    # With shared prefixes the kernel reads each shared block once: its algorithmic bytes are the
    # distinct ones, and the roofline is taken on those.
    roof_bytes = x.unique_kv_bytes if args.shared_prefix else kv_bytes
    cold_mean = float(np.mean(cold_kernel_ms))
    warm_mean = float(np.mean(warm_kernel_ms))
    achieved = roof_bytes / (cold_mean * 1e-3) / 1e9
    warm_achieved = roof_bytes / (warm_mean * 1e-3) / 1e9
    cold_step_median = float(np.median(cold_step_ms))
    plan = pa.decode_plan(cfg.batch, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size,
                          int(x.block_tables.shape[1]), {"fp32": 0, "fp16": 1, "bf16": 2}[cfg.dtype], psize, 0,
                          shared_prefix=args.shared_prefix)
    rec = {
        "config": dict(describe(cfg), kv_bytes_per_step=kv_bytes, unique_kv_bytes=x.unique_kv_bytes,
                       partition_size=psize, plan_range_tokens=plan["range_tokens"],
                       merge_kernel=plan["uses_reduce"], shared_prefix=bool(args.shared_prefix),
                       cached_prefix_tokens=cpt or pa.DEFAULT_CACHED_PREFIX_TOKENS,
                       launch="hip graph replay" if args.graph else "eager",
                       step="pa_decode_step (fused scatter + attention)" if args.fused_step
                       else "pa_store_kvcache + pa_paged_attention_decode"),
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(cfg.batch / (ms_per_step * 1e-3), 1),
        "cold_step": dict(_stats_us(cold_step_ms),
                          kv_gbs=round(kv_bytes / (cold_step_median * 1e-3) / 1e9, 2),
                          tokens_per_s=round(cfg.batch / (cold_step_median * 1e-3), 1),
                          note="events around each cold step (store, attention, merge); the events' own "
                               "recording adds a few us per step on small workloads"),
        "split_cold_median_us": {
            "store": round(float(np.median(cold_store_ms)) * 1e3, 2),
            "attention_kernel": round(float(np.median(cold_kernel_ms)) * 1e3, 2),
            "merge_and_launch_gaps": round((float(np.median(cold_decode_ms)) -
                                            float(np.median(cold_kernel_ms))) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles(profile_name(name, args.shared_prefix, args.fused_step), kv_bytes),
                     "bytes": "distinct K/V bytes (shared blocks once)" if args.shared_prefix else "logical K/V bytes",
                     "algorithmic_bytes_per_launch": roof_bytes,
                     "kernel": "decode_kernel (attention; excludes store and merge; with the shared-prefix option "
                               "also its detection kernel)",
                     "timing": "cold: mean of the K attention-kernel launches of the cold loop (HIP events on the "
                               "library's stream), each after a 1 GiB read",
                     "kernel_mean_ms": round(cold_mean, 5),
                     "kernel_median_ms": round(float(np.median(cold_kernel_ms)), 5),
                     "frac_of_stream_read": round(achieved / sr.ceiling_gbs, 4) if sr.ceiling_gbs else None,
                     "stream_read_same_bytes": same,
                     "time_frac_of_stream_read_same_bytes":
                         round(same["median_us"] / (cold_mean * 1e3), 4) if same else None,
                     "warm": {"achieved": round(warm_achieved, 2), "frac": round(warm_achieved / HBM_PEAK_GBS, 4),
                              "kernel_mean_ms": round(warm_mean, 5),
                              "note": "back-to-back launches of the warm loop: cache-assisted where the K/V "
                                      "or part of it fits the 256 MB last-level cache"},
                     "achieved_on_unique_bytes": round(x.unique_kv_bytes / (cold_mean * 1e-3) / 1e9, 2)},
    }
    if auto_cold_ms:
        am = float(np.mean(auto_cold_ms))
        rec["roofline"]["automatic_mode"] = {
            "partition_size": 0, "range_tokens": pa.decode_plan(
                cfg.batch, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size, int(x.block_tables.shape[1]),
                {"fp32": 0, "fp16": 1, "bf16": 2}[cfg.dtype], 0, 0)["range_tokens"],
            "kernel_mean_ms": round(am, 5), "achieved": round(roof_bytes / (am * 1e-3) / 1e9, 2),
            "frac": round(roof_bytes / (am * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "the library's own choice for this batch (0 = automatic), cold, attention kernel only"}
    if default_policy_cold_ms:
        dm = float(np.mean(default_policy_cold_ms))
        rec["roofline"]["library_default_cache_policy"] = {
            "cached_prefix_tokens": pa.DEFAULT_CACHED_PREFIX_TOKENS, "kernel_mean_ms": round(dm, 5),
            "achieved": round(roof_bytes / (dm * 1e-3) / 1e9, 2),
            "frac": round(roof_bytes / (dm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "the same launch with the library's default cache policy (no hit length passed), cold, "
                    "attention kernel only"}
    if not args.fused_step and not args.graph and not args.no_extra_timings:
        # The library's fused step (pa_decode_step: the scatter done inside the attention launch)
        # on the same inputs, timed as `value` is: a warm loop of K steps, wall clock around them.
        # It writes the same bits to the same slots, so the inputs are unchanged afterwards.
        def fused():
            pa.decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, x.scale, out,
                           partition_size=psize, cached_prefix_tokens=cpt,
                           shared_prefix=args.shared_prefix)
        for _ in range(max(1, args.warmup)):
            fused()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            fused()
        torch.cuda.synchronize()
        fms = (time.perf_counter() - t0) * 1e3 / K
        rec["fused_step"] = {"ms_per_step": round(fms, 5), "value": round(kv_bytes / (fms * 1e-3) / 1e9, 2),
                             "tokens_per_s": round(cfg.batch / (fms * 1e-3), 1),
                             "note": "pa_decode_step, warm loop of the same step count, wall clock (as value)"}
    if headline and not args.no_extra_timings:
        calls = {"store": store, "decode": decode, "store_plus_decode": step}
        for pz, nm in ((-2, "decode_balanced"), (-1, "decode_one_pass"), (512, "decode_split_512")):
            calls[nm] = (lambda pz=pz: decode(None, pz, False))
        calls["decode_balanced_shared_prefix"] = lambda: decode(None, -2, True)
        timings = extra_timings(calls, 20)
        timings["decode_tokens_per_s"] = round(cfg.batch / (timings["decode"]["median_us"] * 1e-6), 1)
        timings["note"] = ("event pairs per call on the current stream, back to back (warm caches); "
                           "decode includes the merge kernel where the plan splits")
        rec["timings"] = timings
    if args.comparators:
        print(f"[bench] {name}: comparator torch gather-and-mask", file=sys.stderr, flush=True)
        max_len = int(x.context_lens.max())
        ref = torch_gather_mask_decode(q, k_cache, v_cache, block_tables, context_lens, x.scale, max_len)
        torch.cuda.synchronize()
        reps = 3
        t0 = time.perf_counter()
        for _ in range(reps):
            torch_gather_mask_decode(q, k_cache, v_cache, block_tables, context_lens, x.scale, max_len)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / reps
        rec["comparators"] = {"torch_gather_mask": {
            "ms_per_decode": round(ms, 4), "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
            "speedup_of_library_kernel": round(ms / cold_mean, 2),
            "max_abs_diff_vs_library": float((ref - out).abs().max().item()),
            "note": "decode only (no store), fp32 math, padded to the longest context"}}
        del ref
    if not args.no_cpu_baseline:
        print(f"[bench] {name}: cpu baseline (oracle)", file=sys.stderr, flush=True)
        budget = args.cpu_budget_s if headline else min(args.cpu_budget_s, 3.0)
        one = 3.0 if name in ONE_THREAD_BASELINE else 0.0
        rec["cpu_baseline"] = cpu_baseline(x, gpu_out, budget, one)
    del k_cache, v_cache, q, k_new, v_new, block_tables, context_lens, slots, out
    torch.cuda.empty_cache()
    return rec


def graph_layers_bench(args) -> None:
    """N decode steps (store + attention (+ merge)) on N layers' own caches: eager launches against one
    captured HIP graph replayed. Per-step times are wall clock over the whole pass / N."""
    import numpy as np
    import torch

    import paged_attention_decode_amd as pa
    from workloads import get_config, make_inputs

    dev = torch.device("cuda:0")
    cfg = get_config(args.workload)
    n = args.graph_layers
    psize = args.partition_size if args.partition_size is not None else WORKLOAD_PARTITION.get(cfg.name, 0)
    print(f"[bench] graph layers: generating {cfg.name}, {n} layers", file=sys.stderr, flush=True)
    x = make_inputs(cfg)
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    k0 = _upload(x.k_cache, cfg.dtype, dev).view(
        pa.k_cache_shape(x.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.block_size, tdt))
    v0 = _upload(x.v_cache, cfg.dtype, dev).view(
        pa.v_cache_shape(x.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.block_size))
    layers = []
    for _ in range(n):
        layers.append({"k_cache": k0.clone(), "v_cache": v0.clone(),
                       "q": _upload(x.q, cfg.dtype, dev), "k_new": _upload(x.k_new, cfg.dtype, dev),
                       "v_new": _upload(x.v_new, cfg.dtype, dev),
                       "out": torch.empty((cfg.batch, cfg.num_heads, cfg.head_dim), dtype=torch.float32,
                                          device=dev)})
    del k0, v0
    block_tables = torch.from_numpy(x.block_tables).to(dev)
    context_lens = torch.from_numpy(x.context_lens).to(dev)
    slots = torch.from_numpy(x.slot_mapping).to(dev)
    # the library's workspace, sized before capture (the graph records its address)
    ws_bytes = pa.workspace_bytes(cfg.batch, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size,
                                  int(x.block_tables.shape[1]), {"fp32": 0, "fp16": 1, "bf16": 2}[cfg.dtype], psize)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def one_pass():
        for L in layers:
            if args.fused_step:
                pa.decode_step(L["q"], L["k_new"], L["v_new"], L["k_cache"], L["v_cache"], block_tables,
                               context_lens, x.scale, L["out"], partition_size=psize, workspace=ws)
            else:
                pa.store_kvcache(L["k_new"], L["v_new"], slots, L["k_cache"], L["v_cache"])
                pa.paged_attention_decode(L["q"], L["k_cache"], L["v_cache"], block_tables, context_lens, x.scale,
                                          L["out"], partition_size=psize, workspace=ws)

    for _ in range(max(1, args.warmup)):
        one_pass()
    torch.cuda.synchronize()
    eager_ref = [L["out"].clone() for L in layers]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    same = all(bool(torch.equal(L["out"], r)) for L, r in zip(layers, eager_ref))

    def timed(fn, reps):
        walls = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t0)
        return float(np.median(walls))

    reps = max(3, args.steps)
    eager_s = timed(one_pass, reps)
    graph_s = timed(graph.replay, reps)
    # back to back, no synchronisation between passes: the steady state of a serving loop
    k = max(3, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(k):
        one_pass()
    torch.cuda.synchronize()
    eager_bb = (time.perf_counter() - t0) / k
    t0 = time.perf_counter()
    for _ in range(k):
        graph.replay()
    torch.cuda.synchronize()
    graph_bb = (time.perf_counter() - t0) / k
    kv = x.kv_bytes
    print(json.dumps({
        "metric": "decode step time in an N-layer pass, eager launches vs one captured HIP graph",
        "value": round(graph_bb / n * 1e6, 2), "unit": "us per layer step (graph, back to back)",
        "n_gpus": 1, "steps": reps, "warmup": args.warmup, "higher_is_better": False, "dtype": cfg.dtype,
        "config": dict(describe(cfg), layers=n, partition_size=psize,
                       step="pa_decode_step" if args.fused_step else "pa_store_kvcache + pa_paged_attention_decode"),
        "graph_replay_matches_eager_bitwise": same,
        "per_layer_step_us": {
            "eager_back_to_back": round(eager_bb / n * 1e6, 2), "graph_back_to_back": round(graph_bb / n * 1e6, 2),
            "eager_one_pass_synchronised": round(eager_s / n * 1e6, 2),
            "graph_one_pass_synchronised": round(graph_s / n * 1e6, 2)},
        "pass_us": {"eager_back_to_back": round(eager_bb * 1e6, 1), "graph_back_to_back": round(graph_bb * 1e6, 1)},
        "kv_gbs_graph": round(kv * n / graph_bb / 1e9, 1), "kv_gbs_eager": round(kv * n / eager_bb / 1e9, 1)}),
        flush=True)


def main():
    args = parse()
    workload = args.workload or DEFAULT_WORKLOAD
    if args.summarize_pmc:
        print(summarize_pmc(workload, args.summarize_pmc[0], args.summarize_pmc[1], args.pmc_commands,
                            args.shared_prefix))
        return
    if args.summarize_latency:
        print(summarize_latency(workload, args.summarize_latency, args.sq_commands))
        return
    if args.summarize_graph_trace:
        print(summarize_graph_trace(workload, args.summarize_graph_trace, args.trace_command, args.graph_layers,
                                    1 if args.fused_step else 2))
        return
    if args.summarize_sq:
        print(summarize_sq(workload, args.summarize_sq, args.sq_commands, "prefill" if args.prefill else "decode"))
        return
    if args.summarize_trace:
        print(summarize_trace(workload, args.summarize_trace, args.trace_command,
                              "prefill" if args.prefill else "decode", args.shared_prefix, args.fused_step))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the library "
              "has no cross-GPU step; each GPU would run its own shard of sequences or kv heads", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_attention_decode_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pa.load_library()
    args.workload = workload
    if args.prefill:
        prefill_bench(args)
        return
    if args.graph_layers > 0:
        graph_layers_bench(args)
        return
    dev = torch.device("cuda:0")
    sr = StreamRead(dev)
    ceiling = None
    if not args.no_extra_timings:
        print("[bench] streaming-read ceiling", file=sys.stderr, flush=True)
        ceiling = sr.ceiling()
        sr.ceiling_gbs = ceiling["gbs"]

    head = measure_workload(workload, args, dev, sr, headline=True)
    records = {}
    # Default run: the other workloads get records of their own in the same line.
    if args.workload_given is False and not args.no_records:
        for name in RECORD_WORKLOADS:
            if name != workload:
                records[name] = measure_workload(name, args, dev, sr, headline=False)

    result = {
        "metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": get_dtype(workload), "data": "synthetic (seeded, shapes of the workload)",
        "config": dict(head["config"], parallelism="single GPU"),
        "tokens_per_s": head["tokens_per_s"],
        "pct_hbm_peak": round(100.0 * head["value"] / HBM_PEAK_GBS, 2),
        "roofline": head["roofline"],
    }
    for key in ("cold_step", "split_cold_median_us", "fused_step", "timings", "comparators", "cpu_baseline"):
        if key in head:
            result[key] = head[key]
    if ceiling:
        result["stream_read_ceiling"] = ceiling
    if records:
        result["workloads"] = records
        # The next row's kernel (paged prefill), on the prompts of two workloads. The same step
        # counts as a --prefill run: with fewer warm-up launches after the host-side input
        # generation, the first timed launches run slower and the record understates the kernel.
        prefill = {}
        for name in PREFILL_RECORDS:
            print(f"[bench] prefill record {name}", file=sys.stderr, flush=True)
            r = measure_prefill(name, PREFILL_RECORD_STEPS, PREFILL_RECORD_WARMUP)
            prefill[name] = {"value": r["value"], "unit": r["unit"], "dtype": r["dtype"],
                             "ms_per_step": r["roofline"]["kernel_mean_ms"],
                             "prompt_tokens": r["config"]["prompt_tokens"], "roofline": r["roofline"]}
        result["prefill"] = prefill
    print(json.dumps(result), flush=True)


def get_dtype(name: str) -> str:
    from workloads import get_config
    return get_config(name).dtype


if __name__ == "__main__":
    main()
