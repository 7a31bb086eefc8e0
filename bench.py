#!/usr/bin/env python3
"""Decode-step benchmark for libpagedattn on one MI355X.

One step = the whole hot path over one batch: store_kvcache of the step's new
token per sequence, then paged_attention_decode (attention kernel plus, when
contexts are split, the merge kernel). Inputs are seeded synthetic data of the
workload's shape, resident in HBM before timing starts.

Prints ONE JSON line:
  value        KV GB/s: logical K+V bytes one decode must read (sum over
               sequences of L * Hkv * D * 2 bytes * 2) / wall time per step
  tokens_per_s sequences advanced per second (B / time per step)
  roofline     the attention kernel alone: the same KV bytes / its mean
               duration from HIP events recorded on its stream, against
               MI355X's 8 TB/s HBM peak; traffic from committed rocprofv3
               counter summaries when they match the current kernel source
  cpu_baseline the float64 CPU oracle timed on this host on a bounded sample
               of the same workload (a reported baseline, not the target)

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
KERNEL_SOURCE = ROOT / "paged_attention_decode_amd" / "csrc" / "decode.hip"
PROFILES = ROOT / "profiles"
COPY_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--partition-size", type=int, default=0,
                    help="0 automatic, -1 one pass, -2 balanced split, >0 fixed ranges of that many tokens")
    ap.add_argument("--cached-prefix-tokens", type=int, default=0,
                    help="leading tokens per context read with cached loads (0 library default, -1 none)")
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
    ap.add_argument("--comparators", action="store_true",
                    help="also time a PyTorch gather-and-mask decode on the same inputs (benchmark only)")
    ap.add_argument("--cold-steps", type=int, default=5, help="extra steps timed after a 1 GiB cache flush each")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-timings", action="store_true",
                    help="skip the per-call and per-mode timings (profiled runs: only the timed steps launch)")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0, help="target seconds of oracle work")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/decode_<workload>_traffic.txt from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, then WRITE_SIZE) of this script, then exit")
    ap.add_argument("--pmc-commands", nargs=2, metavar=("FETCH_CMD", "WRITE_CMD"), default=("", ""),
                    help="the two profiling commands, recorded in the summary")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write profiles/decode_<workload>_kernel_trace.txt from a rocprofv3 --kernel-trace "
                         "--stats run of this script, then exit")
    ap.add_argument("--trace-command", default="", help="the profiling command, recorded in the summary")
    ap.add_argument("--summarize-sq", nargs="+", metavar="PMC_DIR",
                    help="write profiles/<kernel>_<workload>_sq_counters.txt from rocprofv3 --pmc runs of SQ_ "
                         "counters (the attention kernel, or the prefill kernel with --prefill), then exit")
    ap.add_argument("--sq-commands", nargs="*", default=[], help="the profiling commands, recorded in the summary")
    return ap.parse_args()


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
        if TimingEvent._hip is not None and getattr(self, "cuda_event", None):
            TimingEvent._hip.hipEventDestroy(self.cuda_event)


def kernel_source_sha(kernel: str = "decode") -> str:
    """sha256 of the source file that holds `kernel` ("decode" or "prefill")."""
    src = KERNEL_SOURCE.with_name(f"{kernel}.hip")
    return hashlib.sha256(src.read_bytes()).hexdigest()


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


def summarize_pmc(workload: str, fetch_dir: str, write_dir: str, commands) -> Path:
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
    path = PROFILES / f"decode_{workload}_traffic.txt"
    PROFILES.mkdir(exist_ok=True)
    path.write_text("\n".join([
        f"# HBM traffic of the attention kernel (decode_kernel) on workload {workload}",
        "# from two rocprofv3 --pmc runs of bench.py; FETCH_SIZE / WRITE_SIZE are KiB per dispatch,",
        f"# scaled by the same counter on a plain {COPY_BYTES >> 20} MiB copy kernel in the same run",
        f"# fetch command: {commands[0]}",
        f"# write command: {commands[1]}",
        f"# summary command: python bench.py --workload {workload} --summarize-pmc {fetch_dir} {write_dir}",
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
    run's timestamps at the box's 2.4 GHz peak clock, so it is a lower bound."""
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


def summarize_trace(workload: str, directory: str, command: str, kernel: str = "decode") -> Path:
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace --stats run, as text."""
    import csv
    files = sorted(Path(directory).rglob("*kernel_stats.csv"))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {directory}")
    lines = [f"# rocprofv3 kernel statistics, workload {workload}",
             f"# command: {command}",
             f"# summary command: python bench.py --workload {workload} {'--prefill ' if kernel == 'prefill' else ''}"
             f"--summarize-trace {directory}",
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
    path = PROFILES / f"{kernel}_{workload}_kernel_trace.txt"
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


def cpu_baseline(x, gpu_out, budget_s: float) -> dict:
    """Time the float64 oracle on a bounded sample of the batch and compare it with the GPU output."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    c = x.cfg
    geo = oracle.CacheGeometry(x.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.dtype)
    k2, v2 = oracle.store_kvcache(x.k_new, x.v_new, x.slot_mapping, x.k_cache, x.v_cache, geo)
    # sequences in a seeded order, in chunks, until the time budget is spent or the batch is done
    order = np.random.default_rng(12345).permutation(c.batch).tolist()
    seqs, tokens, dt = [], 0, 0.0
    ref = np.zeros((c.batch, c.num_heads, c.head_dim))
    while order and dt < budget_s:
        chunk, order = order[:8], order[8:]
        t = time.perf_counter()
        part = oracle.decode(x.q, k2, v2, x.block_tables, x.context_lens, x.scale, geo, seqs=chunk)
        dt += time.perf_counter() - t
        ref[chunk] = part[chunk]
        seqs += chunk
        tokens += int(x.context_lens[chunk].sum())
    kv = tokens * c.num_kv_heads * c.head_dim * c.elem_bytes * 2
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    err = float(np.abs(gpu_out[seqs] - ref[seqs]).max())
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(seqs)} of {c.batch} sequences ({tokens} context tokens) after the step's scatter, float64 numpy",
            "seconds": dt, "tokens_per_s": len(seqs) / dt, "host_cpus": len(os.sched_getaffinity(0)),
            "parity_max_abs_err_vs_gpu": err}


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}


def _pcts(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"p10_us": round(float(np.percentile(a, 10)), 2), "median_us": round(float(np.median(a)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2)}


def extra_timings(calls: dict, reps: int, stream_bytes: int, dev) -> dict:
    """Per-call event timings (p10 / median / p90) of each callable, measured back to back.

    Also times torch's sum over `stream_bytes` of fp32 as a plain streaming-read reference rate.
    """
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
    buf = torch.ones(stream_bytes // 4, dtype=torch.float32, device=dev)
    buf.sum()
    torch.cuda.synchronize()
    evs = [(TimingEvent(), TimingEvent()) for _ in range(5)]
    for b, e in evs:
        b.record()
        buf.sum()
        e.record()
    torch.cuda.synchronize()
    best = min(b.elapsed_time(e) for b, e in evs)
    out["stream_read_reference"] = {"gbs": round(stream_bytes / (best * 1e-3) / 1e9, 1),
                                    "what": f"torch.sum over {stream_bytes >> 30} GiB fp32, best of 5"}
    del buf
    torch.cuda.empty_cache()
    return out


def prefill_useful_flops(head_dim: int, num_heads: int, new_tokens, context_lens) -> float:
    """Useful flops of a causal paged prefill: 4*D*Hq per visible (query, key) pair. A sequence
    with n new tokens among L sees n*L - n(n-1)/2 pairs (query i, at position L-n+i, sees
    L-n+i+1 keys)."""
    import numpy as np
    n = np.asarray(new_tokens, dtype=np.float64)
    L = np.asarray(context_lens, dtype=np.float64)
    return 4.0 * head_dim * num_heads * float(np.sum(n * L - n * (n - 1) / 2))


def prefill_bench(args) -> None:
    """Full-prompt causal prefill over the workload's paged caches; useful flops = 4*D*Hq*sum(n*L - n(n-1)/2)."""
    import numpy as np
    import torch

    import paged_attention_decode_amd as pa
    from workloads import get_config, make_inputs, to_storage

    dev = torch.device("cuda:0")
    cfg = get_config(args.workload)
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
    for _ in range(max(1, args.warmup)):
        pa.paged_prefill(q, k_cache, v_cache, bt, cl, qst, x.scale, out)
    torch.cuda.synchronize()
    ev = [TimingEvent() for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(args.steps):
        pa.paged_prefill(q, k_cache, v_cache, bt, cl, qst, x.scale, out)
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    print(json.dumps({
        "metric": "paged prefill TFLOP/s (causal, full prompts)", "value": round(tflops, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded, shapes of the workload)",
        "config": dict(describe(cfg), prompt_tokens=int(qs[-1]), useful_flops=flops),
        "tokens_per_s": round(float(qs[-1]) / (ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None, "kernel": "prefill_kernel",
                     "kernel_mean_ms": round(ms, 5)}}), flush=True)


def main():
    args = parse()
    if args.summarize_pmc:
        print(summarize_pmc(args.workload, args.summarize_pmc[0], args.summarize_pmc[1], args.pmc_commands))
        return
    if args.summarize_sq:
        print(summarize_sq(args.workload, args.summarize_sq, args.sq_commands, "prefill" if args.prefill else "decode"))
        return
    if args.summarize_trace:
        print(summarize_trace(args.workload, args.summarize_trace, args.trace_command,
                              "prefill" if args.prefill else "decode"))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the library "
              "has no cross-GPU step; each GPU would run its own shard of sequences or kv heads", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_attention_decode_amd as pa
    from workloads import get_config, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pa.load_library()
    if args.prefill:
        prefill_bench(args)
        return
    dev = torch.device("cuda:0")
    cfg = get_config(args.workload)
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    x = make_inputs(cfg)
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]

    def up(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    k_cache = up(x.k_cache).view(pa.k_cache_shape(x.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.block_size, tdt))
    v_cache = up(x.v_cache).view(pa.v_cache_shape(x.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.block_size))
    q, k_new, v_new = up(x.q), up(x.k_new), up(x.v_new)
    block_tables = torch.from_numpy(x.block_tables).to(dev)
    context_lens = torch.from_numpy(x.context_lens).to(dev)
    slots = torch.from_numpy(x.slot_mapping).to(dev)
    out = torch.empty((cfg.batch, cfg.num_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        if args.fused_step:
            pa.decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, x.scale, out,
                           partition_size=args.partition_size, cached_prefix_tokens=args.cached_prefix_tokens,
                           events=events, shared_prefix=args.shared_prefix)
            return
        pa.store_kvcache(k_new, v_new, slots, k_cache, v_cache)
        pa.paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, x.scale, out,
                                  partition_size=args.partition_size,
                                  cached_prefix_tokens=args.cached_prefix_tokens, events=events,
                                  shared_prefix=args.shared_prefix)

    # A plain copy of known size (COPY_BYTES read + written): counter runs scale HBM bytes by it.
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    # The first call allocates the library's workspace; warm-up keeps that out of the timed region.
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    events = [(TimingEvent(), TimingEvent())
              for _ in range(args.steps)]
    for e in events:  # materialise the HIP events outside the timed region
        e[0].record(stream)
        e[1].record(stream)
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
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
        for i in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        kernel_ms = [e[0].elapsed_time(e[1]) for e in events]
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kernel_ms = [e[0].elapsed_time(e[1]) for e in events]

    ms_per_step = wall * 1e3 / args.steps
    kv_bytes = x.kv_bytes
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    mean_kernel_ms = sum(kernel_ms) / len(kernel_ms)
    achieved = kv_bytes / (mean_kernel_ms * 1e-3) / 1e9
    # The distinct K/V bytes of the batch (a block shared by several sequences counted once): the
    # least any kernel must read. Logical bytes above it are re-reads that caches or the
    # shared-prefix option serve.
    achieved_unique = x.unique_kv_bytes / (mean_kernel_ms * 1e-3) / 1e9
    # With shared prefixes the kernel reads each shared block once: its algorithmic bytes are the
    # distinct ones, and the roofline is taken on those.
    roof_bytes = "distinct K/V bytes (shared blocks once)" if args.shared_prefix else "logical K/V bytes"
    roof_achieved = achieved_unique if args.shared_prefix else achieved

    # Steps timed after overwriting 1 GiB, so last-level caches hold no KV (reported beside the main figure).
    cold = []
    if args.cold_steps > 0:
        # reading (not writing) 1 GiB leaves no dirty lines to be written back during the step
        scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(args.cold_steps):
            scratch.sum()
            ev = (TimingEvent(), TimingEvent())
            step(ev)
            torch.cuda.synchronize()
            cold.append(ev[0].elapsed_time(ev[1]))
        del scratch

    comparators = None
    if args.comparators:
        print("[bench] comparator: torch gather-and-mask", file=sys.stderr, flush=True)
        max_len = int(context_lens.max().item())
        ref = torch_gather_mask_decode(q, k_cache, v_cache, block_tables, context_lens, x.scale, max_len)
        torch.cuda.synchronize()
        reps = 3
        t0 = time.perf_counter()
        for _ in range(reps):
            torch_gather_mask_decode(q, k_cache, v_cache, block_tables, context_lens, x.scale, max_len)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / reps
        comparators = {"torch_gather_mask": {
            "ms_per_decode": round(ms, 4), "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
            "speedup_of_library_kernel": round(ms / mean_kernel_ms, 2),
            "max_abs_diff_vs_library": float((ref - out).abs().max().item()),
            "note": "decode only (no store), fp32 math, padded to the longest context"}}
        del ref
        torch.cuda.empty_cache()

    # Per-call distributions, outside the timed region above. The store here rewrites the same
    # slots with the same rows, so the cache contents do not change.
    def decode_with(psize, shared=args.shared_prefix):
        return lambda: pa.paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, x.scale, out,
                                                 partition_size=psize,
                                                 cached_prefix_tokens=args.cached_prefix_tokens,
                                                 shared_prefix=shared)
    calls = {"store": lambda: pa.store_kvcache(k_new, v_new, slots, k_cache, v_cache),
             "decode": decode_with(args.partition_size), "store_plus_decode": step}
    for psize, name in ((-2, "decode_balanced"), (-1, "decode_one_pass"), (512, "decode_split_512")):
        calls[name] = decode_with(psize, False)
    calls["decode_balanced_shared_prefix"] = decode_with(-2, True)
    timings = None
    if not args.no_extra_timings:
        timings = extra_timings(calls, 20, 2 << 30, dev)
        timings["decode_tokens_per_s"] = round(cfg.batch / (timings["decode"]["median_us"] * 1e-6), 1)
        timings["note"] = ("cudaEvent pairs per call on the current stream, back to back (warm caches); "
                           "decode includes the merge kernel where the plan splits")

    traffic = traffic_from_profiles(cfg.name, kv_bytes)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded, shapes of the workload)",
        "config": dict(describe(cfg), kv_bytes_per_step=kv_bytes, unique_kv_bytes=x.unique_kv_bytes,
                       partition_size=args.partition_size, shared_prefix=bool(args.shared_prefix),
                       cached_prefix_tokens=args.cached_prefix_tokens or pa.DEFAULT_CACHED_PREFIX_TOKENS,
                       launch="hip graph replay" if args.graph else "eager",
                       step="pa_decode_step (fused scatter + attention)" if args.fused_step
                       else "pa_store_kvcache + pa_paged_attention_decode", parallelism="single GPU"),
        "tokens_per_s": round(cfg.batch / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(roof_achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(roof_achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "bytes": roof_bytes,
                     "achieved_on_logical_bytes": round(achieved, 2),
                     "achieved_on_unique_bytes": round(achieved_unique, 2),
                     "kernel": "decode_kernel (attention, excludes store and merge; with the shared-prefix "
                               "option also its detection kernel)",
                     "kernel_mean_ms": round(mean_kernel_ms, 5),
                     "cold_kernel_median_ms": round(sorted(cold)[len(cold) // 2], 5) if cold else None},
    }
    if timings:
        result["timings"] = timings
    if comparators:
        result["comparators"] = comparators
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(x, out.cpu().numpy(), args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
