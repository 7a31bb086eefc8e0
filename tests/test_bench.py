"""Host logic of bench.py (no GPU): the prefill flop count, the rocprofv3 summaries and their
staleness check, and the one-GPU guard. Summaries are written to a temporary directory."""

from __future__ import annotations

import csv
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


@pytest.fixture
def profiles(tmp_path, monkeypatch):
    d = tmp_path / "profiles"
    monkeypatch.setattr(bench, "PROFILES", d)
    return d


def _write_csv(path: Path, header, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_prefill_flops_count_visible_pairs():
    rng = np.random.default_rng(3)
    L = rng.integers(1, 40, 9)
    n = np.minimum(L, rng.integers(1, 40, 9))
    pairs = sum(L[s] - n[s] + i + 1 for s in range(len(L)) for i in range(n[s]))
    assert bench.prefill_useful_flops(64, 8, n, L) == 4.0 * 64 * 8 * pairs
    # full prompts: L(L+1)/2 pairs each
    assert bench.prefill_useful_flops(128, 1, [5], [5]) == 4.0 * 128 * 15


def _counter_rows(kernel_values, counter):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = [[i, name, counter, v, 1000 * i, 1000 * i + 500] for i, (name, v) in enumerate(kernel_values)]
    return hdr, rows


def test_traffic_summary_scales_by_the_copy_and_goes_stale(profiles, tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    # FETCH_SIZE reads half the true bytes on the copy (factor 2), WRITE_SIZE all of them (factor 1)
    hdr, rows = _counter_rows([("__amd_rocclr_copyBuffer", copy_kib / 2), ("pa::decode_kernel<2, 128, false>", 1000.0),
                               ("pa::decode_kernel<2, 128, false>", 1200.0)], "FETCH_SIZE")
    _write_csv(tmp_path / "f" / "run_counter_collection.csv", hdr, rows)
    hdr, rows = _counter_rows([("__amd_rocclr_copyBuffer", copy_kib), ("pa::decode_kernel<2, 128, false>", 10.0),
                               ("pa::decode_kernel<2, 128, false>", 10.0)], "WRITE_SIZE")
    _write_csv(tmp_path / "w" / "run_counter_collection.csv", hdr, rows)
    path = bench.summarize_pmc("wl", str(tmp_path / "f"), str(tmp_path / "w"), ("fetch cmd", "write cmd"))
    text = path.read_text()
    assert "fetch cmd" in text and "write cmd" in text
    expect = 1100.0 * 2 * 1024 + 10.0 * 1024
    got = bench.traffic_from_profiles("wl", 0.0)
    assert got == pytest.approx(expect, rel=1e-9)
    # another kernel source: the summary no longer applies
    path.write_text(text.replace("kernel_source_sha256: ", "kernel_source_sha256: 0"))
    assert bench.traffic_from_profiles("wl", 0.0) is None
    assert bench.traffic_from_profiles("missing", 0.0) is None


def test_trace_summary_lists_every_kernel(profiles, tmp_path):
    hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
    rows = [["void pa::(anonymous namespace)::decode_kernel<2, 128, false>(pa::DecodeArgs)", 13, 2.9e6, 228990.0,
             90.5, 220770.0, 292760.0, 1.0],
            ["void pa::(anonymous namespace)::reduce_kernel<2, 128>(pa::DecodeArgs)", 13, 7.0e4, 5410.0, 2.1, 4960.0,
             6800.0, 1.0]]
    _write_csv(tmp_path / "t" / "run_kernel_stats.csv", hdr, rows)
    # per-launch trace: 3 warm-up launches (slow) then 2 timed ones, with a merge kernel between
    k = "void pa::(anonymous namespace)::decode_kernel<2, 128, false>(pa::DecodeArgs)"
    trace = [[k, 0, 300000], ["reduce_kernel", 300000, 305000], [k, 400000, 690000], [k, 800000, 1050000],
             [k, 1100000, 1320000], [k, 1400000, 1630000]]
    _write_csv(tmp_path / "t" / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    path = bench.summarize_trace("wl", str(tmp_path / "t"), "rocprofv3 ... -- python -u bench.py --steps 2")
    text = path.read_text()
    assert path.name == "decode_wl_kernel_trace.txt"
    assert "# command: rocprofv3 ... -- python -u bench.py --steps 2" in text and "anonymous namespace" not in text
    assert "timed_launches: 2" in text and "timed_launches_mean_us: 225.00" in text
    assert "228.99" in text and "5.41" in text
    assert f"kernel_source_sha256: {bench.kernel_source_sha()}" in text


def test_sq_summary_shares(profiles, tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    k = "pa::prefill_shared_kernel<2, 128>"
    rows = [[1, k, "SQ_WAVE_CYCLES", 1000, 0, 10000], [1, k, "SQ_ACTIVE_INST_VALU", 300, 0, 10000],
            [1, k, "SQ_WAIT_INST_ANY", 400, 0, 10000], [1, k, "SQ_WAIT_ANY", 200, 0, 10000],
            [1, "__amd_rocclr_copyBuffer", "SQ_WAVE_CYCLES", 5, 0, 10]]
    _write_csv(tmp_path / "a" / "run_counter_collection.csv", hdr, rows)
    rows = [[1, k, "SQ_INSTS_VALU", 450, 0, 10000], [1, k, "SQ_INSTS_MFMA", 100, 0, 10000]]
    _write_csv(tmp_path / "b" / "run_counter_collection.csv", hdr, rows)
    path = bench.summarize_sq("wl", [str(tmp_path / "a"), str(tmp_path / "b")], ["c1", "c2"], "prefill")
    text = path.read_text()
    assert path.name == "prefill_wl_sq_counters.txt"
    assert "issuing VALU (incl. MFMA): 0.300" in text
    assert "waiting to issue: 0.400" in text
    assert "waiting on s_waitcnt or a barrier: 0.200" in text
    assert "valu_instructions_per_mfma: 3.50" in text
    assert "SQ_WAVE_CYCLES: 1000 (1 dispatches)" in text  # the copy kernel's row is not counted


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_measurement_library_rejects_bad_arguments_before_any_launch():
    """libpa_stream_read.so (the streaming-read and matrix-core ceilings) exports both entry points
    and checks its arguments on the host: each bad call returns 1 without touching the GPU."""
    import ctypes
    lib_path = ROOT / "paged_attention_decode_amd" / "libpa_stream_read.so"
    if not lib_path.exists():
        pytest.skip("measurement library not built")
    lib = ctypes.CDLL(str(lib_path))
    lib.pa_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.pa_bench_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails its checks first
    assert lib.pa_bench_stream_read(None, 1 << 20, 0, 8, 4, p, None) == 1
    assert lib.pa_bench_stream_read(p, 1000, 0, 8, 4, p, None) == 1          # not a multiple of 16 KiB
    assert lib.pa_bench_stream_read(p, 1 << 31, 0, 8, 4, p, None) == 1       # past one buffer resource
    assert lib.pa_bench_stream_read(p, 1 << 20, 3, 8, 4, p, None) == 1       # unknown policy
    assert lib.pa_bench_mfma(3, 10, 4, 0, p, None) == 1                      # unknown kind
    assert lib.pa_bench_mfma(0, 0, 4, 0, p, None) == 1                       # no iterations
    assert lib.pa_bench_mfma(0, 10, 0, 0, p, None) == 1                      # empty grid
    assert lib.pa_bench_mfma(0, 10, 4, 65537, p, None) == 1                  # LDS request too large
    assert lib.pa_bench_mfma(0, 10, 4, 0, None, None) == 1                   # no sink
