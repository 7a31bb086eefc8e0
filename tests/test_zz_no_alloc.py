"""Entry point without allocation: pa_paged_attention_decode_noalloc, called through the C ABI,
against pa_paged_attention_decode_ex (library-owned workspace) on the same inputs."""

from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

import oracle
from workloads import make_inputs
from _gpu_helpers import TOL, custom_config, geometry, oracle_after_store, to_device

pytestmark = pytest.mark.gpu

PA_ERR_WORKSPACE = 5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _call(lib, name, dev, x, out, psize, shared_prefix=False, workspace=None):
    """One decode call through the C ABI; returns the status code."""
    import paged_attention_decode_amd as pa
    c = x.cfg
    opts = pa.DecodeOpts()
    opts.partition_size = psize
    opts.shared_prefix = 1 if shared_prefix else 0
    if workspace is not None:
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel()
    q = dev["q"]
    dt = {"fp32": pa.DTYPE_F32, "fp16": pa.DTYPE_F16, "bf16": pa.DTYPE_BF16}[c.dtype]
    stream = q.get_device()
    import torch
    return getattr(lib, name)(
        q.data_ptr(), dev["k_cache"].data_ptr(), dev["v_cache"].data_ptr(), dev["block_tables"].data_ptr(),
        dev["context_lens"].data_ptr(), ctypes.c_float(x.scale), out.data_ptr(), c.batch, c.num_heads,
        c.num_kv_heads, c.head_dim, c.block_size, int(x.block_tables.shape[1]), x.num_blocks, q.stride(0), dt,
        pa.DTYPE_F32, ctypes.byref(opts), ctypes.c_void_p(torch.cuda.current_stream(stream).cuda_stream))


def _store(dev):
    import paged_attention_decode_amd as pa
    pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])


# (config, partition_size, shared_prefix): a larger split-mode call, then a smaller one
CALLS = [
    (dict(dtype="bf16", batch=48, hq=16, hkv=8, d=128, bs=16,
          lens=tuple(int(v) for v in np.random.default_rng(21).integers(1, 3000, 48)), seed=21), -2, False),
    (dict(dtype="fp16", batch=5, hq=8, hkv=2, d=64, bs=16, lens=(1, 40, 17, 700, 129), seed=22), 48, False),
]


def test_noalloc_matches_decode_ex_on_two_calls_in_a_row(cuda):
    import torch
    import paged_attention_decode_amd as pa
    lib = pa.load_library()
    cases = []
    for kw, psize, shared in CALLS:
        x = make_inputs(custom_config(**kw))
        dev = to_device(x, cuda)
        _store(dev)
        plan = pa.decode_plan(x.cfg.batch, x.cfg.num_heads, x.cfg.num_kv_heads, x.cfg.head_dim,
                              x.cfg.block_size, int(x.block_tables.shape[1]),
                              {"fp16": pa.DTYPE_F16, "bf16": pa.DTYPE_BF16}[x.cfg.dtype], psize, 0,
                              shared_prefix=shared)
        assert plan["uses_reduce"] and 0 < plan["workspace_bytes"] <= pa.NOALLOC_SCRATCH_BYTES
        out = torch.full((x.cfg.batch, x.cfg.num_heads, x.cfg.head_dim), float("nan"), device=cuda)
        ref_out = torch.full_like(out, float("nan"))
        cases.append((x, dev, out, ref_out, psize, shared))
    torch.cuda.synchronize()
    # Set-up and module loading outside the measured region: one call of each entry point per case.
    for x, dev, out, ref_out, psize, shared in cases:
        assert _call(lib, "pa_paged_attention_decode_noalloc", dev, x, out, psize, shared) == 0
        assert _call(lib, "pa_paged_attention_decode_ex", dev, x, ref_out, psize, shared) == 0
    torch.cuda.synchronize()
    pa.shutdown()  # frees the library-owned workspace of the _ex calls
    for _, _, out, ref_out, _, _ in cases:
        out.fill_(float("nan"))
        ref_out.fill_(float("nan"))
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info(cuda)[0]
    # Two no-allocation calls in a row, the second with a smaller input.
    for i, (x, dev, out, _, psize, shared) in enumerate(cases):
        _say(f"[gpu] noalloc call {i}: B={x.cfg.batch} D={x.cfg.head_dim} {x.cfg.dtype} partition_size={psize}")
        rc = _call(lib, "pa_paged_attention_decode_noalloc", dev, x, out, psize, shared)
        assert rc == 0, lib.pa_last_error().decode()
    torch.cuda.synchronize()
    free_after = torch.cuda.mem_get_info(cuda)[0]
    assert free_after == free_before, "the no-allocation calls changed the device's free memory"
    # The existing entry point on the same inputs, in the same order.
    for x, dev, _, ref_out, psize, shared in cases:
        assert _call(lib, "pa_paged_attention_decode_ex", dev, x, ref_out, psize, shared) == 0
    torch.cuda.synchronize()
    for i, (x, dev, out, ref_out, _, _) in enumerate(cases):
        got, want = out.cpu().numpy(), ref_out.cpu().numpy()
        assert np.isfinite(got).all()
        # same kernels, same plan: the same bits
        assert got.tobytes() == want.tobytes(), f"call {i}: outputs differ from pa_paged_attention_decode_ex"
        _, _, oref = oracle_after_store(x)
        err = np.abs(got - oref).max()
        _say(f"[gpu] noalloc call {i}: max-abs error {err:.3e} against the oracle")
        assert err <= TOL[x.cfg.dtype]


def test_noalloc_rejects_a_caller_workspace_and_plans_beyond_the_scratch(cuda):
    """Host-side refusals: nothing is enqueued, the output stays as it was."""
    import torch
    import paged_attention_decode_amd as pa
    lib = pa.load_library()
    x = make_inputs(custom_config(dtype="bf16", batch=4, hq=8, hkv=2, d=128, bs=16, lens=(5, 100, 33, 64), seed=23))
    dev = to_device(x, cuda)
    out = torch.full((4, 8, 128), 7.0, device=cuda)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=cuda)
    rc = _call(lib, "pa_paged_attention_decode_noalloc", dev, x, out, -2, workspace=ws)
    assert rc == PA_ERR_WORKSPACE and "NULL" in lib.pa_last_error().decode()
    # A wide block table (8192 entries per sequence) with 16-token fixed ranges: the plan sizes its
    # workspace for the longest contexts the table allows, far beyond the scratch. The contexts
    # are short and every entry is a valid block, so the inputs themselves are sound.
    wide = torch.zeros((4, 8192), dtype=torch.int32, device=cuda)
    wide[:, :x.block_tables.shape[1]] = dev["block_tables"]
    dev2 = dict(dev, block_tables=wide)
    plan = pa.decode_plan(4, 8, 2, 128, 16, 8192, pa.DTYPE_BF16, 16, 0)
    assert plan["workspace_bytes"] > pa.NOALLOC_SCRATCH_BYTES
    x2 = type("X", (), {})()
    x2.cfg, x2.scale, x2.num_blocks, x2.block_tables = x.cfg, x.scale, x.num_blocks, np.zeros((4, 8192), np.int32)
    rc = _call(lib, "pa_paged_attention_decode_noalloc", dev2, x2, out, 16)
    assert rc == PA_ERR_WORKSPACE and "fixed scratch" in lib.pa_last_error().decode()
    torch.cuda.synchronize()
    assert (out == 7.0).all()
    # the same inputs through the regular entry point are fine (it grows its own workspace)
    assert _call(lib, "pa_paged_attention_decode_ex", dev2, x2, out, 16) == 0
    torch.cuda.synchronize()
    ref = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, x.scale, geometry(x))
    assert np.abs(out.cpu().numpy() - ref).max() <= TOL["bf16"]
