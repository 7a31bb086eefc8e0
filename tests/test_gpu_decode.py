"""GPU parity: store_kvcache and paged_attention_decode through the C ABI against the CPU oracle.

Tolerances (max-abs on fp32 output): 1e-5 for fp32 inputs, 2e-3 for fp16/bf16
inputs. With output in the input dtype the bound is 2e-3 (or 1e-5) plus half
an ulp of that dtype at the oracle value: one final round-to-nearest-even.
The scatter must be bit-exact over the whole cache buffers.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import CONFIG_ORDER, get_config, make_inputs, nan_of, poison_blocks, to_storage
from _gpu_helpers import (TOL, custom_config, geometry, half_ulp, np_to_torch, oracle_after_store, to_device,
                          torch_dtype, torch_to_np)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_step(dev, x, partition_size=0, out_dtype=None):
    import torch
    import paged_attention_decode_amd as pa
    pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
    out = pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                    dev["context_lens"], x.scale, out_dtype=out_dtype or torch.float32,
                                    partition_size=partition_size)
    torch.cuda.synchronize()
    return out


def _sample_seqs(x, limit):
    """All sequences if few, else the shortest, the longest and a seeded random rest, ``limit`` in all."""
    b = x.cfg.batch
    if b <= limit:
        return list(range(b))
    order = np.argsort(x.context_lens, kind="stable")
    ends = max(1, min(4, limit // 4))
    pick = list(dict.fromkeys(order[:ends].tolist() + order[-ends:].tolist()))[:limit]
    rest = [s for s in np.random.default_rng(0).permutation(b).tolist() if s not in pick]
    return sorted(pick + rest[:limit - len(pick)])


_CACHE = {}


def _inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = make_inputs(get_config(name))
    return _CACHE[name]


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_full_config_store_bit_exact_and_decode_parity(cuda, name):
    """Every workload at full size, default launch (the one the bench times)."""
    import torch
    _say(f"[gpu] full config {name}: generating")
    x = _inputs(name)
    limit = {"long_ctx_bf16": 3, "skewed_prefix_bf16": 40}.get(name, 10 ** 9)
    seqs = _sample_seqs(x, limit)
    dev = to_device(x, cuda)
    _say(f"[gpu] full config {name}: store + decode, B={x.cfg.batch}")
    out = _run_step(dev, x).cpu().numpy()
    k2, v2, ref = oracle_after_store(x, seqs=seqs)
    assert torch_to_np(dev["k_cache"], x.cfg.dtype).reshape(-1).tobytes() == k2.reshape(-1).tobytes()
    assert torch_to_np(dev["v_cache"], x.cfg.dtype).reshape(-1).tobytes() == v2.reshape(-1).tobytes()
    assert np.isfinite(out).all()
    err = np.abs(out[seqs] - ref[seqs]).max()
    _say(f"[gpu] {name}: max-abs error {err:.3e} over {len(seqs)} sequences")
    assert err <= TOL[x.cfg.dtype]
    # the same step with output in the input dtype: one extra rounding at most
    if x.cfg.dtype != "fp32":
        out_t = _run_step(dev, x, out_dtype=torch_dtype(x.cfg.dtype)).float().cpu().numpy()
        bound = TOL[x.cfg.dtype] + half_ulp(ref[seqs], x.cfg.dtype)
        assert (np.abs(out_t[seqs] - ref[seqs]) <= bound).all()
    del dev
    torch.cuda.empty_cache()


def test_long_context_in_512_token_partitions_full_size(cuda):
    """The 16 x 32768-token workload as specified: fixed 512-token partitions, each segment's 64
    pieces merged by the log-sum-exp reduce kernel. Store bit-exact over both whole caches;
    decode of sampled sequences (first, last and two seeded others) against the oracle."""
    import torch
    import paged_attention_decode_amd as pa
    _say("[gpu] long_ctx_bf16 at partition_size=512: generating")
    x = _inputs("long_ctx_bf16")
    c = x.cfg
    plan = pa.decode_plan(c.batch, c.num_heads, c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks_per_seq,
                          pa.DTYPE_BF16, partition_size=512)
    assert plan["range_tokens"] == 512 and plan["uses_reduce"]
    # every context is 64 whole partitions, so every segment is cut into 64 merged pieces
    assert (x.context_lens == 32768).all()
    seqs = sorted({0, c.batch - 1, *np.random.default_rng(4).choice(np.arange(1, c.batch - 1), 2, replace=False)})
    dev = to_device(x, cuda)
    _say(f"[gpu] long_ctx_bf16 at partition_size=512: store + decode, checking sequences {seqs}")
    out = _run_step(dev, x, partition_size=512).cpu().numpy()
    k2, v2, ref = oracle_after_store(x, seqs=seqs)
    assert torch_to_np(dev["k_cache"], c.dtype).reshape(-1).tobytes() == k2.reshape(-1).tobytes()
    assert torch_to_np(dev["v_cache"], c.dtype).reshape(-1).tobytes() == v2.reshape(-1).tobytes()
    assert np.isfinite(out).all()
    err = np.abs(out[seqs] - ref[seqs]).max()
    _say(f"[gpu] long_ctx_bf16 at 512: max-abs error {err:.3e}")
    assert err <= TOL[c.dtype]
    # bf16 output: one extra round-to-nearest-even at most
    out_t = _run_step(dev, x, partition_size=512, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert (np.abs(out_t[seqs] - ref[seqs]) <= TOL[c.dtype] + half_ulp(ref[seqs], c.dtype)).all()
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["qwen3_0p6b_bf16", "llama32_1b_fp16"])
def test_torch_gather_mask_comparator_matches_oracle(cuda, name):
    """The benchmark's PyTorch comparator (batched gather through the block tables, masked
    softmax, weighted sum) computes the oracle's result on the workload's own inputs."""
    import torch
    from bench import torch_gather_mask_decode
    _say(f"[gpu] comparator {name}")
    x = _inputs(name)
    dev = to_device(x, cuda)
    ref = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, x.scale, geometry(x))
    got = torch_gather_mask_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], x.scale, int(x.context_lens.max()))
    got = got.float().cpu().numpy()
    err = np.abs(got - ref).max()
    _say(f"[gpu] comparator {name}: max-abs error {err:.3e}")
    assert err <= TOL[x.cfg.dtype]
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("psize", [-3, -2, -1, 0, 16, 48, 512])
@pytest.mark.parametrize("name", ["tiny_fp32", "qwen3_0p6b_bf16", "llama32_1b_fp16"])
def test_launch_modes_agree_with_oracle(cuda, name, psize):
    _say(f"[gpu] modes {name} partition_size={psize}")
    x = _inputs(name)
    dev = to_device(x, cuda)
    out = _run_step(dev, x, partition_size=psize).cpu().numpy()
    _, _, ref = oracle_after_store(x)
    assert np.abs(out - ref).max() <= TOL[x.cfg.dtype]


@pytest.mark.parametrize("psize", [-3, -2, -1, 32])
@pytest.mark.parametrize("dt,d", [("bf16", 128), ("fp16", 64)])
def test_large_logits_in_every_mode(cuda, dt, d, psize):
    """q and K scaled by 32 (exact, a power of two): logits in the thousands (log2 units), so each
    tile moves the running maximum by hundreds, and split pieces of one context carry log-sum-exp
    values far apart (most merge weights underflow to zero). Store + decode against the oracle."""
    from _paged_helpers import widen_np
    _say(f"[gpu] large logits {dt} head_dim {d} partition_size={psize}")
    x = make_inputs(custom_config(dtype=dt, batch=5, hq=8, hkv=2, d=d, lens=(1, 40, 300, 777, 1500), seed=606))
    x.k_cache = to_storage((widen_np(x.k_cache, dt) * 32.0).astype(np.float32), dt)
    x.k_new = to_storage((widen_np(x.k_new, dt) * 32.0).astype(np.float32), dt)
    x.q = to_storage((widen_np(x.q, dt) * 32.0).astype(np.float32), dt)
    dev = to_device(x, cuda)
    out = _run_step(dev, x, partition_size=psize).cpu().numpy()
    _, _, ref = oracle_after_store(x)
    assert np.isfinite(out).all()
    assert np.abs(out - ref).max() <= TOL[dt], np.abs(out - ref).max()


@pytest.mark.parametrize("psize", [-2, 32])
def test_more_pieces_per_wavefront_than_lds_row_slots(cuda, psize):
    """A wavefront keeps the rows of at most 8 pieces in LDS until its last tile; further pieces
    are written at once. 3000 one-tile contexts (and a few long ones, which are cut) over 8 kv
    heads put about 12 whole segments in each balanced range, and with 32-token ranges a
    wavefront loops over about 12 ranges: both paths run in one launch."""
    import paged_attention_decode_amd as pa
    lens = [16] * 3000
    for i, L in ((7, 700), (1500, 1234), (2999, 333)):
        lens[i] = L
    x = make_inputs(custom_config(dtype="bf16", batch=len(lens), hq=16, hkv=8, d=128, lens=tuple(lens), seed=31))
    plan = pa.decode_plan(len(lens), 16, 8, 128, 16, int(x.block_tables.shape[1]), pa.DTYPE_BF16,
                          partition_size=psize)
    assert plan["uses_reduce"]
    _say(f"[gpu] LDS row slots overflow, partition_size={psize}, {plan['num_waves']} wavefronts")
    dev = to_device(x, cuda)
    out = _run_step(dev, x, partition_size=psize).cpu().numpy()
    _, _, ref = oracle_after_store(x)
    assert np.abs(out - ref).max() <= TOL["bf16"]


CASES = [
    # dtype, batch, Hq, Hkv, D, bs, lengths
    ("bf16", 5, 8, 2, 128, 16, (1, 2, 15, 16, 17)),
    ("fp16", 4, 4, 4, 64, 32, (31, 32, 33, 95)),
    ("fp32", 3, 6, 2, 128, 16, (5, 40, 77)),
    ("bf16", 3, 40, 2, 64, 16, (50, 1, 130)),          # 20 heads per kv head: groups of 16 + 4
    ("fp16", 2, 3, 1, 256, 64, (200, 63)),             # odd group, head_dim 256
    ("bf16", 4, 16, 2, 256, 256, (300, 256, 257, 1)),
    ("fp32", 2, 8, 1, 64, 128, (129, 300)),
    ("bf16", 6, 8, 8, 128, 16, (0, 5, 0, 64, 3, 1)),   # empty contexts give zeros
    ("fp32", 2, 4, 2, 256, 16, (40, 77)),              # fp32 at head_dim 256 (largest register set)
    ("bf16", 3, 32, 2, 256, 16, (70, 33, 16)),         # 16 heads at head_dim 256: workgroup split runs as one pass
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("psize", [-3, -2, -1, 0, 16, 64])
def test_small_shapes_and_edges(cuda, case, psize):
    dt, b, hq, hkv, d, bs, lens = CASES[case]
    _say(f"[gpu] small case {CASES[case]} partition_size={psize}")
    x = make_inputs(custom_config(dtype=dt, batch=b, hq=hq, hkv=hkv, d=d, bs=bs, lens=lens, seed=100 + case))
    dev = to_device(x, cuda)
    out = _run_step(dev, x, partition_size=psize).cpu().numpy()
    k2, v2, ref = oracle_after_store(x)
    assert torch_to_np(dev["k_cache"], dt).reshape(-1).tobytes() == k2.reshape(-1).tobytes()
    assert np.abs(out - ref).max() <= TOL[dt]
    for s in np.flatnonzero(x.context_lens == 0):
        assert (out[s] == 0).all()


def test_length_one_returns_value_row_exactly(cuda):
    import torch
    import paged_attention_decode_amd as pa
    x = make_inputs(custom_config(dtype="bf16", batch=4, hq=8, hkv=2, lens=(1, 1, 1, 1), seed=3))
    dev = to_device(x, cuda)
    for psize in (-3, -2, -1, 0):
        out = _run_step(dev, x, partition_size=psize).cpu().numpy()
        k2, v2, _ = oracle_after_store(x)
        geo = geometry(x)
        for s in range(4):
            _, v = oracle.gather_kv(k2, v2, x.block_tables[s], 1, geo)
            for h in range(8):
                np.testing.assert_array_equal(out[s, h], v[0, h // 4])


def test_identical_keys_give_mean_of_values(cuda):
    import torch
    import paged_attention_decode_amd as pa
    x = make_inputs(custom_config(dtype="bf16", batch=2, hq=8, hkv=2, lens=(77, 300), seed=4))
    geo = geometry(x)
    # one key row repeated over every slot of both caches' K (identical keys for every token)
    k = x.k_cache.reshape(geo.k_shape).copy()
    k[...] = k[:1, :, :, :1, :]
    x.k_cache = k.reshape(-1)
    x.slot_mapping[:] = -1
    dev = to_device(x, cuda)
    out = _run_step(dev, x).cpu().numpy()
    for s in range(2):
        _, v = oracle.gather_kv(x.k_cache, x.v_cache, x.block_tables[s], int(x.context_lens[s]), geo)
        mean = v.mean(axis=0)
        for h in range(8):
            assert np.abs(out[s, h] - mean[h // 4]).max() <= 2e-3


def test_poisoned_tail_slots_and_unused_blocks_change_nothing(cuda):
    """NaN in slots past each context and in unreferenced blocks, and garbage block-table entries
    past each context's last block (the kernel may read them, never use them), must not reach the
    output."""
    cfg = custom_config(dtype="bf16", batch=5, hq=8, hkv=2, lens=(3, 17, 250, 33, 1), seed=5)
    x = make_inputs(cfg)
    x.slot_mapping[:] = -1
    geo = geometry(x)
    modes = (-3, -2, -1, 0, 16)
    clean = {p: _run_step(to_device(x, cuda), x, partition_size=p).cpu().numpy() for p in modes}
    bs = cfg.block_size
    junk = np.array([-1, -(2 ** 31), 2 ** 31 - 1, x.num_blocks, 7 * x.num_blocks + 3], np.int64)
    for s in range(cfg.batch):
        used = (int(x.context_lens[s]) + bs - 1) // bs
        tail_entries = x.block_tables.shape[1] - used
        x.block_tables[s, used:] = np.resize(junk, tail_entries).astype(np.int32)
    assert (x.block_tables < 0).any(), "some sequence must have table entries past its context"
    kp = poison_blocks(x.k_cache, x.unused_blocks, cfg)
    vp = poison_blocks(x.v_cache, x.unused_blocks, cfg)
    # tail slots of each sequence's last block, written with NaN rows by the oracle's scatter
    tail = []
    for s in range(cfg.batch):
        L = int(x.context_lens[s])
        blk = int(x.block_tables[s, (L - 1) // bs])
        tail += [blk * bs + o for o in range(L % bs or bs, bs)]
    nan_rows = np.full((len(tail), cfg.num_kv_heads, cfg.head_dim), nan_of("bf16"), dtype=np.uint16)
    kp, vp = oracle.store_kvcache(nan_rows, nan_rows, np.array(tail, np.int32), kp, vp, geo)
    x.k_cache, x.v_cache = kp, vp
    for p, ref in clean.items():
        out = _run_step(to_device(x, cuda), x, partition_size=p).cpu().numpy()
        assert out.tobytes() == ref.tobytes(), f"partition_size={p}"


def test_relabelling_physical_blocks_is_bit_identical(cuda):
    cfg = custom_config(dtype="fp16", batch=4, hq=16, hkv=4, d=64, lens=(100, 7, 64, 513), seed=6)
    x = make_inputs(cfg)
    x.slot_mapping[:] = -1
    out = _run_step(to_device(x, cuda), x).cpu().numpy()
    geo = geometry(x)
    pi = np.random.default_rng(1).permutation(x.num_blocks)
    for name in ("k_cache", "v_cache"):
        a = getattr(x, name).reshape(geo.num_blocks, -1)
        b = np.empty_like(a)
        b[pi] = a
        setattr(x, name, b.reshape(-1))
    x.block_tables = pi[x.block_tables].astype(np.int32)
    out2 = _run_step(to_device(x, cuda), x).cpu().numpy()
    assert out.tobytes() == out2.tobytes()


def test_repeat_runs_are_deterministic(cuda):
    x = _inputs("llama32_1b_fp16")
    dev = to_device(x, cuda)
    a = _run_step(dev, x).cpu().numpy()
    b = _run_step(dev, x).cpu().numpy()
    assert a.tobytes() == b.tobytes()


def test_strided_q_and_k_v_slices(cuda):
    """q, k and v taken as column slices of one fused projection output."""
    import torch
    import paged_attention_decode_amd as pa
    cfg = custom_config(dtype="bf16", batch=3, hq=8, hkv=2, lens=(40, 1, 90), seed=8)
    x = make_inputs(cfg)
    dev = to_device(x, cuda)
    b, hq, hkv, d = 3, 8, 2, 128
    fused = torch.zeros(b, (hq + 2 * hkv) * d, dtype=torch.bfloat16, device=cuda)
    fused[:, :hq * d] = dev["q"].reshape(b, -1)
    fused[:, hq * d:(hq + hkv) * d] = dev["k_new"].reshape(b, -1)
    fused[:, (hq + hkv) * d:] = dev["v_new"].reshape(b, -1)
    q = fused[:, :hq * d].view(b, hq, d)
    k = fused[:, hq * d:(hq + hkv) * d].view(b, hkv, d)
    v = fused[:, (hq + hkv) * d:].view(b, hkv, d)
    assert q.stride(0) == (hq + 2 * hkv) * d
    pa.store_kvcache(k, v, dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
    out = pa.paged_attention_decode(q, dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                                    x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    k2, v2, ref = oracle_after_store(x)
    assert torch_to_np(dev["k_cache"], "bf16").reshape(-1).tobytes() == k2.reshape(-1).tobytes()
    assert np.abs(out.cpu().numpy() - ref).max() <= 2e-3


def test_store_skips_negative_and_out_of_range_slots(cuda):
    import torch
    import paged_attention_decode_amd as pa
    cfg = custom_config(dtype="fp16", batch=4, hq=4, hkv=2, d=64, lens=(5, 9, 12, 3), seed=9)
    x = make_inputs(cfg)
    nslots = x.num_blocks * cfg.block_size
    x.slot_mapping = np.array([x.slot_mapping[0], -1, nslots, x.slot_mapping[3]], np.int32)
    dev = to_device(x, cuda)
    pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
    torch.cuda.synchronize()
    geo = geometry(x)
    sm = x.slot_mapping.copy()
    sm[2] = -1
    k2, v2 = oracle.store_kvcache(x.k_new, x.v_new, sm, x.k_cache, x.v_cache, geo)
    assert torch_to_np(dev["k_cache"], "fp16").reshape(-1).tobytes() == k2.reshape(-1).tobytes()
    assert torch_to_np(dev["v_cache"], "fp16").reshape(-1).tobytes() == v2.reshape(-1).tobytes()


def test_caller_workspace_and_events(cuda):
    import torch
    import paged_attention_decode_amd as pa
    x = _inputs("qwen3_0p6b_bf16")
    c = x.cfg
    dev = to_device(x, cuda)
    # balanced ranges: the mode with a workspace (automatic takes one pass for this batch)
    need = pa.workspace_bytes(c.batch, c.num_heads, c.num_kv_heads, c.head_dim, c.block_size,
                              c.max_blocks_per_seq, pa.DTYPE_BF16, -2)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=cuda)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    out = pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                    dev["context_lens"], x.scale, out_dtype=torch.float32, workspace=ws, events=ev,
                                    partition_size=-2)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0
    ref = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, x.scale, geometry(x))
    assert np.abs(out.cpu().numpy() - ref).max() <= 2e-3
    with pytest.raises(pa.PagedAttnError) as ei:
        pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                  dev["context_lens"], x.scale, workspace=ws[:need // 2], partition_size=-2)
    assert ei.value.code == 5


@pytest.mark.parametrize("use_caller_ws", [False, True])
def test_graph_capture_of_the_decode_step_replays_exactly(cuda, use_caller_ws):
    """store_kvcache + paged_attention_decode recorded into a HIP graph; every replay matches eager."""
    import torch
    import paged_attention_decode_amd as pa
    x = make_inputs(custom_config(dtype="bf16", batch=6, hq=16, hkv=4, lens=(1, 40, 300, 17, 1000, 64), seed=11))
    c = x.cfg
    dev = to_device(x, cuda)
    ws = None
    if use_caller_ws:
        need = pa.workspace_bytes(c.batch, c.num_heads, c.num_kv_heads, c.head_dim, c.block_size,
                                  c.max_blocks_per_seq, pa.DTYPE_BF16, 0)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=cuda)
    out = torch.empty((c.batch, c.num_heads, c.head_dim), dtype=torch.float32, device=cuda)

    def step():
        pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
        pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                  dev["context_lens"], x.scale, out, workspace=ws)

    step()  # eager: allocates the library workspace if needed (allocation is not capturable)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    _, _, ref = oracle_after_store(x)
    for rep in range(4):
        out.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == eager.cpu().numpy().tobytes(), f"replay {rep}"
    assert np.abs(eager.cpu().numpy() - ref).max() <= 2e-3
    # new inputs in the same buffers are picked up by a replay
    dev["q"].copy_(dev["q"].flip(0))
    g.replay()
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    eager2 = out.clone()
    g.replay()
    torch.cuda.synchronize()
    assert out.cpu().numpy().tobytes() == eager2.cpu().numpy().tobytes()


def _fused_vs_two_calls(cuda, x, psize, out_dtype=None):
    import torch
    import paged_attention_decode_amd as pa
    odt = out_dtype or torch.float32
    dev_a = to_device(x, cuda)
    out_a = _run_step(dev_a, x, partition_size=psize, out_dtype=odt)
    dev_b = to_device(x, cuda)
    out_b = pa.decode_step(dev_b["q"], dev_b["k_new"], dev_b["v_new"], dev_b["k_cache"], dev_b["v_cache"],
                           dev_b["block_tables"], dev_b["context_lens"], x.scale, out_dtype=odt,
                           partition_size=psize)
    torch.cuda.synchronize()
    dt = x.cfg.dtype
    assert torch_to_np(dev_b["k_cache"], dt).tobytes() == torch_to_np(dev_a["k_cache"], dt).tobytes()
    assert torch_to_np(dev_b["v_cache"], dt).tobytes() == torch_to_np(dev_a["v_cache"], dt).tobytes()
    assert out_b.cpu().numpy().tobytes() == out_a.cpu().numpy().tobytes()
    return out_b


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("psize", [-3, -2, -1, 0, 16])
def test_fused_step_equals_store_then_decode(cuda, case, psize):
    dt, b, hq, hkv, d, bs, lens = CASES[case]
    _say(f"[gpu] fused step {CASES[case]} partition_size={psize}")
    x = make_inputs(custom_config(dtype=dt, batch=b, hq=hq, hkv=hkv, d=d, bs=bs, lens=lens, seed=200 + case))
    out = _fused_vs_two_calls(cuda, x, psize).cpu().numpy()
    _, _, ref = oracle_after_store(x)
    assert np.abs(out - ref).max() <= TOL[dt]


@pytest.mark.parametrize("name,psize", [("qwen3_0p6b_bf16", 0), ("llama32_1b_fp16", 0), ("skewed_prefix_bf16", 0),
                                        ("llama32_1b_fp16", 48), ("qwen3_0p6b_bf16", -3)])
def test_fused_step_full_configs(cuda, name, psize):
    # psize 48 on the Llama shape needs more ranges than resident wavefronts (they loop)
    _say(f"[gpu] fused step full config {name} partition_size={psize}")
    x = _inputs(name)
    _fused_vs_two_calls(cuda, x, psize)


def _tiny_weight_case(length=16384, d=64, bs=16, dtype="fp16"):
    """One sequence, G = 1: key 0 dominates and every other key has weight ~2^-15 of it, all
    with the same value sign, so rounding errors on the small weights add up in one direction.
    Built with the oracle's own scatter on a shuffled block table."""
    geo = oracle.CacheGeometry(num_blocks=length // bs + 8, num_kv_heads=1, head_dim=d, block_size=bs, dtype=dtype)
    rng = np.random.default_rng(2024)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 8.0
    k = np.zeros((length, 1, d), np.float32)
    k[0, 0, 0] = 10.3984375                 # scale 1/8: logit gap 10.398 = 15.0 in log2 units (fp16)
    v = np.full((length, 1, d), 4.0, np.float32)
    v[0] = -4.0
    v[1:, 0, :] += rng.integers(0, 8, (length - 1, d)).astype(np.float32) * np.float32(0.125)
    q, k, v = (to_storage(a, dtype) for a in (q, k, v))
    blocks = rng.permutation(geo.num_blocks)[:length // bs].astype(np.int32)
    slots = (blocks[np.arange(length) // bs] * bs + np.arange(length) % bs).astype(np.int32)
    kc = np.zeros(int(np.prod(geo.k_shape)), k.dtype)
    vc = np.zeros(int(np.prod(geo.v_shape)), v.dtype)
    kc, vc = oracle.store_kvcache(k, v, slots, kc, vc, geo)
    return geo, q, kc, vc, blocks[None, :], np.array([length], np.int32)


def _one_rounding_bound(geo, q, kc, vc, bt, cl):
    """Bound of a one-token prefill that rounds each weight once to fp16: weights in units of the
    dominant one's (2^7, exact) are p = 2^7 * exp(scale * (0 - q.k0)) for the n small keys, each
    rounded to fp16 (error <= half an ulp, all in one direction). With S = the sum of their values
    per dim, out = (2^7 v0 + p S) / (2^7 + n p) moves by 2^7 (S - n v0) / (2^7 + n p)^2 per unit of
    p. Plus 1e-4 for fp32 accumulation."""
    n = int(cl[0]) - 1
    k, v = oracle.gather_kv(kc, vc, bt[0], int(cl[0]), geo)
    v0, S = v[0, 0], v[1:, 0].sum(axis=0)
    qk0 = float(oracle.widen(q, geo.dtype)[0, 0] @ k[0, 0])
    p = 2.0 ** 7 * np.exp(float(np.float32(0.125)) * (0.0 - qk0))
    half_ulp_p = 2.0 ** (np.floor(np.log2(p)) - 11)
    return 2.0 ** 7 * np.abs(S - n * v0) / (2.0 ** 7 + n * p) ** 2 * half_ulp_p + 1e-4


def test_fp16_many_tiny_weights_keep_their_precision(cuda):
    """Without scaling, each 2^-15 weight would be an fp16 subnormal with absolute precision 2^-25
    in its value + remainder pair, and 16383 aligned rounding errors reach about 1e-3 (measured
    1.08e-3 in one pass). With scaling what remains is fp32 accumulation: one wavefront adding
    16383 equal terms (one pass) measures about 5e-5, split ranges about 4e-6. The bound 2e-4
    separates the two by a factor of 20.

    The one-token prefill rounds each fp16 weight once (no remainder), and here the 16383 small
    weights are equal, so their rounding errors align: its bound is that rounding's effect, derived
    below, plus the same fp32 accumulation allowance."""
    import torch
    import paged_attention_decode_amd as pa
    geo, q, kc, vc, bt, cl = _tiny_weight_case()
    ref = oracle.decode(q, kc, vc, bt, cl, 0.125, geo)
    dev = dict(q=torch.from_numpy(q).to(cuda),
               k=torch.from_numpy(kc).view(geo.k_shape).to(cuda), v=torch.from_numpy(vc).view(geo.v_shape).to(cuda),
               bt=torch.from_numpy(bt).to(cuda), cl=torch.from_numpy(cl).to(cuda))
    for psize in (-3, -2, -1, 0, 512):
        out = pa.paged_attention_decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], 0.125,
                                        out_dtype=torch.float32, partition_size=psize)
        torch.cuda.synchronize()
        err = float(np.abs(out.cpu().numpy() - ref).max())
        _say(f"[gpu] tiny fp16 weights, partition_size={psize}: max-abs error {err:.2e}")
        assert err <= 2e-4, psize
    pre = pa.paged_prefill(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"],
                           torch.tensor([0, 1], dtype=torch.int32, device=cuda), 0.125, out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = np.abs(pre.cpu().numpy() - ref[0])[0]
    _say(f"[gpu] tiny fp16 weights, one-token prefill: max-abs error {err.max():.2e}")
    bound = _one_rounding_bound(geo, q, kc, vc, bt, cl)
    assert (err <= bound).all(), (err.max(), bound.min())
    assert bound.max() < 1e-3  # well inside the 2e-3 parity tolerance


