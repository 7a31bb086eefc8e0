"""Properties of the seeded workload generator (host logic, CPU only)."""

from __future__ import annotations

import numpy as np
import pytest

from workloads import CONFIG_ORDER, get_config, make_inputs


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_block_tables_are_valid(name):
    cfg = get_config(name)
    x = make_inputs(cfg, structure_only=True)
    bs = cfg.block_size
    assert x.block_tables.shape == (cfg.batch, cfg.max_blocks_per_seq)
    assert x.block_tables.dtype == np.int32 and x.context_lens.dtype == np.int32
    assert (x.block_tables >= 0).all() and (x.block_tables < x.num_blocks).all()
    used = []
    for s in range(cfg.batch):
        nb = -(-int(x.context_lens[s]) // bs)
        used.extend(x.block_tables[s, :nb].tolist())
    shared = set(x.shared_blocks)
    private = [b for b in used if b not in shared]
    assert len(private) == len(set(private)), "private blocks must not repeat"
    assert not (set(used) & set(x.unused_blocks))
    assert len(set(used)) + len(x.unused_blocks) <= x.num_blocks


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_store_slots_unique_and_at_last_position(name):
    cfg = get_config(name)
    x = make_inputs(cfg, structure_only=True)
    bs = cfg.block_size
    assert len(set(x.slot_mapping.tolist())) == cfg.batch
    for s in range(cfg.batch):
        pos = int(x.context_lens[s]) - 1
        assert x.slot_mapping[s] == x.block_tables[s, pos // bs] * bs + pos % bs
        assert x.slot_mapping[s] // bs not in set(x.shared_blocks)


def test_empty_contexts_store_nothing():
    # An empty context has no position L-1: its slot is -1 (skipped), so two empty sequences never
    # share a slot and the fused step (which writes position L-1) and store_kvcache agree.
    from workloads import Config
    cfg = Config(name="custom", dtype="bf16", batch=6, num_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                 lengths="list", len_list=(0, 5, 0, 64, 3, 1), seed=1)
    x = make_inputs(cfg, structure_only=True)
    assert x.slot_mapping.tolist()[0] == -1 and x.slot_mapping.tolist()[2] == -1
    live = [int(v) for v, L in zip(x.slot_mapping, x.context_lens) if L > 0]
    assert all(v >= 0 for v in live) and len(set(live)) == len(live)


def test_length_distributions():
    c = make_inputs(get_config("tiny_fp32"), structure_only=True)
    assert c.context_lens.tolist() == [1, 17, 33, 64] and c.num_blocks == 32
    q = make_inputs(get_config("qwen3_0p6b_bf16"), structure_only=True).context_lens
    assert q.min() >= 32 and q.max() <= 288
    l3 = make_inputs(get_config("llama32_1b_fp16"), structure_only=True).context_lens
    assert l3.min() >= 512 and l3.max() <= 4096 and 1800 < l3.mean() < 2800
    l4 = make_inputs(get_config("long_ctx_bf16"), structure_only=True).context_lens
    assert (l4 == 32768).all()
    l5 = make_inputs(get_config("skewed_prefix_bf16"), structure_only=True).context_lens
    assert l5.min() >= 1 and l5.max() <= 16384 and 700 < np.median(l5) < 1500


def test_prefix_sharing_structure():
    cfg = get_config("skewed_prefix_bf16")
    x = make_inputs(cfg, structure_only=True)
    bs, grp, pre = cfg.block_size, cfg.prefix_group, cfg.prefix_tokens // cfg.block_size
    for g0 in range(0, cfg.batch, grp):
        rows = range(g0, g0 + grp)
        nshared = {s: min(pre, (int(x.context_lens[s]) - 1) // bs) for s in rows}
        longest = max(rows, key=lambda s: nshared[s])
        for s in rows:
            k = nshared[s]
            assert (x.block_tables[s, :k] == x.block_tables[longest, :k]).all()
            nb = -(-int(x.context_lens[s]) // bs)
            assert not set(x.block_tables[s, k:nb].tolist()) & set(x.shared_blocks)
    assert x.unique_kv_bytes < x.kv_bytes


def test_generation_is_deterministic_and_seeded():
    cfg = get_config("tiny_fp32")
    a, b = make_inputs(cfg), make_inputs(cfg)
    assert a.k_cache.tobytes() == b.k_cache.tobytes() and a.q.tobytes() == b.q.tobytes()
    c = make_inputs(cfg, seed=99)
    assert a.k_cache.tobytes() != c.k_cache.tobytes()
    s = make_inputs(cfg, structure_only=True)
    assert (s.block_tables == a.block_tables).all() and (s.slot_mapping == a.slot_mapping).all()


def test_values_are_rounded_normal_draws():
    x = make_inputs(get_config("qwen3_0p6b_bf16"))
    import torch
    v = torch.from_numpy(x.k_cache[:200000].view(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(v.mean()) < 0.02 and abs(v.std() - 1) < 0.02
    assert x.k_cache.size == x.num_blocks * 8 * 256 * 128
