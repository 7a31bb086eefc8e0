"""GPU parity at the size limits: the largest batch the library accepts, and caches past 4 GiB.

Both compare against the oracle on the same seeded inputs.
- 16383 sequences. This is the largest batch: the split modes keep a per-sequence prefix in LDS,
  64 KiB at this size. With shared prefixes, 8191 sequences (sharing words beside the prefix).
- Caches of about 4.3 GiB each. A small case's blocks are relabelled to ids whose byte offsets
  pass 2^32, so the store, decode, prefill and block copy address them with 64-bit offsets. The
  oracle runs on the small case itself; relabelling blocks does not change attention.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import make_inputs, to_storage
from _gpu_helpers import TOL, custom_config, geometry, np_to_torch, oracle_after_store, to_device, torch_dtype

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_largest_batch_in_every_mode(cuda):
    import torch
    import paged_attention_decode_amd as pa
    rng = np.random.default_rng(16383)
    lens = tuple(int(v) for v in rng.integers(1, 41, 16383))
    x = make_inputs(custom_config(dtype="bf16", batch=len(lens), hq=8, hkv=2, d=128, bs=16, lens=lens, seed=16383))
    dev = to_device(x, cuda)
    seqs = list(range(0, len(lens), 181)) + [len(lens) - 1]
    _, _, ref = oracle_after_store(x, seqs=seqs)
    for psize in (0, -3, -2, -1, 512):
        _say(f"[gpu] 16383 sequences, partition_size={psize}")
        k_cache, v_cache = dev["k_cache"].clone(), dev["v_cache"].clone()
        pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], k_cache, v_cache)
        out = pa.paged_attention_decode(dev["q"], k_cache, v_cache, dev["block_tables"], dev["context_lens"],
                                        x.scale, out_dtype=torch.float32, partition_size=psize)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        assert np.abs(out[seqs] - ref[seqs]).max() <= TOL["bf16"], psize
    # prefill of one new token per sequence over the same caches (after the store)
    _say("[gpu] 16383 sequences, prefill")
    k2, v2, _ = oracle_after_store(x, seqs=[])
    dk = np_to_torch(k2, "bf16").view(dev["k_cache"].shape).to(cuda)
    dv = np_to_torch(v2, "bf16").view(dev["v_cache"].shape).to(cuda)
    qs = torch.arange(len(lens) + 1, dtype=torch.int32, device=cuda)
    pre = pa.paged_prefill(dev["q"], dk, dv, dev["block_tables"], dev["context_lens"], qs, x.scale,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    pre = pre.cpu().numpy()
    assert np.abs(pre[seqs] - ref[seqs]).max() <= TOL["bf16"]


def test_largest_batch_with_shared_prefixes(cuda):
    """8191 sequences, the largest batch for shared prefixes (prefix sums and sharing words fill
    64 KiB of LDS), in groups of 8 sharing their first blocks: sampled rows against the oracle,
    in the balanced and a fixed mode."""
    import torch
    import paged_attention_decode_amd as pa
    rng = np.random.default_rng(8191)
    lens = tuple(int(v) for v in rng.integers(1, 100, 8191))
    x = make_inputs(custom_config(dtype="bf16", batch=len(lens), hq=4, hkv=2, d=128, bs=16, lens=lens, seed=8191,
                                  prefix_group=8, prefix_tokens=64))
    dev = to_device(x, cuda)
    plan = pa.decode_plan(len(lens), 4, 2, 128, 16, x.block_tables.shape[1], pa.DTYPE_BF16, -2, 0,
                          shared_prefix=True)
    assert plan["shared_prefix_window"] == 8
    seqs = list(range(0, len(lens), 97)) + [len(lens) - 1]
    k2, v2, ref = oracle_after_store(x, seqs=seqs)
    pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
    for psize in (-2, 64):
        _say(f"[gpu] 8191 sequences with shared prefixes, partition_size={psize}")
        out = pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                        dev["context_lens"], x.scale, out_dtype=torch.float32, partition_size=psize,
                                        shared_prefix=True)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        assert np.abs(out[seqs] - ref[seqs]).max() <= TOL["bf16"], psize


def test_caches_past_4_gib(cuda):
    import torch
    import paged_attention_decode_amd as pa
    dt, hq, hkv, d, bs = "bf16", 4, 1, 128, 16
    x = make_inputs(custom_config(dtype=dt, batch=3, hq=hq, hkv=hkv, d=d, bs=bs, lens=(40, 300, 17), seed=42))
    nb = x.num_blocks
    block_bytes = hkv * bs * d * 2
    offset = (1 << 32) // block_bytes + 12345          # first relabelled block starts past 4 GiB
    nb_big = offset + nb + 8
    _say(f"[gpu] caches of {nb_big} blocks ({nb_big * block_bytes / 2**30:.2f} GiB each), blocks relabelled by "
         f"+{offset}")
    tdt = torch_dtype(dt)
    k_big = torch.empty(pa.k_cache_shape(nb_big, hkv, d, bs, tdt), dtype=tdt, device=cuda)
    v_big = torch.empty(pa.v_cache_shape(nb_big, hkv, d, bs), dtype=tdt, device=cuda)
    dev = to_device(x, cuda)
    k_big[offset:offset + nb].copy_(dev["k_cache"])
    v_big[offset:offset + nb].copy_(dev["v_cache"])
    bt = dev["block_tables"] + offset
    slots = dev["slot_mapping"] + offset * bs

    # store + decode in every mode, against the oracle's small case
    _, _, ref = oracle_after_store(x)
    for psize in (0, -3, -2, -1, 16):
        k_c, v_c = k_big.clone(), v_big.clone()
        pa.store_kvcache(dev["k_new"], dev["v_new"], slots, k_c, v_c)
        out = pa.paged_attention_decode(dev["q"], k_c, v_c, bt, dev["context_lens"], x.scale,
                                        out_dtype=torch.float32, partition_size=psize)
        torch.cuda.synchronize()
        assert np.abs(out.cpu().numpy() - ref).max() <= TOL[dt], psize
        del k_c, v_c
        torch.cuda.empty_cache()

    # the store wrote exactly the relabelled slots
    k2, v2, _ = oracle_after_store(x, seqs=[])
    pa.store_kvcache(dev["k_new"], dev["v_new"], slots, k_big, v_big)
    torch.cuda.synchronize()
    kb = k_big[offset:offset + nb].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    vb = v_big[offset:offset + nb].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    assert kb.tobytes() == k2.tobytes() and vb.tobytes() == v2.tobytes()

    # causal prefill of whole prompts over the relabelled blocks
    lens = x.context_lens.astype(np.int64)
    qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = to_storage(np.random.default_rng(5).standard_normal((int(qs[-1]), hq, d), dtype=np.float32), dt)
    pre = pa.paged_prefill(np_to_torch(q, dt).to(cuda), k_big, v_big, bt, dev["context_lens"],
                           torch.from_numpy(qs).to(cuda), x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_p = oracle.prefill(q, k2, v2, x.block_tables, x.context_lens, qs, x.scale, geometry(x))
    assert np.abs(pre.cpu().numpy() - ref_p).max() <= TOL[dt]

    # a block copy between two ids past 4 GiB is a bit copy
    src, dst = offset + int(x.block_tables[1, 0]), offset + nb + 3
    pa.copy_blocks(k_big, v_big, torch.tensor([src], dtype=torch.int32, device=cuda),
                   torch.tensor([dst], dtype=torch.int32, device=cuda))
    torch.cuda.synchronize()
    assert torch.equal(k_big[dst].view(torch.int16), k_big[src].view(torch.int16))
    assert torch.equal(v_big[dst].view(torch.int16), v_big[src].view(torch.int16))
