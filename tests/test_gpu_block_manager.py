"""GPU: block tables and slot mappings from the prefix-caching block manager drive store, copy and decode.

Each token's K/V row is a seeded function of the token ids up to and including
it (as a real model's would be), so sequences sharing a prefix share rows and
may share cached blocks. The expected output of each sequence is the oracle's
dense attention over that sequence's own rows, with no cache involved.
"""

from __future__ import annotations

import hashlib

import numpy as np
import pytest

import oracle
from workloads import to_storage
from _gpu_helpers import np_to_torch
from test_gpu_shared_prefix import expected_words

pytestmark = pytest.mark.gpu

HKV, G, D, BS = 2, 4, 128, 16


def _rows(prefix):
    """Seeded (k, v) rows [HKV, D] for the last token of `prefix`."""
    seed = int.from_bytes(hashlib.sha256(np.asarray(prefix, np.int64).tobytes()).digest()[:8], "little")
    rng = np.random.default_rng(seed)
    return (to_storage(rng.standard_normal((HKV, D), dtype=np.float32), "bf16"),
            to_storage(rng.standard_normal((HKV, D), dtype=np.float32), "bf16"))


def test_manager_tables_drive_store_copy_and_decode(cuda):
    import torch
    import paged_attention_decode_amd as pa

    nb = 64
    m = pa.BlockManager(nb, BS)
    k_cache, v_cache = pa.allocate_kv_cache(nb, HKV, D, BS, torch.bfloat16, cuda)
    k_cache.fill_(float("nan"))
    v_cache.fill_(float("nan"))
    rng = np.random.default_rng(0)
    base = rng.integers(0, 1000, 50).tolist()
    prompts = {0: base, 1: base[:40] + rng.integers(0, 1000, 25).tolist(), 3: base[:33]}
    seqs = {}

    def store(sid, first):
        toks = seqs[sid]
        if first >= len(toks):
            return
        ks, vs = zip(*[_rows(toks[:t + 1]) for t in range(first, len(toks))])
        slots = torch.tensor(m.slots(sid, first, len(toks) - first), dtype=torch.int32, device=cuda)
        pa.store_kvcache(np_to_torch(np.stack(ks), "bf16").to(cuda), np_to_torch(np.stack(vs), "bf16").to(cuda),
                         slots, k_cache, v_cache)

    for sid, p in prompts.items():
        cached = m.add_sequence(sid, p)
        seqs[sid] = list(p)
        store(sid, cached)
    assert m.stats()["hits"] >= 4          # seq 1 and seq 3 reuse seq 0's leading blocks
    m.fork(0, 2)                            # parallel sample: shares seq 0's partial last block
    seqs[2] = list(seqs[0])
    copies = 0
    for step in range(20):                  # decode steps: one new token per sequence
        for sid in sorted(seqs):
            tok = int(rng.integers(0, 1000))
            slot, copy = m.append_token(sid, tok)
            if copy is not None:
                copies += 1
                pa.copy_blocks(k_cache, v_cache, torch.tensor([copy[0]], dtype=torch.int32, device=cuda),
                               torch.tensor([copy[1]], dtype=torch.int32, device=cuda))
            seqs[sid].append(tok)
            store(sid, len(seqs[sid]) - 1)
    assert copies >= 1

    order = sorted(seqs)
    mb = max(len(m.block_table(s)) for s in order)
    tables = np.zeros((len(order), mb), np.int32)
    for i, s in enumerate(order):
        t = m.block_table(s)
        tables[i, :len(t)] = t
    lens = np.array([len(seqs[s]) for s in order], np.int32)
    q = to_storage(rng.standard_normal((len(order), HKV * G, D), dtype=np.float32), "bf16")
    scale = 1.0 / np.sqrt(D)
    # the four sequences form one shared-prefix window (G = 4); 1, 2 and 3 share seq 0's leading
    # blocks (prefix-cache hits and a fork), so the option groups them
    for psize, shared in ((-3, False), (-2, False), (-1, False), (0, False), (16, False), (-2, True), (16, True)):
        ws = None
        if shared:
            plan = pa.decode_plan(len(order), HKV * G, HKV, D, BS, mb, pa.DTYPE_BF16, psize, 0, shared_prefix=True)
            ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device=cuda)
        out = pa.paged_attention_decode(np_to_torch(q, "bf16").to(cuda), k_cache, v_cache,
                                        torch.from_numpy(tables).to(cuda), torch.from_numpy(lens).to(cuda), scale,
                                        out_dtype=torch.float32, partition_size=psize, shared_prefix=shared,
                                        workspace=ws)
        torch.cuda.synchronize()
        if shared:
            # the sharing words are the workspace's last num_seqs int32 values (256-byte aligned)
            tail = (len(order) * 4 + 255) // 256 * 256
            end = plan["workspace_bytes"] - tail + len(order) * 4
            words = ws[end - len(order) * 4:end].cpu().view(torch.int32).numpy()
            want = expected_words(tables, lens, BS, G, nb, mb)
            assert words.tolist() == want.tolist() and (want != 0).all(), (words, want)
        out = out.cpu().numpy()
        for i, s in enumerate(order):
            toks = seqs[s]
            ks, vs = zip(*[_rows(toks[:t + 1]) for t in range(len(toks))])
            kd = oracle.widen(np.stack(ks), "bf16")
            vd = oracle.widen(np.stack(vs), "bf16")
            ref = oracle.decode_sequence(oracle.widen(q[i], "bf16"), kd, vd, scale)
            assert np.abs(out[i] - ref).max() <= 2e-3, (psize, shared, s)
    m.close()
