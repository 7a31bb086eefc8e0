"""GPU parity on seeded random shapes: decode (every partition mode), the fused step, prefill, and
multi-token stores.

Each case draws a dtype, head_dim, block size, kv heads, group size (including sizes that do not
divide 16 and groups above 16), a batch, and context lengths mixing 0, 1, tile and block edges
and random values. It then checks:
- store + decode against the oracle (fp32 output: the dtype's bound; 16-bit output: the bound
  plus half an ulp);
- the fused step, bit for bit against store + decode in the same mode;
- a causal prefill of a random number of new tokens per sequence, over the cache after the
  store, against the oracle.
The draws are fixed by the case number, so a failure names its shape.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import make_inputs, to_storage
from _gpu_helpers import TOL, custom_config, geometry, half_ulp, np_to_torch, oracle_after_store, to_device, \
    torch_dtype, torch_to_np

pytestmark = pytest.mark.gpu

NUM_CASES = 40


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def draw(case: int) -> dict:
    rng = np.random.default_rng(90000 + case)
    dt = str(rng.choice(["fp32", "fp16", "bf16"]))
    d = int(rng.choice([64, 128, 256]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 17, 20]))
    b = int(rng.integers(1, 8))
    lens = []
    for _ in range(b):
        kind = rng.integers(0, 5)
        if kind == 0:
            lens.append(int(rng.choice([0, 1])))
        elif kind == 1:
            lens.append(max(1, int(rng.integers(1, 5)) * bs + int(rng.choice([-1, 0, 1]))))
        elif kind == 2:
            lens.append(max(1, int(rng.integers(1, 20)) * 16 + int(rng.choice([-1, 0, 1]))))
        else:
            lens.append(int(rng.integers(1, 600)))
    psize = int(rng.choice([0, -1, -2, -3, 16, 48, 512]))
    out_f32 = bool(rng.random() < 0.7)
    return dict(dt=dt, d=d, bs=bs, hkv=hkv, hq=hkv * g, b=b, lens=tuple(lens), psize=psize, out_f32=out_f32,
                seed=case)


@pytest.mark.parametrize("case", range(NUM_CASES))
def test_random_shape(cuda, case):
    import torch
    import paged_attention_decode_amd as pa
    p = draw(case)
    _say(f"[gpu] random case {case}: {p}")
    dt = p["dt"]
    x = make_inputs(custom_config(dtype=dt, batch=p["b"], hq=p["hq"], hkv=p["hkv"], d=p["d"], bs=p["bs"],
                                  lens=p["lens"], seed=p["seed"]))
    odt = torch.float32 if p["out_f32"] else torch_dtype(dt)
    k2, v2, ref = oracle_after_store(x)
    bound = TOL[dt] + (0.0 if p["out_f32"] else half_ulp(ref, dt))

    # store + decode
    dev = to_device(x, cuda)
    pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
    out = pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                    dev["context_lens"], x.scale, out_dtype=odt, partition_size=p["psize"])
    torch.cuda.synchronize()
    assert torch_to_np(dev["k_cache"], dt).reshape(-1).tobytes() == k2.reshape(-1).tobytes()
    assert torch_to_np(dev["v_cache"], dt).reshape(-1).tobytes() == v2.reshape(-1).tobytes()
    got = out.float().cpu().numpy()
    assert np.all(np.abs(got - ref) <= bound), float(np.abs(got - ref).max())

    # fused step: the same bits as store + decode
    dev_f = to_device(x, cuda)
    fused = pa.decode_step(dev_f["q"], dev_f["k_new"], dev_f["v_new"], dev_f["k_cache"], dev_f["v_cache"],
                           dev_f["block_tables"], dev_f["context_lens"], x.scale, out_dtype=odt,
                           partition_size=p["psize"])
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int32) if odt == torch.float32 else fused.view(torch.int16),
                       out.view(torch.int32) if odt == torch.float32 else out.view(torch.int16))
    assert torch.equal(dev_f["k_cache"].view(torch.int8), dev["k_cache"].view(torch.int8))
    assert torch.equal(dev_f["v_cache"].view(torch.int8), dev["v_cache"].view(torch.int8))

    # prefill of 0 .. min(L, 40) new tokens per sequence over the stored cache
    rng = np.random.default_rng(70000 + case)
    lens = x.context_lens.astype(np.int64)
    n = np.array([int(rng.integers(0, min(int(L), 40) + 1)) for L in lens], dtype=np.int64)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    t = int(qs[-1])
    if t == 0:
        return
    q = to_storage(rng.standard_normal((t, p["hq"], p["d"]), dtype=np.float32), dt)
    pre = pa.paged_prefill(np_to_torch(q, dt).to(cuda), dev["k_cache"], dev["v_cache"], dev["block_tables"],
                           dev["context_lens"], torch.from_numpy(qs).to(cuda), x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_p = oracle.prefill(q, k2, v2, x.block_tables, x.context_lens, qs, x.scale, geometry(x))
    assert np.abs(pre.cpu().numpy() - ref_p).max() <= TOL[dt]


@pytest.mark.parametrize("case", range(12))
def test_random_multi_token_store(cuda, case):
    """store_kvcache of many tokens (a prompt's worth): runs of consecutive slots, scattered
    slots, skipped (negative) slots and token rows wider than Hkv*D, bit for bit over the whole
    caches against the oracle's scatter."""
    import torch
    import paged_attention_decode_amd as pa
    rng = np.random.default_rng(80000 + case)
    dt = str(rng.choice(["fp32", "fp16", "bf16"]))
    d = int(rng.choice([64, 128, 256]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.integers(1, 5))
    nb = int(rng.integers(4, 24))
    num_slots = nb * bs
    # a run of consecutive slots (a prompt written in order), then scattered unique slots
    run = int(rng.integers(1, min(num_slots, 300) + 1))
    start = int(rng.integers(0, num_slots - run + 1))
    chosen = list(range(start, start + run))
    rest = [int(s) for s in rng.permutation(num_slots) if not start <= s < start + run]
    chosen += rest[:int(rng.integers(0, min(len(rest), 200) + 1))]
    slots = np.array(chosen, dtype=np.int32)
    slots[rng.random(len(slots)) < 0.1] = -1
    rng.shuffle(slots)
    n = len(slots)
    _say(f"[gpu] random store {case}: {dt} D={d} bs={bs} Hkv={hkv} blocks={nb} tokens={n}")
    geo = oracle.CacheGeometry(nb, hkv, d, bs, dt)
    elems = nb * hkv * bs * d
    k_cache = to_storage(rng.standard_normal(elems, dtype=np.float32), dt)
    v_cache = to_storage(rng.standard_normal(elems, dtype=np.float32), dt)
    pad = int(rng.choice([0, 8, 64]))
    k_rows = to_storage(rng.standard_normal((n, hkv * d + pad), dtype=np.float32), dt)
    v_rows = to_storage(rng.standard_normal((n, hkv * d + pad), dtype=np.float32), dt)
    k_new = np.ascontiguousarray(k_rows[:, :hkv * d]).reshape(n, hkv, d)
    v_new = np.ascontiguousarray(v_rows[:, :hkv * d]).reshape(n, hkv, d)
    k2, v2 = oracle.store_kvcache(k_new, v_new, slots, k_cache, v_cache, geo)

    tdt = torch_dtype(dt)
    kc = np_to_torch(k_cache, dt).view(pa.k_cache_shape(nb, hkv, d, bs, tdt)).to(cuda)
    vc = np_to_torch(v_cache, dt).view(pa.v_cache_shape(nb, hkv, d, bs)).to(cuda)
    kr = np_to_torch(k_rows, dt).to(cuda)
    vr = np_to_torch(v_rows, dt).to(cuda)
    kn = kr[:, :hkv * d].view(n, hkv, d)   # token stride hkv*d + pad
    vn = vr[:, :hkv * d].view(n, hkv, d)
    pa.store_kvcache(kn, vn, torch.from_numpy(slots).to(cuda), kc, vc)
    torch.cuda.synchronize()
    assert torch_to_np(kc, dt).reshape(-1).tobytes() == k2.reshape(-1).tobytes()
    assert torch_to_np(vc, dt).reshape(-1).tobytes() == v2.reshape(-1).tobytes()
