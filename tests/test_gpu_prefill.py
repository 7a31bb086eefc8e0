"""GPU parity of pa_paged_prefill (causal attention of new tokens over the paged cache) against the oracle."""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import make_inputs, to_storage
from _gpu_helpers import TOL, custom_config, geometry, half_ulp, np_to_torch, to_device, torch_dtype

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, Hq, Hkv, D, bs, context lengths, new tokens per sequence
    ("bf16", 8, 2, 128, 16, (40, 17, 100), (40, 17, 100)),        # full prefills
    ("bf16", 8, 2, 128, 16, (300, 64, 129), (37, 1, 64)),         # after cached tokens
    ("fp16", 32, 8, 64, 16, (200, 33), (200, 5)),                 # G = 4, head_dim 64
    ("fp32", 4, 4, 64, 32, (50, 3), (50, 3)),                     # G = 1
    ("bf16", 16, 2, 128, 256, (520, 9), (300, 9)),                # G = 8, big blocks
    ("bf16", 40, 2, 64, 16, (70, 31), (70, 2)),                   # G = 20: head groups 16 + 4
    ("fp16", 6, 2, 256, 64, (90, 130), (90, 17)),                 # odd G, head_dim 256
    ("bf16", 8, 2, 128, 16, (5, 0, 30), (5, 0, 30)),              # an empty sequence
    ("bf16", 16, 8, 128, 16, (700, 333), (700, 100)),             # many workgroup items per sequence
    ("fp16", 8, 8, 64, 32, (257, 64, 3), (257, 64, 3)),           # G = 1, partly idle workgroups
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_matches_oracle(cuda, case):
    import torch
    import paged_attention_decode_amd as pa
    dt, hq, hkv, d, bs, lens, news = CASES[case]
    print(f"[gpu] prefill case {CASES[case]}", flush=True)
    x = make_inputs(custom_config(dtype=dt, batch=len(lens), hq=hq, hkv=hkv, d=d, bs=bs, lens=lens, seed=300 + case))
    rng = np.random.default_rng(case)
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = to_storage(rng.standard_normal((int(qs[-1]), hq, d), dtype=np.float32), dt)
    dev = to_device(x, cuda)
    for out_dt in ("fp32", dt):
        out = pa.paged_prefill(np_to_torch(q, dt).to(cuda), dev["k_cache"], dev["v_cache"], dev["block_tables"],
                               dev["context_lens"], torch.from_numpy(qs).to(cuda), x.scale,
                               out_dtype=torch_dtype(out_dt))
        torch.cuda.synchronize()
        out = out.float().cpu().numpy()
        ref = oracle.prefill(q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, qs, x.scale, geometry(x))
        bound = TOL[dt] + (half_ulp(ref, dt) if out_dt != "fp32" else 0.0)
        assert (np.abs(out - ref) <= bound).all(), np.abs(out - ref).max()


def test_prefill_of_one_token_matches_decode(cuda):
    import torch
    import paged_attention_decode_amd as pa
    x = make_inputs(custom_config(dtype="bf16", batch=5, hq=16, hkv=4, lens=(1, 77, 300, 16, 1000), seed=9))
    dev = to_device(x, cuda)
    qs = torch.arange(6, dtype=torch.int32, device=cuda)
    pre = pa.paged_prefill(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"], qs,
                           x.scale, out_dtype=torch.float32)
    dec = pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                    dev["context_lens"], x.scale, out_dtype=torch.float32, partition_size=-1)
    torch.cuda.synchronize()
    # Both kernels split the weights the same way (bf16 value + remainder, rounded to nearest);
    # they differ only in fp32 summation order and the exp2 argument's rounding.
    diff = (pre - dec).abs().max().item()
    assert diff <= 2e-5, diff


def test_store_then_prefill_then_decode_chain(cuda):
    """A prompt stored and prefilled, then one decode step: both against the oracle."""
    import torch
    import paged_attention_decode_amd as pa
    dt, hq, hkv, d, bs = "bf16", 8, 2, 128, 16
    prompt = 75
    rng = np.random.default_rng(5)
    nb = 16
    k_cache, v_cache = pa.allocate_kv_cache(nb, hkv, d, bs, torch.bfloat16, cuda)
    k_cache.zero_()
    v_cache.zero_()
    table = rng.permutation(nb)[:8].astype(np.int32)
    kv = [to_storage(rng.standard_normal((prompt + 1, hkv, d), dtype=np.float32), dt) for _ in range(2)]
    slots = (table[np.arange(prompt + 1) // bs] * bs + np.arange(prompt + 1) % bs).astype(np.int32)
    pa.store_kvcache(np_to_torch(kv[0][:prompt], dt).to(cuda), np_to_torch(kv[1][:prompt], dt).to(cuda),
                     torch.from_numpy(slots[:prompt]).to(cuda), k_cache, v_cache)
    q = to_storage(rng.standard_normal((prompt + 1, hq, d), dtype=np.float32), dt)
    bt = torch.from_numpy(table[None, :].copy()).to(cuda)
    pre = pa.paged_prefill(np_to_torch(q[:prompt], dt).to(cuda), k_cache, v_cache, bt,
                           torch.tensor([prompt], dtype=torch.int32, device=cuda),
                           torch.tensor([0, prompt], dtype=torch.int32, device=cuda), 0.1, out_dtype=torch.float32)
    step = pa.decode_step(np_to_torch(q[prompt:], dt).to(cuda), np_to_torch(kv[0][prompt:], dt).to(cuda),
                          np_to_torch(kv[1][prompt:], dt).to(cuda), k_cache, v_cache, bt,
                          torch.tensor([prompt + 1], dtype=torch.int32, device=cuda), 0.1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    kd, vd = oracle.widen(kv[0], dt), oracle.widen(kv[1], dt)
    qf = oracle.widen(q, dt)
    for i in range(prompt + 1):
        ref = oracle.decode_sequence(qf[i], kd[:i + 1], vd[:i + 1], 0.1)
        got = pre[i].cpu().numpy() if i < prompt else step[0].cpu().numpy()
        assert np.abs(got - ref).max() <= 2e-3, i


def test_prefill_of_many_sequences_uses_the_per_wavefront_kernel(cuda):
    """8200 sequences: the shared variant's LDS (item prefix + step buffers) would pass 64 KiB, so
    the library takes the per-wavefront kernel; both must agree with the oracle."""
    import torch
    import paged_attention_decode_amd as pa
    rng = np.random.default_rng(77)
    lens = tuple(int(v) for v in rng.integers(1, 5, 8200))
    x = make_inputs(custom_config(dtype="bf16", batch=len(lens), hq=8, hkv=2, d=128, bs=16, lens=lens, seed=77))
    news = lens
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = to_storage(rng.standard_normal((int(qs[-1]), 8, 128), dtype=np.float32), "bf16")
    dev = to_device(x, cuda)
    print(f"[gpu] prefill of {len(lens)} sequences", flush=True)
    out = pa.paged_prefill(np_to_torch(q, "bf16").to(cuda), dev["k_cache"], dev["v_cache"], dev["block_tables"],
                           dev["context_lens"], torch.from_numpy(qs).to(cuda), x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    seqs = range(0, len(lens), 97)
    ref = oracle.prefill(q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, qs, x.scale, geometry(x),
                         seqs=list(seqs))
    for s_ in seqs:
        rows = slice(qs[s_], qs[s_ + 1])
        assert np.abs(out[rows] - ref[rows]).max() <= TOL["bf16"], s_


def test_malformed_query_start_stays_inside_the_buffers(cuda):
    """query_start lives on the device and is not checked on the host: starts past num_tokens,
    negative starts and decreasing ends are clamped, so q and out outside the described rows are
    never touched. Rows of well-formed sequences are still correct."""
    import torch
    import paged_attention_decode_amd as pa
    x = make_inputs(custom_config(dtype="bf16", batch=4, hq=8, hkv=2, d=128, bs=16, lens=(40, 60, 30, 50), seed=91))
    dev = to_device(x, cuda)
    num_tokens = 70
    # seq 0 starts at -5 (clamped to 0), seq 1 ends past num_tokens (clamped to 70), seq 2 starts
    # past num_tokens, seq 3 ends before it starts: after clamping, seqs 0 and 1 own rows 0..39
    # and 40..69, seqs 2 and 3 none
    qs = np.array([-5, 40, 1000, 70, 30], np.int32)
    rng = np.random.default_rng(91)
    q_host = to_storage(rng.standard_normal((num_tokens, 8, 128), dtype=np.float32), "bf16")
    # guard rows on both sides of q and out: a read or write outside [guard, guard + num_tokens)
    # would show there
    guard = 64
    q_big = torch.zeros((num_tokens + 2 * guard, 8, 128), dtype=torch.bfloat16, device=cuda)
    q_big[guard:guard + num_tokens] = np_to_torch(q_host, "bf16").to(cuda)
    out_big = torch.full((num_tokens + 2 * guard, 8, 128), 7.0, dtype=torch.float32, device=cuda)
    pa.paged_prefill(q_big[guard:guard + num_tokens], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                     dev["context_lens"], torch.from_numpy(qs).to(cuda), x.scale,
                     out=out_big[guard:guard + num_tokens])
    torch.cuda.synchronize()
    ob = out_big.cpu().numpy()
    assert (ob[:guard] == 7.0).all() and (ob[guard + num_tokens:] == 7.0).all()
    # the clamped rows are the last 40 and 30 queries of sequences 0 and 1
    ref = oracle.prefill(q_host, x.k_cache, x.v_cache, x.block_tables, x.context_lens,
                         np.array([0, 40, 70, 70, 70], np.int32), x.scale, geometry(x), seqs=[0, 1])
    assert np.abs(ob[guard:guard + num_tokens] - ref).max() <= TOL["bf16"]
