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


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_of_one_token_matches_decode(cuda, d):
    import torch
    import paged_attention_decode_amd as pa
    x = make_inputs(custom_config(dtype="bf16", batch=5, hq=16, hkv=4, d=d, lens=(1, 77, 300, 16, 1000), seed=9))
    dev = to_device(x, cuda)
    qs = torch.arange(6, dtype=torch.int32, device=cuda)
    pre = pa.paged_prefill(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"], qs,
                           x.scale, out_dtype=torch.float32)
    dec = pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                    dev["context_lens"], x.scale, out_dtype=torch.float32, partition_size=-1)
    torch.cuda.synchronize()
    diff = (pre - dec).abs().cpu().numpy()
    print(f"[gpu] one-token prefill vs decode, head_dim {d}: max diff {diff.max():.2e}", flush=True)
    # Both kernels (per-wavefront at head_dim 64, workgroup-shared at 128) split the weights the same
    # way (bf16 value + remainder, rounded to nearest); they differ only in fp32 summation order and
    # the exp2 argument's rounding.
    assert diff.max() <= 2e-5, diff.max()


def _set_v(x, s, t, value_bits):
    """Set every value element of token t of sequence s (all kv heads, dims) to one bf16 pattern."""
    geo = geometry(x)
    v5 = x.v_cache.reshape(geo.v_shape)
    blk = int(x.block_tables[s][t // geo.block_size])
    v5[blk, :, (t % geo.block_size) // 4, :, t % 4] = value_bits


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_prefill_with_large_values(cuda, d):
    """bf16 values far beyond fp16's range (65536 .. 131072) among ordinary ones, at both head dims:
    outputs reach hundreds, and the weights' value + remainder pair (relative error <= 2^-16) keeps
    the error within 2e-3 plus 4 * 2^-16 * sum_t w_t |v_t|."""
    import torch
    import paged_attention_decode_amd as pa
    dt, hq, hkv = "bf16", 8, 2
    lens, news = (300, 200, 64), (300, 50, 64)
    x = make_inputs(custom_config(dtype=dt, batch=3, hq=hq, hkv=hkv, d=d, lens=lens, seed=404))
    for s, t, bits in ((0, 37, 0x4780), (0, 38, 0xC780), (0, 299, 0x4800), (1, 5, 0x47C0), (1, 120, 0x477F),
                       (2, 63, 0x4780)):
        _set_v(x, s, t, bits)
    rng = np.random.default_rng(404)
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = to_storage(rng.standard_normal((int(qs[-1]), hq, d), dtype=np.float32), dt)
    dev = to_device(x, cuda)
    out = pa.paged_prefill(np_to_torch(q, dt).to(cuda), dev["k_cache"], dev["v_cache"], dev["block_tables"],
                           dev["context_lens"], torch.from_numpy(qs).to(cuda), x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    ref = oracle.prefill(q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, qs, x.scale, geometry(x))
    # sum_t w_t |v_t| per (query row, head, dim): the oracle's output over |V| (sign bits cleared).
    mag = oracle.prefill(q, x.k_cache, x.v_cache & np.uint16(0x7FFF), x.block_tables, x.context_lens, qs, x.scale,
                         geometry(x))
    err = np.abs(out - ref)
    print(f"[gpu] bf16 large values, head_dim {d}: max err {err.max():.3e}, max |out| {np.abs(ref).max():.1f}",
          flush=True)
    assert (err <= 2e-3 + 4 * 2.0 ** -16 * mag).all(), (err - 2e-3 - 4 * 2.0 ** -16 * mag).max()
    assert np.abs(ref).max() > 100.0  # the large values do reach the output


@pytest.mark.parametrize("dt,d", [("fp16", 64), ("bf16", 128), ("bf16", 64)])
def test_prefill_with_large_logits(cuda, dt, d):
    """Logits in the thousands (log2 units): q and K scaled by 32 (exact, a power of two), so the
    running maximum jumps by hundreds from key to key and most rescales flush the accumulators.
    Covers the per-wavefront kernel (fp16 and bf16 at head_dim 64) and the workgroup-shared one
    (bf16 at 128) against the oracle, inside the score range the lazy rescale assumes."""
    import torch
    import paged_attention_decode_amd as pa
    from _paged_helpers import widen_np
    hq, hkv = 8, 2
    lens, news = (260, 97, 33), (260, 40, 33)
    x = make_inputs(custom_config(dtype=dt, batch=3, hq=hq, hkv=hkv, d=d, lens=lens, seed=505))
    x.k_cache = to_storage((widen_np(x.k_cache, dt) * 32.0).astype(np.float32), dt)
    rng = np.random.default_rng(505)
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = to_storage(32.0 * rng.standard_normal((int(qs[-1]), hq, d), dtype=np.float32), dt)
    dev = to_device(x, cuda)
    out = pa.paged_prefill(np_to_torch(q, dt).to(cuda), dev["k_cache"], dev["v_cache"], dev["block_tables"],
                           dev["context_lens"], torch.from_numpy(qs).to(cuda), x.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = oracle.prefill(q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, qs, x.scale, geometry(x))
    err = np.abs(out - ref)
    # The logits' spread, in log2 units: the scores the kernel's running maximum tracks.
    geo = geometry(x)
    kk, _ = oracle.gather_kv(x.k_cache, x.v_cache, x.block_tables[0], int(lens[0]), geo)
    spread = np.abs(widen_np(q[:news[0]], dt)[:, 0] @ kk[:, 0].T).max() * x.scale / np.log(2.0)
    print(f"[gpu] large logits {dt} head_dim {d}: max |logit| {spread:.0f} (log2), max err {err.max():.2e}",
          flush=True)
    assert spread > 1000.0
    assert np.isfinite(out[: int(qs[-1])]).all()
    assert (err <= TOL[dt]).all(), err.max()


@pytest.mark.parametrize("dt,hq,d", [("bf16", 16, 128), ("fp16", 32, 64)])
def test_prefill_repeats_and_graph_replays_are_bit_identical(cuda, dt, hq, d):
    """Both prefill kernels take their work items from counters that every launch sets back to zero
    when it ends, and each call takes the next of 1024 counter sets. With more items than resident
    workgroups (so most come from the counters), 1030 calls in a row (every set used, then reused)
    and four replays of a captured call, each into a NaN-filled output with eager work between,
    give the same bits as the first call, which matches the oracle on its short sequences (a
    skipped item would leave NaN)."""
    import torch
    import paged_attention_decode_amd as pa
    lens = (2000, 1500, 1000, 700, 33, 1)
    x = make_inputs(custom_config(dtype=dt, batch=len(lens), hq=hq, hkv=8, d=d, lens=lens, seed=808))
    rng = np.random.default_rng(808)
    qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = to_storage(rng.standard_normal((int(qs[-1]), hq, d), dtype=np.float32), dt)
    dev = to_device(x, cuda)
    qd = np_to_torch(q, dt).to(cuda)
    qsd = torch.from_numpy(qs).to(cuda)
    out = torch.empty((int(qs[-1]), hq, d), dtype=torch.float32, device=cuda)

    def call():
        pa.paged_prefill(qd, dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"], qsd, x.scale,
                         out)

    out.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    first = out.cpu().numpy().copy()
    assert np.isfinite(first).all()
    short = [3, 4, 5]
    ref = oracle.prefill(q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, qs, x.scale, geometry(x),
                         seqs=short)
    for s_ in short:
        rows = slice(qs[s_], qs[s_ + 1])
        assert np.abs(first[rows] - ref[rows]).max() <= TOL[dt], s_
    first_d = torch.from_numpy(first).to(cuda)
    for i in range(1030):
        out.fill_(float("nan"))
        call()
        # bit equality on the device (NaN-free by the first call's check, so equal means equal bits)
        assert torch.equal(out.view(torch.int32), first_d.view(torch.int32)), f"call {i}"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == first.tobytes(), f"replay {rep}"
    print(f"[gpu] prefill repeats and replays, {dt} head_dim {d}: bit-identical", flush=True)


def test_prefill_calls_overlapping_on_two_streams(cuda):
    """Calls that run at the same time on one device take different counter sets. Two prefills with
    fewer workgroups than the device holds (so both can be resident together), one for each kernel
    (bf16 head_dim 128: workgroup-shared; fp16 head_dim 64: per wavefront), are launched 16 times
    each, alternating between two streams, into NaN-filled outputs of their own. Every output
    must have the bits of the same prefill run alone, which matches the oracle on its short
    sequences."""
    import torch
    import paged_attention_decode_amd as pa
    lens = (2000, 1500, 40, 1)
    short = [2, 3]
    probs = []
    for dt, d, seed in (("bf16", 128, 811), ("fp16", 64, 812)):
        x = make_inputs(custom_config(dtype=dt, batch=len(lens), hq=8, hkv=2, d=d, lens=lens, seed=seed))
        rng = np.random.default_rng(seed)
        qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        q = to_storage(rng.standard_normal((int(qs[-1]), 8, d), dtype=np.float32), dt)
        dev = to_device(x, cuda)
        args = (np_to_torch(q, dt).to(cuda), dev["k_cache"], dev["v_cache"], dev["block_tables"],
                dev["context_lens"], torch.from_numpy(qs).to(cuda), x.scale)
        alone = torch.full((int(qs[-1]), 8, d), float("nan"), dtype=torch.float32, device=cuda)
        pa.paged_prefill(*args, alone)
        torch.cuda.synchronize()
        got = alone.cpu().numpy()
        assert np.isfinite(got).all(), dt
        ref = oracle.prefill(q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, qs, x.scale, geometry(x),
                             seqs=short)
        for s_ in short:
            rows = slice(qs[s_], qs[s_ + 1])
            assert np.abs(got[rows] - ref[rows]).max() <= TOL[dt], (dt, s_)
        outs = [torch.full_like(alone, float("nan")) for _ in range(16)]
        probs.append((dt, args, alone, outs))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for i in range(16):
        for (dt, args, alone, outs), st in zip(probs, streams):
            with torch.cuda.stream(st):
                pa.paged_prefill(*args, outs[i])
    torch.cuda.synchronize()
    for dt, args, alone, outs in probs:
        for i, o in enumerate(outs):
            assert torch.equal(o.view(torch.int32), alone.view(torch.int32)), (dt, i)
    print("[gpu] prefill on two streams at once: every call bit-identical to a call alone", flush=True)


def test_prefill_without_items_leaves_out_and_its_counters_clean(cuda):
    """Every context empty (no work items): 1025 launches, enough to use every one of the 1024
    counter sets, leave out untouched and their counters at zero, so a real call afterwards on a
    recycled set matches the oracle."""
    import torch
    import paged_attention_decode_amd as pa
    dt, hq, hkv, d = "bf16", 8, 2, 128
    lens = (300, 120, 45)
    x = make_inputs(custom_config(dtype=dt, batch=len(lens), hq=hq, hkv=hkv, d=d, lens=lens, seed=909))
    rng = np.random.default_rng(909)
    qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = to_storage(rng.standard_normal((int(qs[-1]), hq, d), dtype=np.float32), dt)
    dev = to_device(x, cuda)
    qd = np_to_torch(q, dt).to(cuda)
    qsd = torch.from_numpy(qs).to(cuda)
    zero_lens = torch.zeros_like(dev["context_lens"])
    out = torch.full((int(qs[-1]), hq, d), float("nan"), dtype=torch.float32, device=cuda)
    for _ in range(1025):
        pa.paged_prefill(qd, dev["k_cache"], dev["v_cache"], dev["block_tables"], zero_lens, qsd, x.scale, out)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    pa.paged_prefill(qd, dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"], qsd, x.scale, out)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, qs, x.scale, geometry(x))
    assert np.abs(out.cpu().numpy() - ref).max() <= TOL[dt]


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
