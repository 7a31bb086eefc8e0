"""GPU parity of shared-prefix decode (pa_decode_opts.shared_prefix) through the C ABI.

With the option, a detection kernel groups, in each window of 16 / G consecutive sequences,
those whose leading block-table entries are the same physical blocks, and the attention
kernel reads the group's common prefix once. The result must be the same attention:
- every case is compared with the oracle at the usual bounds;
- sharing patterns are built to catch a wrong detection. Members share exactly k blocks and
  then differ, so a prefix one block too long reads another sequence's K/V and fails parity.
  Patterns include chunk edges of the compare loop, leaders that are not first, two candidate
  groups in one window, excluded short members, all group sizes and block sizes;
- the detection's per-sequence words are read back from a caller workspace (they are its last
  num_seqs int32 values) and compared with a Python model of the rule in pagedattn.h;
- the fused step must equal store + decode bit for bit with the option on.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from workloads import get_config, make_inputs
from _gpu_helpers import TOL, custom_config, geometry, oracle_after_store, to_device, torch_to_np

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def expected_words(bt, lens, bs, group, num_blocks, max_blocks):
    """Sharing words by the rule stated for pa_decode_opts.shared_prefix (a model for the test)."""
    w = 16 // group
    b = len(lens)
    out = np.zeros(b, np.int64)
    if group > 8:
        return out
    clamp = lambda v: min(max(int(v), 0), num_blocks - 1)  # noqa: E731
    max_len = max_blocks * bs
    for s0 in range(0, b, w):
        n = min(w, b - s0)
        ls = [min(max(int(lens[s0 + m]), 0), max_len) for m in range(n)]
        cap = [(L - 1) // bs if L > 0 else 0 for L in ls]
        first = [clamp(bt[s0 + m][0]) for m in range(n)]
        cnt = [sum(1 for j in range(n) if cap[j] > 0 and first[j] == first[m]) if cap[m] > 0 else -1
               for m in range(n)]
        best = max(cnt)
        if best < 2:
            continue
        leader = cnt.index(best)
        share = [0] * n
        for m in range(n):
            if m == leader:
                share[m] = cap[m]
            elif cap[m] > 0 and first[m] == first[leader]:
                lim = min(cap[m], cap[leader])
                k = 0
                while k < lim and clamp(bt[s0 + m][k]) == clamp(bt[s0 + leader][k]):
                    k += 1
                share[m] = k
        saving = [0] * n
        for m in range(n):
            if m != leader and share[m] > 0:
                c = sum(1 for j in range(n) if j != leader and share[j] > 0 and share[j] >= share[m])
                saving[m] = c * share[m]
        top = max(saving)
        if top == 0:
            continue
        p = share[saving.index(top)]
        tpb = bs // 16
        p = min(p, 0xFFFF // tpb)
        pt = p * tpb
        if pt < 2:
            continue
        for m in range(n):
            if m == leader or share[m] >= p:
                out[s0 + m] = (1 << 20) | (leader << 16) | pt
    return out


def _decode(dev, x, psize, shared, workspace=None):
    import torch
    import paged_attention_decode_amd as pa
    out = pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                    dev["context_lens"], x.scale, out_dtype=torch.float32, partition_size=psize,
                                    shared_prefix=shared, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _with_sharing(cfg, groups, seed_tables=0):
    """Draw a batch without sharing, then make each group's members reuse the leading blocks of
    the group's first listed sequence: groups = [(source, [(member, n_blocks), ...]), ...]."""
    x = make_inputs(cfg)
    bt = x.block_tables.copy()
    for src, members in groups:
        for m, k in members:
            bt[m, :k] = bt[src, :k]
    x.block_tables = bt
    return x


def _decode_ref(x):
    return oracle.decode(x.q, x.k_cache, x.v_cache, x.block_tables, x.context_lens, x.scale, geometry(x))


# (name, dtype, Hq, Hkv, D, bs, lengths, groups)
CASES = [
    ("window of 8, all share 5 blocks", "bf16", 4, 2, 128, 16, (100, 90, 200, 150, 81, 300, 120, 97),
     [(0, [(m, 5) for m in range(1, 8)])]),
    ("mixed shares: best prefix excludes some", "bf16", 4, 2, 128, 16, (200, 180, 90, 170, 400, 60, 300, 250),
     [(0, [(1, 10), (2, 3), (3, 7), (4, 10), (5, 1), (6, 10), (7, 2)])]),
    ("leader is not the first slot", "bf16", 4, 2, 64, 16, (50, 99, 120, 140, 88, 130, 77, 150),
     [(1, [(m, 4) for m in range(2, 8)])]),
    ("two candidate groups, the larger wins", "fp16", 4, 2, 64, 16, (70, 99, 120, 140, 88, 130, 77, 150),
     [(0, [(1, 4), (2, 4)]), (3, [(4, 3), (5, 3), (6, 3), (7, 3)])]),
    ("G=1, window 16, ragged tail window", "bf16", 2, 2, 128, 16, tuple(range(40, 40 + 19 * 13, 13)),
     [(0, [(m, 2) for m in range(1, 16)]), (16, [(17, 2), (18, 2)])]),
    ("G=3, window 5", "bf16", 6, 2, 128, 32, (300, 280, 190, 333, 250, 260),
     [(0, [(1, 5), (2, 5), (3, 5), (4, 2)])]),
    ("G=4, window 4", "fp16", 8, 2, 64, 16, (100, 200, 300, 400, 120, 130, 140, 150),
     [(0, [(1, 6), (2, 6), (3, 6)]), (4, [(5, 7), (6, 7), (7, 7)])]),
    ("G=8, window 2", "fp32", 8, 1, 64, 16, (100, 200, 300, 90),
     [(0, [(1, 6)]), (2, [(3, 5)])]),
    ("G=16: sharing ignored", "bf16", 16, 1, 128, 16, (100, 200),
     [(0, [(1, 6)])]),
    ("block size 64: one block is four tiles", "bf16", 4, 2, 128, 64, (300, 260, 190, 400, 64, 65, 700, 129),
     [(0, [(1, 3), (2, 2), (3, 4), (4, 1), (5, 1), (6, 4), (7, 2)])]),
    ("block size 256 and short members", "bf16", 4, 2, 128, 256, (600, 513, 300, 256, 257, 1, 0, 900),
     [(0, [(1, 2), (2, 1), (3, 1), (4, 1), (5, 1), (6, 1), (7, 2)])]),
    ("shares across compare chunks (63, 64, 65, 256, 300 blocks)", "bf16", 2, 1, 128, 16,
     (6000, 5000, 5200, 4200, 5100, 5900, 1500, 2000),
     [(0, [(1, 63), (2, 64), (3, 65), (4, 256), (5, 300), (6, 70), (7, 93)])]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("psize", [-2, 0, 16, 64])
def test_constructed_sharing(cuda, case, psize):
    import torch
    import paged_attention_decode_amd as pa
    name, dt, hq, hkv, d, bs, lens, groups = CASES[case]
    _say(f"[gpu] shared prefix: {name}, partition_size={psize}")
    cfg = custom_config(dtype=dt, batch=len(lens), hq=hq, hkv=hkv, d=d, bs=bs, lens=lens, seed=300 + case)
    x = _with_sharing(cfg, groups)
    dev = to_device(x, cuda)
    plan = pa.decode_plan(len(lens), hq, hkv, d, bs, x.block_tables.shape[1], pa.DTYPE_BF16 if dt == "bf16" else
                          (pa.DTYPE_F16 if dt == "fp16" else pa.DTYPE_F32), psize, 0, shared_prefix=True)
    ws = torch.zeros(plan["workspace_bytes"] + 256, dtype=torch.uint8, device=cuda)
    out = _decode(dev, x, psize, True, workspace=ws)
    ref = _decode_ref(x)
    assert np.abs(out - ref).max() <= TOL[dt]
    if plan["shared_prefix_window"] > 0:
        nb = len(lens)
        tail = (nb * 4 + 255) // 256 * 256
        words = ws[plan["workspace_bytes"] - tail:plan["workspace_bytes"] - tail + nb * 4].cpu().view(torch.int32)
        want = expected_words(x.block_tables, x.context_lens, bs, hq // hkv, x.num_blocks, x.block_tables.shape[1])
        assert words.numpy().tolist() == want.tolist()
        if psize in (-2, 0) and case == 0:
            assert (want != 0).all()  # the whole window is one group
    else:
        assert hq // hkv > 8 or psize == 0


def test_identical_tables_share_only_blocks_before_the_last(cuda):
    """Equal rows and lengths: everything but the last-token block is shared, and the result
    still matches the oracle (the last block is read by each sequence itself)."""
    cfg = custom_config(dtype="bf16", batch=8, hq=4, hkv=2, d=128, bs=16, lens=(333,) * 8, seed=41)
    x = _with_sharing(cfg, [(0, [(m, 21) for m in range(1, 8)])])
    dev = to_device(x, cuda)
    out = _decode(dev, x, -2, True)
    assert np.abs(out - _decode_ref(x)).max() <= TOL["bf16"]


@pytest.mark.parametrize("psize", [-2, 0, 512])
def test_skewed_workload_with_shared_prefix(cuda, psize):
    """The prefix-sharing workload at full size: sampled sequences against the oracle, after the
    store, and the whole output against the run without the option."""
    import torch
    import paged_attention_decode_amd as pa
    from test_gpu_decode import _inputs, _sample_seqs
    x = _inputs("skewed_prefix_bf16")
    _say(f"[gpu] shared prefix: skewed workload, partition_size={psize}")
    dev = to_device(x, cuda)
    pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
    torch.cuda.synchronize()
    on = _decode(dev, x, psize, True)
    off = _decode(dev, x, psize, False)
    seqs = _sample_seqs(x, 24)
    _, _, ref = oracle_after_store(x, seqs=seqs)
    assert np.isfinite(on).all()
    assert np.abs(on[seqs] - ref[seqs]).max() <= TOL["bf16"]
    assert np.abs(on - off).max() <= 2 * TOL["bf16"]
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("psize", [-2, 16])
@pytest.mark.parametrize("dt,hq,hkv,d,bs", [("bf16", 16, 8, 128, 16), ("fp16", 8, 2, 64, 32), ("fp32", 4, 2, 64, 16)])
def test_fused_step_with_shared_prefix(cuda, psize, dt, hq, hkv, d, bs):
    """Groups of sequences sharing their first blocks (the generator's prefix sharing, new-token
    blocks private): the fused step equals store + decode bit for bit, and both the oracle."""
    import torch
    import paged_attention_decode_amd as pa
    rng = np.random.default_rng(hq + d + bs)
    lens = tuple(int(v) for v in rng.integers(1, 400, 24))
    cfg = custom_config(dtype=dt, batch=24, hq=hq, hkv=hkv, d=d, bs=bs, lens=lens, seed=77, prefix_group=16 // (hq // hkv),
                        prefix_tokens=128)
    x = make_inputs(cfg)
    _say(f"[gpu] shared prefix fused step {dt} Hq={hq} Hkv={hkv} D={d} bs={bs} partition_size={psize}")
    dev_a = to_device(x, cuda)
    pa.store_kvcache(dev_a["k_new"], dev_a["v_new"], dev_a["slot_mapping"], dev_a["k_cache"], dev_a["v_cache"])
    out_a = pa.paged_attention_decode(dev_a["q"], dev_a["k_cache"], dev_a["v_cache"], dev_a["block_tables"],
                                      dev_a["context_lens"], x.scale, out_dtype=torch.float32, partition_size=psize,
                                      shared_prefix=True)
    dev_b = to_device(x, cuda)
    out_b = pa.decode_step(dev_b["q"], dev_b["k_new"], dev_b["v_new"], dev_b["k_cache"], dev_b["v_cache"],
                           dev_b["block_tables"], dev_b["context_lens"], x.scale, out_dtype=torch.float32,
                           partition_size=psize, shared_prefix=True)
    torch.cuda.synchronize()
    assert torch_to_np(dev_b["k_cache"], dt).tobytes() == torch_to_np(dev_a["k_cache"], dt).tobytes()
    assert torch_to_np(dev_b["v_cache"], dt).tobytes() == torch_to_np(dev_a["v_cache"], dt).tobytes()
    assert out_b.cpu().numpy().tobytes() == out_a.cpu().numpy().tobytes()
    _, _, ref = oracle_after_store(x)
    assert np.abs(out_a.cpu().numpy() - ref).max() <= TOL[dt]


def test_workspace_without_sharing_room_is_rejected(cuda):
    """A caller workspace sized for the call without the option is too small with it."""
    import torch
    import paged_attention_decode_amd as pa
    cfg = custom_config(dtype="bf16", batch=8, hq=4, hkv=2, d=128, bs=16, lens=(100,) * 8, seed=5)
    x = _with_sharing(cfg, [(0, [(m, 4) for m in range(1, 8)])])
    dev = to_device(x, cuda)
    small = pa.workspace_bytes(8, 4, 2, 128, 16, x.block_tables.shape[1], pa.DTYPE_BF16, -2)
    ws = torch.empty(small, dtype=torch.uint8, device=cuda)
    with pytest.raises(pa.PagedAttnError, match="PA_ERR_WORKSPACE"):
        _decode(dev, x, -2, True, workspace=ws)


def test_shared_prompt_workload(cuda):
    """32 prompts of 4096 tokens sampled 8 times each: sampled sequences against the oracle after
    the store, with the option on, in the automatic mode the bench times."""
    import torch
    import paged_attention_decode_amd as pa
    from test_gpu_decode import _sample_seqs
    x = make_inputs(get_config("shared_prompt_bf16"))
    _say("[gpu] shared prefix: shared-prompt workload")
    dev = to_device(x, cuda)
    pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
    torch.cuda.synchronize()
    out = _decode(dev, x, 0, True)
    seqs = _sample_seqs(x, 12)
    _, _, ref = oracle_after_store(x, seqs=seqs)
    assert np.isfinite(out).all()
    assert np.abs(out[seqs] - ref[seqs]).max() <= TOL["bf16"]
    del dev
    torch.cuda.empty_cache()


def test_graph_capture_with_shared_prefix(cuda):
    """Store + decode with the option, recorded into a HIP graph (detection, attention and merge
    kernels): every replay, with eager work between replays, matches the eager step bit for bit,
    and a changed block table is picked up by the detection on replay."""
    import torch
    import paged_attention_decode_amd as pa
    rng = np.random.default_rng(12)
    lens = tuple(int(v) for v in rng.integers(40, 600, 16))
    cfg = custom_config(dtype="bf16", batch=16, hq=8, hkv=4, d=128, bs=16, lens=lens, seed=13, prefix_group=8,
                        prefix_tokens=256)
    x = make_inputs(cfg)
    c = x.cfg
    dev = to_device(x, cuda)
    need = pa.decode_plan(c.batch, c.num_heads, c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks_per_seq,
                          pa.DTYPE_BF16, -2, 0, shared_prefix=True)["workspace_bytes"]
    ws = torch.empty(need, dtype=torch.uint8, device=cuda)
    out = torch.empty((c.batch, c.num_heads, c.head_dim), dtype=torch.float32, device=cuda)

    def step():
        pa.store_kvcache(dev["k_new"], dev["v_new"], dev["slot_mapping"], dev["k_cache"], dev["v_cache"])
        pa.paged_attention_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                  dev["context_lens"], x.scale, out, workspace=ws, partition_size=-2,
                                  shared_prefix=True)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xA5)                   # the workspace needs no initialisation
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == eager.cpu().numpy().tobytes(), f"replay {rep}"
    _, _, ref = oracle_after_store(x)
    assert np.abs(eager.cpu().numpy() - ref).max() <= TOL["bf16"]
    # break the sharing of most of the second window in place (their first block becomes their own
    # last block): a replay must regroup
    tables = x.block_tables.copy()
    for m in range(9, 16):
        tables[m, 0] = tables[m, (int(x.context_lens[m]) - 1) // 16]
    dev["block_tables"].copy_(torch.from_numpy(tables))
    x2 = x
    x2.block_tables = tables
    g.replay()
    torch.cuda.synchronize()
    _, _, ref2 = oracle_after_store(x2)
    assert np.abs(out.cpu().numpy() - ref2).max() <= TOL["bf16"]
