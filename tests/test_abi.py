"""C-ABI surface on the CPU: the library loads, exports what the header declares, plans and validates on the host."""

from __future__ import annotations

import ctypes
import re
from pathlib import Path

import pytest

import paged_attention_decode_amd as pa

HEADER = Path(__file__).resolve().parents[1] / "include" / "pagedattn.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return pa.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("pa_store_kvcache", "pa_paged_attention_decode", "pa_paged_attention_decode_ex",
                     "pa_decode_plan", "pa_decode_workspace_bytes", "pa_last_error", "pa_version", "pa_shutdown"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in pagedattn.h but not exported"


def test_binding_constants_match_the_header():
    text = HEADER.read_text()
    m = re.search(r"#define\s+PA_DEFAULT_CACHED_PREFIX_TOKENS\s+(\d+)", text)
    assert m and int(m.group(1)) == pa.DEFAULT_CACHED_PREFIX_TOKENS
    m = re.search(r"#define\s+PA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pa.NOALLOC_SCRATCH_BYTES
    for name, code in (("PA_DTYPE_F32", pa.DTYPE_F32), ("PA_DTYPE_F16", pa.DTYPE_F16), ("PA_DTYPE_BF16", pa.DTYPE_BF16)):
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text), name


def test_version(lib):
    assert pa.version().startswith("libpagedattn") and "gfx950" in pa.version()


def _plan(**kw):
    args = dict(num_seqs=256, num_heads=16, num_kv_heads=8, head_dim=128, block_size=16, max_blocks_per_seq=1024,
                dtype_code=pa.DTYPE_BF16, partition_size=0, num_cus=256)
    args.update(kw)
    return pa.decode_plan(**args)


def test_plan_balanced_uses_resident_waves_and_reduce():
    p = _plan()
    assert p["uses_reduce"] and p["range_tokens"] == 0
    assert p["num_waves"] == 256 * 2 * 4
    # workspace: two partial rows per wave, G heads, D floats + lse, plus per-segment records
    rows = p["num_waves"] * 2 * 2
    assert p["workspace_bytes"] >= rows * 128 * 4 + rows * 4 + 256 * 8 * 16


def test_plan_one_pass_needs_no_workspace():
    p = _plan(partition_size=-1)
    assert not p["uses_reduce"] and p["workspace_bytes"] == 0 and p["range_tokens"] == -1
    assert p["num_waves"] == 256 * 8  # one wavefront per (sequence, kv head), fewer than resident


def test_plan_workgroup_split_uses_lds_not_a_workspace():
    # one workgroup of four wavefronts per (sequence, kv head) segment, up to the resident groups
    p = _plan(partition_size=-3)
    assert p["range_tokens"] == -3 and not p["uses_reduce"] and p["workspace_bytes"] == 0
    assert p["num_waves"] == 256 * 2 * 4  # 2048 segments, 512 resident workgroups
    small = _plan(num_seqs=3, num_heads=4, num_kv_heads=2, head_dim=64, max_blocks_per_seq=4, partition_size=-3,
                  dtype_code=pa.DTYPE_F32)
    assert small["num_waves"] == 3 * 2 * 4


def test_plan_workgroup_split_falls_back_where_lds_would_not_fit():
    # four partial rows of 16 heads x 256 dims (plus lse) exceed 64 KiB: one pass instead
    p = _plan(num_heads=32, num_kv_heads=2, head_dim=256, partition_size=-3)
    assert p["range_tokens"] == -1 and not p["uses_reduce"]
    q = _plan(num_heads=30, num_kv_heads=2, head_dim=256, partition_size=-3)
    assert q["range_tokens"] == -3


def test_plan_fixed_ranges_cover_the_upper_bound():
    p = _plan(num_seqs=4, num_heads=4, num_kv_heads=2, head_dim=64, max_blocks_per_seq=4, partition_size=32,
              dtype_code=pa.DTYPE_F32)
    upper_tiles = 4 * 2 * (4 * 16 // 16)
    assert p["range_tokens"] == 32 and p["num_waves"] >= upper_tiles // 2


def test_plan_fixed_ranges_loop_on_resident_waves():
    # 2048 segments x 1024 tiles in 32-tile ranges: 65536 possible ranges, looped over by the
    # resident wavefronts; the workspace still has two partial rows per possible range.
    p = _plan(partition_size=512)
    assert p["range_tokens"] == 512 and p["num_waves"] == 256 * 2 * 4
    ranges = 256 * 8 * 1024 // 32
    rows = ranges * 2 * 2
    assert p["workspace_bytes"] >= rows * 128 * 4 + rows * 4 + 256 * 8 * 16


def test_plan_small_batch_does_not_oversubscribe():
    p = _plan(num_seqs=4, num_heads=4, num_kv_heads=2, head_dim=64, max_blocks_per_seq=4, dtype_code=pa.DTYPE_F32,
              partition_size=-2)
    assert p["range_tokens"] == 0 and p["uses_reduce"]
    assert p["num_waves"] <= 16  # 32 tiles at most, at least 2 tiles per wavefront


@pytest.mark.parametrize("mb,bs,one_pass", [(32, 16, True), (2, 256, True), (33, 16, False), (4, 256, False),
                                            (1024, 16, False)])
def test_plan_automatic_takes_one_pass_for_short_bounded_contexts(mb, bs, one_pass):
    # the host's only bound on a context is max_blocks_per_seq * block_size: one pass up to 512 tokens
    p = _plan(max_blocks_per_seq=mb, block_size=bs)
    assert (p["range_tokens"] == -1) == one_pass
    assert p["uses_reduce"] != one_pass
    forced = _plan(max_blocks_per_seq=mb, block_size=bs, partition_size=-2)
    assert forced["range_tokens"] == 0 and forced["uses_reduce"]


@pytest.mark.parametrize("num_seqs,expect", [(60, -3), (64, -3), (65, -1), (2048, -1)])
def test_plan_automatic_short_contexts_split_in_workgroups_while_they_fit(num_seqs, expect):
    # 8 kv heads: 64 sequences give 512 segments, one resident workgroup each on 256 CUs (2 per CU)
    p = _plan(num_seqs=num_seqs, max_blocks_per_seq=2, block_size=256)
    assert p["range_tokens"] == expect and not p["uses_reduce"] and p["workspace_bytes"] == 0
    # where four partial rows would not fit in LDS (head_dim 256, 16 heads per kv head) it is one pass
    q = _plan(num_seqs=8, num_heads=32, num_kv_heads=2, head_dim=256, max_blocks_per_seq=2, block_size=256)
    assert q["range_tokens"] == -1


def test_plan_large_head_groups_split_into_sixteen():
    p = _plan(num_heads=40, num_kv_heads=2, partition_size=-1)
    assert p["num_waves"] == min(256 * 2 * 2, 256 * 8)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype_code=7), 2),
    (dict(num_heads=12, num_kv_heads=8), 3),
    (dict(head_dim=96), 4),
    (dict(head_dim=0), 3),
    (dict(block_size=8), 4),
    (dict(block_size=48), 4),
    (dict(num_seqs=-1), 3),
    (dict(num_seqs=16384), 4),
    (dict(max_blocks_per_seq=0), 3),
    (dict(partition_size=24), 3),
    (dict(partition_size=-4), 3),
])
def test_plan_rejects_bad_sizes(kw, code):
    with pytest.raises(pa.PagedAttnError) as ei:
        _plan(**kw)
    assert ei.value.code == code
    assert pa.load_library().pa_last_error().decode()


def _decode_raw(lib, **kw):
    a = dict(q=0x1000, k=0x2000, v=0x3000, bt=0x4000, cl=0x5000, scale=0.1, out=0x6000, B=4, Hq=8, Hkv=2, D=128,
             bs=16, MB=4, NB=32, qs=8 * 128, dtype=pa.DTYPE_BF16, odt=pa.DTYPE_F32)
    a.update(kw)
    return lib.pa_paged_attention_decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["scale"], a["out"], a["B"],
                                         a["Hq"], a["Hkv"], a["D"], a["bs"], a["MB"], a["NB"], a["qs"], a["dtype"],
                                         a["odt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(bt=None), 1),
    (dict(odt=pa.DTYPE_F16), 2),
    (dict(dtype=pa.DTYPE_F32, odt=pa.DTYPE_BF16), 2),
    (dict(qs=100), 3),
    (dict(NB=0), 3),
    (dict(q=0x1008), 4),
    (dict(qs=8 * 128 + 4), 4),
])
def test_decode_validation_before_any_device_work(lib, kw, code):
    assert _decode_raw(lib, **kw) == code
    assert lib.pa_last_error()


def test_decode_empty_batch_is_a_noop(lib):
    assert _decode_raw(lib, B=0, q=None, out=None) == 0


def _store_raw(lib, **kw):
    a = dict(k=0x1000, v=0x2000, sm=0x3000, kc=0x4000, vc=0x5000, N=4, Hkv=2, D=128, bs=16, NB=8, ks=256, vs=256,
             dtype=pa.DTYPE_BF16)
    a.update(kw)
    return lib.pa_store_kvcache(a["k"], a["v"], a["sm"], a["kc"], a["vc"], a["N"], a["Hkv"], a["D"], a["bs"],
                                a["NB"], a["ks"], a["vs"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 2),
    (dict(N=-1), 3),
    (dict(Hkv=0), 3),
    (dict(D=100), 4),
    (dict(bs=6), 4),
    (dict(sm=None), 1),
    (dict(ks=100), 3),
    (dict(kc=0x4004), 4),
    (dict(ks=260), 4),
])
def test_store_validation(lib, kw, code):
    assert _store_raw(lib, **kw) == code


def test_store_zero_tokens_is_a_noop(lib):
    assert _store_raw(lib, N=0, k=None, v=None) == 0


def test_workspace_bytes_is_zero_on_bad_sizes(lib):
    assert lib.pa_decode_workspace_bytes(4, 8, 3, 128, 16, 4, 2, 0) == 0


def test_binding_shapes():
    import torch
    assert pa.k_cache_shape(10, 8, 128, 16, torch.bfloat16) == (10, 8, 16, 16, 8)
    assert pa.k_cache_shape(10, 8, 64, 16, torch.float32) == (10, 8, 16, 16, 4)
    assert pa.v_cache_shape(10, 8, 128, 16) == (10, 8, 4, 128, 4)


def test_binding_rejects_cpu_tensors():
    import torch
    k, v = torch.zeros(pa.k_cache_shape(2, 1, 64, 16, torch.float16), dtype=torch.float16), \
        torch.zeros(pa.v_cache_shape(2, 1, 64, 16), dtype=torch.float16)
    with pytest.raises(ValueError):
        pa.paged_attention_decode(torch.zeros(1, 1, 64, dtype=torch.float16), k, v,
                                  torch.zeros(1, 2, dtype=torch.int32), torch.ones(1, dtype=torch.int32), 0.1)


def test_plan_shared_prefix_window_and_workspace():
    # G = 2: windows of 8 sequences; partial rows get 16 columns, plus prefix records and words
    base = _plan(partition_size=-2)
    sp = _plan(partition_size=-2, shared_prefix=True)
    assert base["shared_prefix_window"] == 0 and sp["shared_prefix_window"] == 8
    rows = sp["num_waves"] * 2 * 16
    assert sp["workspace_bytes"] >= rows * 128 * 4 + rows * 4 + 256 * 8 * 16 + 32 * 8 * 16 + 256 * 4
    assert sp["workspace_bytes"] > base["workspace_bytes"]
    assert sp["num_waves"] == base["num_waves"] and sp["range_tokens"] == base["range_tokens"]
    # windows of 16 // G sequences for every G up to 8
    for g, w in ((1, 16), (3, 5), (4, 4), (5, 3), (8, 2)):
        assert _plan(num_heads=2 * g, num_kv_heads=2, partition_size=512, shared_prefix=True)[
            "shared_prefix_window"] == w


@pytest.mark.parametrize("kw", [dict(partition_size=-1), dict(partition_size=-3), dict(num_heads=32, num_kv_heads=2),
                                dict(num_heads=40, num_kv_heads=2), dict(num_seqs=8192),
                                dict(max_blocks_per_seq=16)])  # automatic mode picks one pass at 256 tokens
def test_plan_shared_prefix_does_not_apply(kw):
    args = dict(shared_prefix=True)
    args.update(kw)
    p = _plan(**args)
    assert p["shared_prefix_window"] == 0
    args["shared_prefix"] = False
    assert p["workspace_bytes"] == _plan(**args)["workspace_bytes"]
