"""Host-side argument checks of the Python binding (no GPU).

The library is replaced by a recorder and the device check by a no-op, so that host tensors
stand in for device tensors. Every malformed call must raise before it reaches the library;
the well-formed calls must reach it once, with the sizes and strides read from the tensors.
The device check itself is tested on stand-in objects.
"""

from __future__ import annotations

import pytest

import paged_attention_decode_amd as pa

torch = pytest.importorskip("torch")

NB, HKV, D, BS, B, HQ, MB = 6, 2, 64, 16, 3, 4, 2


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def call(*args):
            self.calls.append((name, args))
            return 0
        return call


@pytest.fixture
def lib(monkeypatch):
    rec = _Recorder()
    monkeypatch.setattr(pa, "_lib", rec)
    monkeypatch.setattr(pa, "_require_cuda", lambda *ts: None)
    monkeypatch.setattr(pa, "_stream_of", lambda t: 0)
    return rec


def _caches(dt=torch.bfloat16):
    return (torch.zeros(pa.k_cache_shape(NB, HKV, D, BS, dt), dtype=dt),
            torch.zeros(pa.v_cache_shape(NB, HKV, D, BS), dtype=dt))


def _decode_args(dt=torch.bfloat16):
    k_cache, v_cache = _caches(dt)
    return dict(q=torch.zeros(B, HQ, D, dtype=dt), k_cache=k_cache, v_cache=v_cache,
                block_tables=torch.zeros(B, MB, dtype=torch.int32), context_lens=torch.ones(B, dtype=torch.int32))


def _store_args(dt=torch.bfloat16, n=5):
    k_cache, v_cache = _caches(dt)
    return dict(k=torch.zeros(n, HKV, D, dtype=dt), v=torch.zeros(n, HKV, D, dtype=dt),
                slot_mapping=torch.arange(n, dtype=torch.int32), k_cache=k_cache, v_cache=v_cache)


def test_well_formed_store_reaches_the_library(lib):
    pa.store_kvcache(**_store_args())
    assert [c[0] for c in lib.calls] == ["pa_store_kvcache"]
    args = lib.calls[0][1]
    assert args[5:12] == (5, HKV, D, BS, NB, HKV * D, HKV * D)


def test_store_token_stride_is_passed_through(lib):
    a = _store_args()
    wide = torch.zeros(5, 3 * HKV * D, dtype=torch.bfloat16)
    a["k"] = wide[:, :HKV * D].view(5, HKV, D)            # token stride 3*Hkv*D, rows contiguous
    a["v"] = wide[:, HKV * D:2 * HKV * D].view(5, HKV, D)
    pa.store_kvcache(**a)
    args = lib.calls[0][1]
    assert args[10] == 3 * HKV * D and args[11] == 3 * HKV * D


@pytest.mark.parametrize("case", [
    "k_rank", "k_heads", "k_dim", "v_shape", "slot_len", "slot_dtype", "slot_strided", "k_dtype", "v_dtype",
    "k_rows_strided", "v_rows_strided", "v_cache_shape", "cache_dtype", "cache_strided", "k_cache_x",
])
def test_malformed_store_is_rejected_before_the_library(lib, case):
    a = _store_args()
    if case == "k_rank":
        a["k"] = a["k"].reshape(5, HKV * D)
    elif case == "k_heads":
        a["k"] = torch.zeros(5, HKV + 1, D, dtype=torch.bfloat16)
    elif case == "k_dim":
        a["k"] = torch.zeros(5, HKV, D // 2, dtype=torch.bfloat16)
    elif case == "v_shape":
        a["v"] = torch.zeros(4, HKV, D, dtype=torch.bfloat16)
    elif case == "slot_len":
        a["slot_mapping"] = torch.arange(4, dtype=torch.int32)
    elif case == "slot_dtype":
        a["slot_mapping"] = torch.arange(5, dtype=torch.int64)
    elif case == "slot_strided":
        a["slot_mapping"] = torch.arange(10, dtype=torch.int32)[::2]
    elif case == "k_dtype":
        a["k"] = a["k"].half()
    elif case == "v_dtype":
        a["v"] = a["v"].float()
    elif case == "k_rows_strided":
        a["k"] = torch.zeros(5, HKV, 2 * D, dtype=torch.bfloat16)[:, :, ::2]
    elif case == "v_rows_strided":
        a["v"] = torch.zeros(5, 2 * HKV, D, dtype=torch.bfloat16)[:, ::2, :]
    elif case == "v_cache_shape":
        a["v_cache"] = torch.zeros(NB, HKV, BS // 4, D, 2, dtype=torch.bfloat16)
    elif case == "cache_dtype":
        a["v_cache"] = a["v_cache"].half()
    elif case == "cache_strided":
        big = torch.zeros((2 * NB,) + tuple(a["k_cache"].shape[1:]), dtype=torch.bfloat16)
        a["k_cache"] = big[::2]
    elif case == "k_cache_x":
        a["k_cache"] = torch.zeros(NB, HKV, D // 4, BS, 4, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        pa.store_kvcache(**a)
    assert lib.calls == []


def test_well_formed_decode_reaches_the_library(lib):
    a = _decode_args()
    out = pa.paged_attention_decode(**a, scale=0.125, out_dtype=torch.float32)
    assert out.shape == (B, HQ, D) and out.dtype == torch.float32
    assert [c[0] for c in lib.calls] == ["pa_paged_attention_decode_ex"]
    args = lib.calls[0][1]
    assert args[7:17] == (B, HQ, HKV, D, BS, MB, NB, HQ * D, pa.DTYPE_BF16, pa.DTYPE_F32)


@pytest.mark.parametrize("case", [
    "q_rank", "q_dim", "q_rows_strided", "q_dtype", "bt_dtype", "cl_dtype", "bt_rows", "bt_rank", "bt_strided",
    "cl_len", "cl_strided", "out_shape", "out_strided",
])
def test_malformed_decode_is_rejected_before_the_library(lib, case):
    a = _decode_args()
    out = None
    if case == "q_rank":
        a["q"] = a["q"].reshape(B, HQ * D)
    elif case == "q_dim":
        a["q"] = torch.zeros(B, HQ, D + 8, dtype=torch.bfloat16)
    elif case == "q_rows_strided":
        a["q"] = torch.zeros(B, HQ, 2 * D, dtype=torch.bfloat16)[:, :, ::2]
    elif case == "q_dtype":
        a["q"] = a["q"].half()
    elif case == "bt_dtype":
        a["block_tables"] = a["block_tables"].long()
    elif case == "cl_dtype":
        a["context_lens"] = a["context_lens"].long()
    elif case == "bt_rows":
        a["block_tables"] = torch.zeros(B + 1, MB, dtype=torch.int32)
    elif case == "bt_rank":
        a["block_tables"] = torch.zeros(B * MB, dtype=torch.int32)
    elif case == "bt_strided":
        a["block_tables"] = torch.zeros(B, 2 * MB, dtype=torch.int32)[:, ::2]
    elif case == "cl_len":
        a["context_lens"] = torch.ones(B + 1, dtype=torch.int32)
    elif case == "cl_strided":
        a["context_lens"] = torch.ones(2 * B, dtype=torch.int32)[::2]
    elif case == "out_shape":
        out = torch.zeros(B, HQ, D // 2)
    elif case == "out_strided":
        out = torch.zeros(B, HQ, 2 * D)[:, :, ::2]
    with pytest.raises((ValueError, TypeError)):
        pa.paged_attention_decode(**a, scale=0.125, out=out)
    assert lib.calls == []


@pytest.mark.parametrize("case", ["k_new_shape", "v_new_shape", "k_new_rows_strided", "k_new_dtype", "q_dim"])
def test_malformed_decode_step_is_rejected_before_the_library(lib, case):
    a = _decode_args()
    k_new, v_new = torch.zeros(B, HKV, D, dtype=torch.bfloat16), torch.zeros(B, HKV, D, dtype=torch.bfloat16)
    if case == "k_new_shape":
        k_new = torch.zeros(B + 1, HKV, D, dtype=torch.bfloat16)
    elif case == "v_new_shape":
        v_new = torch.zeros(B, HKV, D + 16, dtype=torch.bfloat16)
    elif case == "k_new_rows_strided":
        k_new = torch.zeros(B, HKV, 2 * D, dtype=torch.bfloat16)[:, :, ::2]
    elif case == "k_new_dtype":
        k_new = k_new.half()
    elif case == "q_dim":
        a["q"] = torch.zeros(B, HQ, D // 2, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        pa.decode_step(a["q"], k_new, v_new, a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 0.1)
    assert lib.calls == []


def test_well_formed_decode_step_reaches_the_library(lib):
    a = _decode_args()
    wide = torch.zeros(B, 2 * HKV * D, dtype=torch.bfloat16)
    k_new = wide[:, :HKV * D].view(B, HKV, D)
    v_new = torch.zeros(B, HKV, D, dtype=torch.bfloat16)
    pa.decode_step(a["q"], k_new, v_new, a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 0.1)
    assert [c[0] for c in lib.calls] == ["pa_decode_step"]
    args = lib.calls[0][1]
    assert args[3:5] == (2 * HKV * D, HKV * D)


class _Dev:
    def __init__(self, d):
        self.d = d

    def get_device(self):
        return self.d


@pytest.mark.parametrize("devs, ok", [((0, 0, 0), True), ((1,), True), ((0, 0, 1), False), ((-1,), False),
                                      ((0, -1), False), ((-1, -1), False)])
def test_device_check(devs, ok):
    ts = [_Dev(d) for d in devs]
    if ok:
        pa._require_cuda(*ts)
    else:
        with pytest.raises(ValueError):
            pa._require_cuda(*ts)


@pytest.mark.parametrize("shared", [False, True])
def test_options_reach_the_library(lib, shared):
    """partition_size, cached_prefix_tokens and shared_prefix land in pa_decode_opts for both
    decode entry points."""
    a = _decode_args()
    pa.paged_attention_decode(**a, scale=0.1, partition_size=48, cached_prefix_tokens=-1, shared_prefix=shared)
    k_new, v_new = torch.zeros(B, HKV, D, dtype=torch.bfloat16), torch.zeros(B, HKV, D, dtype=torch.bfloat16)
    pa.decode_step(a["q"], k_new, v_new, a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 0.1,
                   partition_size=-2, shared_prefix=shared)
    assert [c[0] for c in lib.calls] == ["pa_paged_attention_decode_ex", "pa_decode_step"]
    o1 = lib.calls[0][1][17]._obj
    o2 = lib.calls[1][1][21]._obj
    assert (o1.partition_size, o1.cached_prefix_tokens, o1.shared_prefix) == (48, -1, int(shared))
    assert (o2.partition_size, o2.shared_prefix) == (-2, int(shared))
    assert not o1.workspace and not o1.event_begin
