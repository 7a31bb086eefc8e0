"""Pins for the CPU oracle: each check rests on something other than the oracle itself."""

from __future__ import annotations

import json
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import oracle.paged_attention as opa
from oracle import CacheGeometry
from _paged_helpers import (PagedCase, logical_to_physical_k, logical_to_physical_v,
                            physical_to_logical_k, physical_to_logical_v, sdpa_reference, widen_np)

GOLDEN = Path(__file__).parent / "golden"


def _scale32(s):
    return float(np.float32(s))


# ---------------------------------------------------------------- layout / gather

@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("bs", [4, 8, 16])
def test_gather_matches_transpose_construction(dtype, bs):
    rng = np.random.default_rng(11)
    case = PagedCase(rng, batch=3, hq=4, hkv=2, d=16, bs=bs, lens=[1, bs + 3, 3 * bs], dtype=dtype)
    geo = case.geometry()
    for s in range(3):
        k, v = oracle.gather_kv(case.k_cache, case.v_cache, case.tables[s], int(case.lens[s]), geo)
        np.testing.assert_array_equal(k, widen_np(case.k_dense[s], dtype))
        np.testing.assert_array_equal(v, widen_np(case.v_dense[s], dtype))


def test_layout_golden_positions():
    fx = json.loads((GOLDEN / "layout_slot5_fp16.json").read_text())
    geo = CacheGeometry(fx["num_blocks"], fx["num_kv_heads"], fx["head_dim"], fx["block_size"], fx["dtype"])
    n = geo.num_blocks * geo.num_kv_heads * geo.block_size * geo.head_dim
    k = np.zeros(n, np.float16)
    v = np.zeros(n, np.float16)
    row = np.arange(1, geo.head_dim + 1, dtype=np.float16).reshape(1, 1, geo.head_dim)
    k2, v2 = oracle.store_kvcache(row, -row, np.array([fx["slot"]]), k, v, geo)
    assert sorted(np.flatnonzero(k2).tolist()) == fx["k_flat_positions"]
    assert sorted(np.flatnonzero(v2).tolist()) == fx["v_flat_positions"]
    np.testing.assert_array_equal(k2[fx["k_flat_positions"]], row.ravel())
    np.testing.assert_array_equal(v2[fx["v_flat_positions"]], -row.ravel())


# ---------------------------------------------------------------- widening of storage types

def _ieee_half_value(bits: int, exp_bits: int, man_bits: int) -> float:
    """Value of a 16-bit IEEE-style pattern from the format's definition (sign, biased exponent,
    fraction; exponent 0 = subnormal, all ones = inf/NaN), independent of any conversion routine."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> man_bits) & ((1 << exp_bits) - 1)
    f = bits & ((1 << man_bits) - 1)
    bias = (1 << (exp_bits - 1)) - 1
    if e == (1 << exp_bits) - 1:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, 1 - bias - man_bits)
    return sign * math.ldexp((1 << man_bits) + f, e - bias - man_bits)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_widen_matches_torch_and_format_definition_on_every_bit_pattern(dtype):
    """oracle.widen of all 65536 16-bit patterns equals torch's own conversion to float64 and the
    value the format defines (bf16: 8 exponent / 7 fraction bits, fp16: 5 / 10), NaN as NaN."""
    import torch
    bits = np.arange(1 << 16, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        got = oracle.widen(bits if dtype == "bf16" else bits.view(np.float16), dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    ref_torch = torch.from_numpy(bits.view(np.int16)).view(tdt).to(torch.float64).numpy()
    eb, mb = (8, 7) if dtype == "bf16" else (5, 10)
    ref_def = np.array([_ieee_half_value(int(b), eb, mb) for b in bits])
    for ref in (ref_torch, ref_def):
        nan = np.isnan(ref)
        np.testing.assert_array_equal(np.isnan(got), nan)
        np.testing.assert_array_equal(got[~nan], ref[~nan])
        # signed zeros keep their sign
        np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert got.dtype == np.float64


def test_widen_fp32_is_exact():
    rng = np.random.default_rng(3)
    a = rng.standard_normal(1000).astype(np.float32)
    a[:4] = [0.0, -0.0, np.float32(2.0 ** -149), np.float32(3.4e38)]
    np.testing.assert_array_equal(oracle.widen(a, "fp32"), np.array([float(v) for v in a.tolist()]))


# ---------------------------------------------------------------- brute force vs library routine

@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**31 - 1), batch=st.integers(1, 4), g=st.sampled_from([1, 2, 4]),
       hkv=st.sampled_from([1, 2]), d=st.sampled_from([8, 16, 64]), bs=st.sampled_from([4, 8, 16]),
       dtype=st.sampled_from(["fp32", "fp16", "bf16"]), data=st.data())
def test_decode_matches_sdpa(seed, batch, g, hkv, d, bs, dtype, data):
    lens = data.draw(st.lists(st.integers(0, 70), min_size=batch, max_size=batch))
    rng = np.random.default_rng(seed)
    case = PagedCase(rng, batch, g * hkv, hkv, d, bs, lens, dtype=dtype)
    scale = data.draw(st.sampled_from([1.0 / math.sqrt(d), 0.3, 1.7]))
    out = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, scale, case.geometry())
    for s in range(batch):
        ref = sdpa_reference(widen_np(case.q[s], dtype), widen_np(case.k_dense[s], dtype),
                             widen_np(case.v_dense[s], dtype), _scale32(scale))
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_golden_rational_softmax():
    fx = json.loads((GOLDEN / "rational_softmax_gqa.json").read_text())
    hq, hkv, d, bs = fx["num_heads"], fx["num_kv_heads"], fx["head_dim"], fx["block_size"]
    geo = CacheGeometry(fx["num_blocks"], hkv, d, bs, fx["dtype"])
    k_log = np.zeros((geo.num_blocks, hkv, bs, d), np.float32)
    v_log = np.full((geo.num_blocks, hkv, bs, d), np.nan, np.float32)  # unused slots poisoned
    for s, L in enumerate(fx["context_lens"]):
        for t in range(L):
            blk, off = fx["block_tables"][s][t // bs], t % bs
            for g in range(hkv):
                a_even, a_odd = fx["a"][s][t][g]
                k_log[blk, g, off, :2] = [2 * math.log(a_even), 2 * math.log(a_odd)]
                v_log[blk, g, off] = fx["v"][s][t][g]
    q = np.zeros((2, hq, d), np.float32)
    for h in range(hq):
        q[:, h, h % 2] = 1.0
    out = oracle.decode(q, logical_to_physical_k(k_log, "fp32"), logical_to_physical_v(v_log),
                        np.array(fx["block_tables"], np.int32), np.array(fx["context_lens"], np.int32),
                        fx["scale"], geo)
    expected = np.array([[[float(Fraction(x)) for x in row] for row in seq] for seq in fx["expected"]])
    np.testing.assert_allclose(out, expected, rtol=1e-6, atol=1e-6)
    # the stored fractions are the integer-weighted means of the value rows
    for s in range(2):
        for h in range(hq):
            ws = [Fraction(tok[h // 2][h % 2]) for tok in fx["a"][s]]
            vs = [tok[h // 2] for tok in fx["v"][s]]
            mean = [sum(w * Fraction(v[j]) for w, v in zip(ws, vs)) / sum(ws) for j in range(d)]
            assert [str(m) for m in mean] == fx["expected"][s][h]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_length_one_returns_value_row_exactly(dtype):
    rng = np.random.default_rng(3)
    case = PagedCase(rng, 3, 8, 2, 64, 16, [1, 1, 1], dtype=dtype)
    out = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 0.125, case.geometry())
    for s in range(3):
        for h in range(8):
            np.testing.assert_array_equal(out[s, h], widen_np(case.v_dense[s][0, h // 4], dtype))


def test_identical_keys_and_zero_query_give_mean_of_values():
    rng = np.random.default_rng(4)
    L, hkv, d = 37, 2, 16
    krow = rng.standard_normal((1, hkv, d)).astype(np.float32)
    kd = [np.repeat(krow, L, axis=0)]
    vd = [rng.standard_normal((L, hkv, d)).astype(np.float32)]
    case = PagedCase(rng, 1, 4, hkv, d, 8, [L], k_dense=kd, v_dense=vd)
    mean = vd[0].astype(np.float64).mean(axis=0)
    out = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 0.7, case.geometry())
    for h in range(4):
        np.testing.assert_allclose(out[0, h], mean[h // 2], atol=1e-14)
    # random keys but a zero query, or a zero scale: uniform weights
    case2 = PagedCase(rng, 1, 4, hkv, d, 8, [L])
    for q, scale in ((np.zeros_like(case2.q), 0.7), (case2.q, 0.0)):
        out2 = oracle.decode(q, case2.k_cache, case2.v_cache, case2.tables, case2.lens, scale, case2.geometry())
        mean2 = case2.v_dense[0].astype(np.float64).mean(axis=0)
        for h in range(4):
            np.testing.assert_allclose(out2[0, h], mean2[h // 2], atol=1e-14)


def test_dominant_logit_selects_its_value_row():
    rng = np.random.default_rng(5)
    L, d = 20, 8
    kd = np.zeros((L, 1, d), np.float32)
    kd[13, 0, 0] = 60.0
    vd = rng.standard_normal((L, 1, d)).astype(np.float32)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    case = PagedCase(rng, 1, 1, 1, d, 4, [L], k_dense=[kd], v_dense=[vd], q=q)
    out = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 1.0, case.geometry())
    # the other 19 weights are about exp(-60) each: far below one ulp of the result
    np.testing.assert_allclose(out[0, 0], vd[13, 0], rtol=0, atol=1e-15)


def test_gqa_head_mapping_with_constant_values():
    # Every token of kv head g carries the value row c_g: query head h must return c_(h // G).
    rng = np.random.default_rng(6)
    hkv, g, d, L = 4, 2, 8, 29
    consts = np.arange(hkv * d, dtype=np.float32).reshape(hkv, d) + 1.0
    vd = np.repeat(consts[None], L, axis=0)
    kd = rng.standard_normal((L, hkv, d)).astype(np.float32)
    case = PagedCase(rng, 1, hkv * g, hkv, d, 8, [L], k_dense=[kd], v_dense=[vd])
    out = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 0.5, case.geometry())
    for h in range(hkv * g):
        np.testing.assert_allclose(out[0, h], consts[h // g], rtol=1e-14)


# ---------------------------------------------------------------- invariants

def test_weights_sum_to_one_and_are_nonnegative():
    rng = np.random.default_rng(7)
    case = PagedCase(rng, 4, 8, 2, 32, 8, [1, 9, 40, 64], dtype="bf16")
    _, w = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 0.2,
                         case.geometry(), return_weights=True)
    for s in range(4):
        assert (w[s] >= 0).all()
        np.testing.assert_allclose(w[s].sum(axis=1), 1.0, atol=1e-14)


def test_relabelling_physical_blocks_is_bit_identical():
    rng = np.random.default_rng(8)
    case = PagedCase(rng, 3, 4, 2, 16, 8, [5, 17, 30], dtype="fp16")
    geo = case.geometry()
    out = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 0.25, geo)
    pi = rng.permutation(case.nb)
    k2 = np.empty_like(case.k_cache)
    v2 = np.empty_like(case.v_cache)
    k2[pi] = case.k_cache
    v2[pi] = case.v_cache
    out2 = oracle.decode(case.q, k2, v2, pi[case.tables].astype(np.int32), case.lens, 0.25, geo)
    np.testing.assert_array_equal(out, out2)


def test_key_shift_and_affine_value_invariance():
    rng = np.random.default_rng(9)
    L, hkv, d = 25, 1, 16
    kd = rng.standard_normal((L, hkv, d))
    vd = rng.standard_normal((L, hkv, d))
    shift = rng.standard_normal((1, hkv, d))
    base = PagedCase(rng, 1, 2, hkv, d, 8, [L], k_dense=[kd.astype(np.float32)], v_dense=[vd.astype(np.float32)])
    q = base.q
    out = oracle.decode(q, base.k_cache, base.v_cache, base.tables, base.lens, 0.4, base.geometry())
    shifted = PagedCase(np.random.default_rng(1), 1, 2, hkv, d, 8, [L], k_dense=[(kd + shift).astype(np.float32)],
                        v_dense=[vd.astype(np.float32)], q=q)
    # the float32 rounding of k + shift perturbs logits by ~1e-7; compare to the exact shifted keys
    k_exact = shifted.k_dense[0].astype(np.float64) - shift
    ref = sdpa_reference(q[0].astype(np.float64), k_exact, vd.astype(np.float32).astype(np.float64), 0.4)
    out_shift = oracle.decode(q, shifted.k_cache, shifted.v_cache, shifted.tables, shifted.lens, 0.4, shifted.geometry())
    np.testing.assert_allclose(out_shift[0], ref, atol=1e-12)
    alpha, beta = 2.0, -0.75  # exact in float32
    affine = PagedCase(np.random.default_rng(2), 1, 2, hkv, d, 8, [L], k_dense=[kd.astype(np.float32)],
                       v_dense=[(alpha * vd.astype(np.float32) + beta).astype(np.float32)], q=q)
    out_aff = oracle.decode(q, affine.k_cache, affine.v_cache, affine.tables, affine.lens, 0.4, affine.geometry())
    np.testing.assert_allclose(out_aff, alpha * out + beta, atol=1e-13)


def test_equal_queries_in_a_group_give_equal_outputs():
    rng = np.random.default_rng(10)
    case = PagedCase(rng, 2, 8, 2, 16, 8, [12, 33])
    q = case.q.copy()
    q[:, 1] = q[:, 0]
    q[:, 3] = q[:, 0]
    out = oracle.decode(q, case.k_cache, case.v_cache, case.tables, case.lens, 0.3, case.geometry())
    np.testing.assert_array_equal(out[:, 1], out[:, 0])
    np.testing.assert_array_equal(out[:, 3], out[:, 0])
    assert not np.array_equal(out[:, 4], out[:, 0])  # other kv head differs


def test_zero_length_gives_zeros():
    rng = np.random.default_rng(12)
    case = PagedCase(rng, 2, 2, 1, 8, 4, [0, 3])
    out = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 1.0, case.geometry())
    assert (out[0] == 0).all() and np.isfinite(out[1]).all()


# ---------------------------------------------------------------- split / merge

@pytest.mark.parametrize("psize", [1, 4, 7, 16, 64, 1000])
def test_split_merge_equals_dense(psize):
    rng = np.random.default_rng(13)
    case = PagedCase(rng, 3, 4, 2, 16, 4, [1, 30, 61], dtype="bf16")
    geo = case.geometry()
    dense = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 0.35, geo)
    merged, lse, parts = oracle.decode_split(case.q, case.k_cache, case.v_cache, case.tables, case.lens,
                                             0.35, geo, psize)
    np.testing.assert_allclose(merged, dense, atol=1e-13)
    # lse of the whole context equals log-sum-exp of the partition lse values
    z0 = 0.35
    k, _ = oracle.gather_kv(case.k_cache, case.v_cache, case.tables[2], 61, geo)
    zfull = np.float64(np.float32(z0)) * (k[:, 0, :] @ oracle.widen(case.q[2, 0], "bf16"))
    total = np.log(np.exp(zfull - zfull.max()).sum()) + zfull.max()
    part = lse[2][0]
    np.testing.assert_allclose(np.log(np.exp(part - part.max()).sum()) + part.max(), total, atol=1e-12)


def test_merge_ignores_empty_partitions():
    parts = np.array([[1.0, 2.0], [9.0, 9.0], [3.0, 4.0]])
    lse = np.array([0.0, -np.inf, math.log(3.0)])
    np.testing.assert_allclose(oracle.merge_partitions(lse, parts), [(1 + 9) / 4, (2 + 12) / 4])
    assert (oracle.merge_partitions(np.array([-np.inf]), parts[:1]) == 0).all()


# ---------------------------------------------------------------- store

@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_store_matches_logical_assignment_and_leaves_other_bytes(dtype):
    rng = np.random.default_rng(14)
    nb, hkv, bs, d, n = 6, 2, 8, 16, 5
    geo = CacheGeometry(nb, hkv, d, bs, dtype)
    case = PagedCase(rng, 1, 2, hkv, d, bs, [nb * bs - 3 * bs], dtype=dtype, extra_blocks=3)
    k_log, v_log = case.k_log.copy(), case.v_log.copy()
    slots = rng.choice(nb * bs, size=n, replace=False).astype(np.int32)
    slots[2] = -1
    from workloads import to_storage
    kn = to_storage(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype)
    vn = to_storage(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype)
    k2, v2 = oracle.store_kvcache(kn, vn, slots, case.k_cache, case.v_cache, geo)
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        k_log[sl // bs, :, sl % bs, :] = kn[i]
        v_log[sl // bs, :, sl % bs, :] = vn[i]
    assert k2.tobytes() == logical_to_physical_k(k_log, dtype).tobytes()
    assert v2.tobytes() == logical_to_physical_v(v_log).tobytes()
    back_k = physical_to_logical_k(k2, nb, hkv, bs, d, dtype)
    back_v = physical_to_logical_v(v2, nb, hkv, bs, d)
    for i, sl in enumerate(slots):
        if sl >= 0:
            assert back_k[sl // bs, :, sl % bs].tobytes() == kn[i].tobytes()
            assert back_v[sl // bs, :, sl % bs].tobytes() == vn[i].tobytes()


def test_store_copies_nan_payload_bits():
    geo = CacheGeometry(2, 1, 8, 4, "bf16")
    k = np.zeros(64, np.uint16)
    row = np.full((1, 1, 8), 0x7FC1, np.uint16)
    k2, v2 = oracle.store_kvcache(row, row, np.array([6]), k, k.copy(), geo)
    assert (k2 == 0x7FC1).sum() == 8 and (v2 == 0x7FC1).sum() == 8


def test_store_then_decode_sees_new_token():
    rng = np.random.default_rng(15)
    case = PagedCase(rng, 2, 4, 2, 16, 8, [9, 20], dtype="bf16")
    geo = case.geometry()
    from workloads import to_storage
    kn = to_storage(rng.standard_normal((2, 2, 16), dtype=np.float32), "bf16")
    vn = to_storage(rng.standard_normal((2, 2, 16), dtype=np.float32), "bf16")
    pos = case.lens - 1
    slots = (case.tables[[0, 1], pos // 8].astype(np.int64) * 8 + pos % 8).astype(np.int32)
    k2, v2 = oracle.store_kvcache(kn, vn, slots, case.k_cache, case.v_cache, geo)
    for s in range(2):
        k, v = oracle.gather_kv(k2, v2, case.tables[s], int(case.lens[s]), geo)
        np.testing.assert_array_equal(k[-1], oracle.widen(kn[s], "bf16"))
        np.testing.assert_array_equal(v[-1], oracle.widen(vn[s], "bf16"))
        np.testing.assert_array_equal(k[:-1], widen_np(case.k_dense[s][:-1], "bf16"))


# ---------------------------------------------------------------- planted mistakes are caught

def _wrong_head_map(q_rows, k, v, scale, return_weights=False):
    hq = q_rows.shape[0]
    hkv = k.shape[1]
    out = np.zeros((hq, q_rows.shape[1]))
    sigma = float(np.float32(scale))
    for h in range(hq):
        g = h % hkv  # plausible mistake: interleaved instead of grouped heads
        z = sigma * (k[:, g, :] @ q_rows[h])
        w = np.exp(z - z.max())
        out[h] = (w / w.sum()) @ v[:, g, :]
    return out


def _dropped_scale(q_rows, k, v, scale, return_weights=False):
    return opa.__dict__["_orig_decode_sequence"](q_rows, k, v, 1.0, return_weights)


def _transposed_gather(k_cache, v_cache, block_row, length, geo):
    k, v = opa.__dict__["_orig_gather_kv"](k_cache, v_cache, block_row, length, geo)
    return v, k


@pytest.mark.parametrize("mutant", ["head_map", "scale", "swap_kv"])
def test_pins_catch_planted_mistakes(monkeypatch, mutant):
    monkeypatch.setitem(opa.__dict__, "_orig_decode_sequence", opa.decode_sequence)
    monkeypatch.setitem(opa.__dict__, "_orig_gather_kv", opa.gather_kv)
    if mutant == "head_map":
        monkeypatch.setattr(opa, "decode_sequence", _wrong_head_map)
    elif mutant == "scale":
        monkeypatch.setattr(opa, "decode_sequence", _dropped_scale)
    else:
        monkeypatch.setattr(opa, "gather_kv", _transposed_gather)
    failed = 0
    for pin in (test_golden_rational_softmax, test_gqa_head_mapping_with_constant_values):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught the planted {mutant} mistake"


# ---------------------------------------------------------------- causal prefill

def _sdpa_causal(q64, k64, v64, scale, offset):
    """SDPA (float64) with query i allowed keys 0 .. offset + i."""
    import torch
    n, hq, d = q64.shape
    L, hkv, _ = k64.shape
    g = hq // hkv
    qt = torch.from_numpy(q64).permute(1, 0, 2).reshape(1, hq, n, d)
    kt = torch.from_numpy(k64).permute(1, 0, 2).repeat_interleave(g, dim=0).reshape(1, hq, L, d).contiguous()
    vt = torch.from_numpy(v64).permute(1, 0, 2).repeat_interleave(g, dim=0).reshape(1, hq, L, d).contiguous()
    allowed = torch.arange(L)[None, :] <= (offset + torch.arange(n))[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=scale)
    return out.reshape(hq, n, d).permute(1, 0, 2).numpy()


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**31 - 1), g=st.sampled_from([1, 2, 4]), hkv=st.sampled_from([1, 2]),
       dtype=st.sampled_from(["fp32", "bf16", "fp16"]), data=st.data())
def test_prefill_matches_sdpa_with_causal_offset_mask(seed, g, hkv, dtype, data):
    lens = data.draw(st.lists(st.integers(1, 40), min_size=1, max_size=3))
    news = [data.draw(st.integers(1, L)) for L in lens]
    _prefill_vs_sdpa(seed, g, hkv, dtype, lens, news)


def _prefill_vs_sdpa(seed, g, hkv, dtype, lens, news):
    rng = np.random.default_rng(seed)
    d = 16
    case = PagedCase(rng, len(lens), g * hkv, hkv, d, 8, lens, dtype=dtype)
    from workloads import to_storage
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = to_storage(rng.standard_normal((int(qs[-1]), g * hkv, d), dtype=np.float32), dtype)
    out = oracle.prefill(q, case.k_cache, case.v_cache, case.tables, case.lens, qs, 0.3, case.geometry())
    for s, (L, n) in enumerate(zip(lens, news)):
        ref = _sdpa_causal(widen_np(q[qs[s]:qs[s + 1]], dtype), widen_np(case.k_dense[s], dtype),
                           widen_np(case.v_dense[s], dtype), _scale32(0.3), L - n)
        np.testing.assert_allclose(out[qs[s]:qs[s + 1]], ref, atol=1e-12)


def test_prefill_of_one_new_token_is_decode():
    rng = np.random.default_rng(21)
    case = PagedCase(rng, 3, 8, 2, 32, 8, [9, 1, 30], dtype="bf16")
    qs = np.arange(4, dtype=np.int32)
    out = oracle.prefill(case.q, case.k_cache, case.v_cache, case.tables, case.lens, qs, 0.2, case.geometry())
    dec = oracle.decode(case.q, case.k_cache, case.v_cache, case.tables, case.lens, 0.2, case.geometry())
    np.testing.assert_array_equal(out, dec)


def test_prefill_first_token_returns_its_value_row():
    # query 0 of a full prefill (n == L) sees only token 0
    rng = np.random.default_rng(22)
    case = PagedCase(rng, 1, 4, 2, 16, 4, [12], dtype="fp32")
    from workloads import to_storage
    q = to_storage(rng.standard_normal((12, 4, 16), dtype=np.float32), "fp32")
    out = oracle.prefill(q, case.k_cache, case.v_cache, case.tables, case.lens, np.array([0, 12], np.int32), 0.5,
                         case.geometry())
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], widen_np(case.v_dense[0][0, h // 2], "fp32"))


# ---------------------------------------------------------------- planted mistakes: prefill and merge

def _prefill_seeing(position):
    """The oracle's prefill with another rule for the last key query i may see (a planted mistake)."""
    def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, geo, seqs=None):
        t_total, hq, dim = q.shape
        qf = oracle.widen(q, geo.dtype)
        group = hq // geo.num_kv_heads
        sigma = float(np.float32(scale))
        out = np.zeros((t_total, hq, dim))
        for s in range(len(context_lens)):
            q0, q1 = int(query_start[s]), int(query_start[s + 1])
            n, length = q1 - q0, int(context_lens[s])
            if n == 0:
                continue
            k, v = oracle.gather_kv(k_cache, v_cache, block_tables[s], length, geo)
            for i in range(n):
                p = position(length, n, i)
                for h in range(hq):
                    z = sigma * (k[:p + 1, h // group, :] @ qf[q0 + i, h])
                    e = np.exp(z - z.max())
                    out[q0 + i, h] = (e / e.sum()) @ v[:p + 1, h // group, :]
        return out
    return prefill


def _merge_flipped(lse, parts):
    finite = np.isfinite(lse)
    m = lse[finite].max()
    w = np.where(finite, np.exp(m - np.where(finite, lse, m)), 0.0)  # sign of the exponent flipped
    return (w[:, None] * np.where(finite[:, None], parts, 0.0)).sum(axis=0) / w.sum()


def _merge_unnormalised(lse, parts):
    finite = np.isfinite(lse)
    m = lse[finite].max()
    w = np.where(finite, np.exp(np.where(finite, lse, m) - m), 0.0)
    return (w[:, None] * np.where(finite[:, None], parts, 0.0)).sum(axis=0)  # no division by the weight sum


@pytest.mark.parametrize("mutant", ["future_token", "no_prefix_offset", "merge_sign", "merge_unnormalised"])
def test_prefill_and_merge_pins_catch_planted_mistakes(monkeypatch, mutant):
    if mutant in ("future_token", "no_prefix_offset"):
        rule = (lambda L, n, i: min(L - n + i + 1, L - 1)) if mutant == "future_token" else (lambda L, n, i: i)
        # the pins call the package's name for it
        monkeypatch.setattr(oracle, "prefill", _prefill_seeing(rule))
    elif mutant == "merge_sign":
        monkeypatch.setattr(opa, "merge_partitions", _merge_flipped)
    else:
        monkeypatch.setattr(opa, "merge_partitions", _merge_unnormalised)
    pins = [test_prefill_of_one_new_token_is_decode, test_prefill_first_token_returns_its_value_row,
            lambda: _prefill_vs_sdpa(5, 2, 2, "fp32", [9, 17], [4, 17]),
            lambda: test_split_merge_equals_dense(7), lambda: test_split_merge_equals_dense(16)]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught the planted {mutant} mistake"


def _v_index_swapped(geo, b, g, o, d):
    return (b, g, o % (geo.block_size // 4), d, o // (geo.block_size // 4))  # token group and position exchanged


def _store_next_slot(k_new, v_new, slot_mapping, k_cache, v_cache, geo):
    shifted = np.where(np.asarray(slot_mapping) >= 0, np.asarray(slot_mapping) + 1, -1)
    shifted = np.where(shifted >= geo.num_blocks * geo.block_size, 0, shifted)
    return opa.__dict__["_orig_store"](k_new, v_new, shifted, k_cache, v_cache, geo)


@pytest.mark.parametrize("mutant", ["v_layout", "store_next_slot"])
def test_layout_and_store_pins_catch_planted_mistakes(monkeypatch, mutant):
    if mutant == "v_layout":
        monkeypatch.setattr(opa, "v_index", _v_index_swapped)
    else:
        monkeypatch.setitem(opa.__dict__, "_orig_store", opa.store_kvcache)
        monkeypatch.setattr(oracle, "store_kvcache", _store_next_slot)
    pins = [lambda: test_gather_matches_transpose_construction("fp16", 8), test_layout_golden_positions,
            lambda: test_store_matches_logical_assignment_and_leaves_other_bytes("bf16"),
            test_store_then_decode_sees_new_token]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught the planted {mutant} mistake"
