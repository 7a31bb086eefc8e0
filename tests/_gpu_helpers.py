"""Helpers for GPU parity tests: move generator output to the device, compare with the oracle."""

from __future__ import annotations

import numpy as np

import oracle
from workloads import Config, make_inputs

TORCH_DT = {"fp32": "float32", "fp16": "float16", "bf16": "bfloat16"}
TOL = {"fp32": 1e-5, "fp16": 2e-3, "bf16": 2e-3}


def torch_dtype(dt: str):
    import torch
    return getattr(torch, TORCH_DT[dt])


def np_to_torch(a: np.ndarray, dt: str):
    import torch
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def torch_to_np(t, dt: str) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def geometry(x) -> oracle.CacheGeometry:
    c = x.cfg
    return oracle.CacheGeometry(x.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.dtype)


def to_device(x, device):
    """Device tensors for one workload; caches viewed in the library's physical layout."""
    import torch
    import paged_attention_decode_amd as pa
    c = x.cfg
    tdt = torch_dtype(c.dtype)
    kshape = pa.k_cache_shape(x.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, tdt)
    vshape = pa.v_cache_shape(x.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, tdt)
    return {
        "q": np_to_torch(x.q, c.dtype).to(device),
        "k_cache": np_to_torch(x.k_cache, c.dtype).view(kshape).to(device),
        "v_cache": np_to_torch(x.v_cache, c.dtype).view(vshape).to(device),
        "block_tables": torch.from_numpy(x.block_tables).to(device),
        "context_lens": torch.from_numpy(x.context_lens).to(device),
        "k_new": np_to_torch(x.k_new, c.dtype).to(device),
        "v_new": np_to_torch(x.v_new, c.dtype).to(device),
        "slot_mapping": torch.from_numpy(x.slot_mapping).to(device),
    }


def custom_config(dtype="bf16", batch=4, hq=8, hkv=2, d=128, bs=16, lens=(1, 17, 100, 333), q_mult=1.0,
                  scale=None, seed=7, prefix_group=0, prefix_tokens=0):
    return Config(name="custom", dtype=dtype, batch=batch, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                  block_size=bs, lengths="list", len_list=tuple(lens), q_mult=q_mult, scale=scale, seed=seed,
                  prefix_group=prefix_group, prefix_tokens=prefix_tokens)


def oracle_after_store(x, seqs=None):
    """Oracle caches after the step's scatter, and the oracle decode of ``seqs``."""
    geo = geometry(x)
    k2, v2 = oracle.store_kvcache(x.k_new, x.v_new, x.slot_mapping, x.k_cache, x.v_cache, geo)
    out = oracle.decode(x.q, k2, v2, x.block_tables, x.context_lens, x.scale, geo, seqs=seqs)
    return k2, v2, out


def half_ulp(ref: np.ndarray, dt: str) -> np.ndarray:
    """Half a unit in the last place of dtype ``dt`` at the magnitude of ``ref``."""
    mant = {"fp32": 23, "fp16": 10, "bf16": 7}[dt]
    mag = np.maximum(np.abs(ref), {"fp32": 2.0 ** -126, "fp16": 2.0 ** -14, "bf16": 2.0 ** -126}[dt])
    return 0.5 * 2.0 ** (np.floor(np.log2(mag)) - mant)
