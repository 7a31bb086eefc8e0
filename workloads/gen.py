"""Seeded input generation for the decode workloads.

Draw order per workload (one ``numpy.random.default_rng(seed)`` stream):
context lengths, physical-block permutation, K cache values, V cache values,
q, new k, new v.

Values are float32 N(0, 1) draws (q times ``q_mult``) rounded to the storage
type with round-to-nearest-even. Storage form on the host:
``fp32`` -> numpy float32, ``fp16`` -> numpy float16, ``bf16`` -> numpy uint16
holding the bfloat16 bit pattern.

The caches are returned flat: ``num_blocks * num_kv_heads * block_size *
head_dim`` i.i.d. values. Physical block ``b`` owns the contiguous range
``[b * E, (b + 1) * E)`` with ``E = num_kv_heads * block_size * head_dim``;
the arrangement inside a block is the consumer's business.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .configs import Config

_CHUNK = 1 << 24


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type (RNE)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x
    if dtype == "fp16":
        return x.astype(np.float16)
    if dtype == "bf16":
        import torch
        out = np.empty(x.shape, dtype=np.uint16)
        flat_in = x.reshape(-1)
        flat_out = out.reshape(-1)
        for i in range(0, flat_in.size, _CHUNK):
            t = torch.from_numpy(flat_in[i:i + _CHUNK]).to(torch.bfloat16)
            flat_out[i:i + _CHUNK] = t.view(torch.int16).numpy().view(np.uint16)
        return out
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal_storage(rng: np.random.Generator, n: int, dtype: str, mult: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype={"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}[dtype])
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        x = rng.standard_normal(m, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out[i:i + m] = to_storage(x, dtype)
    return out


def draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Context lengths, each including the token stored in this step."""
    b = cfg.batch
    if cfg.lengths == "list":
        assert len(cfg.len_list) == b
        lens = np.array(cfg.len_list, dtype=np.int64)
    elif cfg.lengths == "fixed":
        lens = np.full(b, cfg.len_hi, dtype=np.int64)
    elif cfg.lengths == "uniform":
        lens = rng.integers(cfg.len_lo, cfg.len_hi, size=b, endpoint=True)
    elif cfg.lengths == "lognormal":
        z = rng.standard_normal(b)
        lens = np.rint(np.exp(math.log(cfg.len_median) + cfg.len_sigma * z))
        lens = np.clip(lens, cfg.len_lo, cfg.len_hi).astype(np.int64)
    else:
        raise ValueError(cfg.lengths)
    return lens.astype(np.int32)


@dataclass
class Inputs:
    cfg: Config
    context_lens: np.ndarray      # [B] int32
    block_tables: np.ndarray      # [B, MB] int32
    num_blocks: int
    k_cache: np.ndarray           # flat storage, NB*Hkv*bs*D
    v_cache: np.ndarray
    q: np.ndarray                 # [B, Hq, D] storage
    k_new: np.ndarray             # [B, Hkv, D] storage
    v_new: np.ndarray
    slot_mapping: np.ndarray      # [B] int32: slot of token L-1 of each sequence (-1 when L = 0)
    scale: float
    unused_blocks: List[int] = field(default_factory=list)
    shared_blocks: List[int] = field(default_factory=list)

    @property
    def kv_bytes(self) -> int:
        """Logical K+V bytes one decode reads: sum_s L_s * Hkv * D * e * 2."""
        c = self.cfg
        return int(self.context_lens.astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * c.elem_bytes * 2

    @property
    def unique_kv_bytes(self) -> int:
        """K+V bytes of the distinct (block, token) slots referenced by the batch."""
        c = self.cfg
        seen = set()
        tokens = 0
        for s in range(c.batch):
            L = int(self.context_lens[s])
            nb = -(-L // c.block_size)
            for j in range(nb):
                blk = int(self.block_tables[s, j])
                used = min(c.block_size, L - j * c.block_size)
                key = blk
                if key in seen:
                    continue
                seen.add(key)
                tokens += used if j == nb - 1 else c.block_size
        return tokens * c.num_kv_heads * c.head_dim * c.elem_bytes * 2


def _assign_blocks(cfg: Config, lens: np.ndarray, rng: np.random.Generator):
    bs = cfg.block_size
    b = cfg.batch
    nblk = [-(-int(L) // bs) for L in lens]
    mb = cfg.max_blocks_per_seq
    if cfg.prefix_group > 0:
        pre = cfg.prefix_tokens // bs
        ngroups = -(-b // cfg.prefix_group)
        n_shared = [min(pre, (int(L) - 1) // bs) for L in lens]
        group_shared = [max(n_shared[g * cfg.prefix_group:(g + 1) * cfg.prefix_group]) for g in range(ngroups)]
        unique = sum(group_shared) + sum(nb - ns for nb, ns in zip(nblk, n_shared))
    else:
        n_shared = [0] * b
        group_shared = []
        unique = sum(nblk)
    pool = cfg.pool_blocks if cfg.pool_blocks is not None else int(math.ceil(1.25 * unique))
    assert pool >= unique, (pool, unique)
    perm = rng.permutation(pool).astype(np.int64)
    nxt = 0
    shared_ids = []
    for gs in group_shared:
        shared_ids.append(perm[nxt:nxt + gs])
        nxt += gs
    tables = np.empty((b, mb), dtype=np.int64)
    for s in range(b):
        row = []
        if cfg.prefix_group > 0:
            row.extend(int(x) for x in shared_ids[s // cfg.prefix_group][:n_shared[s]])
        priv = nblk[s] - n_shared[s]
        row.extend(int(x) for x in perm[nxt:nxt + priv])
        nxt += priv
        tables[s, :len(row)] = row
        tables[s, len(row):] = -1
    unused = [int(x) for x in perm[nxt:]]
    filler = unused[0] if unused else int(perm[0])
    tables[tables < 0] = filler
    shared = sorted(int(x) for ids in shared_ids for x in ids)
    return tables.astype(np.int32), pool, unused, shared


def make_inputs(cfg: Config, seed: Optional[int] = None, structure_only: bool = False) -> Inputs:
    """Draw one workload. ``structure_only`` stops after the block tables (no values drawn)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lens = draw_lengths(cfg, rng)
    tables, pool, unused, shared = _assign_blocks(cfg, lens, rng)
    bs = cfg.block_size
    pos = lens.astype(np.int64) - 1
    slots = (tables[np.arange(cfg.batch), pos // bs].astype(np.int64) * bs + pos % bs).astype(np.int32)
    # An empty context has no token at position L-1: nothing to store (a negative slot is skipped).
    slots[lens == 0] = -1
    if structure_only:
        empty = np.zeros(0, np.float32)
        return Inputs(cfg=cfg, context_lens=lens, block_tables=tables, num_blocks=pool,
                      k_cache=empty, v_cache=empty, q=empty, k_new=empty, v_new=empty,
                      slot_mapping=slots, scale=cfg.softmax_scale, unused_blocks=unused,
                      shared_blocks=shared)
    elems = pool * cfg.num_kv_heads * cfg.block_size * cfg.head_dim
    k_cache = _normal_storage(rng, elems, cfg.dtype)
    v_cache = _normal_storage(rng, elems, cfg.dtype)
    q = _normal_storage(rng, cfg.batch * cfg.num_heads * cfg.head_dim, cfg.dtype, cfg.q_mult)
    q = q.reshape(cfg.batch, cfg.num_heads, cfg.head_dim)
    kn = _normal_storage(rng, cfg.batch * cfg.num_kv_heads * cfg.head_dim, cfg.dtype)
    vn = _normal_storage(rng, cfg.batch * cfg.num_kv_heads * cfg.head_dim, cfg.dtype)
    kn = kn.reshape(cfg.batch, cfg.num_kv_heads, cfg.head_dim)
    vn = vn.reshape(cfg.batch, cfg.num_kv_heads, cfg.head_dim)
    return Inputs(cfg=cfg, context_lens=lens, block_tables=tables, num_blocks=pool,
                  k_cache=k_cache, v_cache=v_cache, q=q, k_new=kn, v_new=vn,
                  slot_mapping=slots, scale=cfg.softmax_scale,
                  unused_blocks=unused, shared_blocks=shared)


def nan_of(dtype: str):
    """The storage-form NaN value for ``dtype``."""
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    if dtype == "fp16":
        return np.float16(np.nan)
    return np.float32(np.nan)


def poison_blocks(cache: np.ndarray, blocks, cfg: Config) -> np.ndarray:
    """Return a copy of a flat cache with every element of ``blocks`` set to NaN."""
    out = cache.copy()
    e = cfg.num_kv_heads * cfg.block_size * cfg.head_dim
    nan = nan_of(cfg.dtype)
    for b in blocks:
        out[b * e:(b + 1) * e] = nan
    return out
