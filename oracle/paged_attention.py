"""Plain float64 paged-attention decode (test infrastructure only; see package docstring).

What is computed. The miniVLLM documentation (page "miniVLLM", section "What is
miniVLLM?") names two pieces: a paged KV cache kept in fixed-size pages, and a
paged-attention kernel for decode. The hysenlabs review of MinivLLM (section
on the prefilling baseline being capped at 128 tokens, last paragraph) describes
the decode benchmark's plainest baseline as a per-sequence PyTorch loop over
the paged cache, and (same section, first paragraphs) the standard form of
attention as one that materialises the whole score matrix. A decode step is
therefore: for each sequence, walk its block table to collect the keys and
values of its ``L`` context tokens, then compute ordinary softmax attention of
its one query row per head against them. Online softmax (miniVLLM docs,
"Explore by topic"; tiny-vllm note, "Chi tiết") reaches the same numbers
blockwise; the oracle does not use it.

Readings where the pages are silent (each listed in the design notes):
  * query head ``h`` attends through KV head ``h // G`` with ``G = Hq / Hkv``;
  * ``context_lens[s]`` counts the token stored in this step;
  * the score scale is the fp32 value the GPU receives, widened exactly;
  * no mask other than ``t < L``; ``L == 0`` yields zeros;
  * a negative slot in the scatter means "skip this token".

Physical cache layout (a definition of this library, not of the pages):
  * K cache ``[NB, Hkv, D/x, bs, x]`` with ``x = 16 / sizeof(T)`` elements
    (one 16-byte chunk): key element (block b, head g, offset o, dim d) lives
    at ``[b, g, d // x, o, d % x]``;
  * V cache ``[NB, Hkv, bs/4, D, 4]``: value element (b, g, o, d) lives at
    ``[b, g, o // 4, d, o % 4]``.
Token ``t`` of sequence ``s`` is offset ``t % bs`` of physical block
``block_tables[s, t // bs]``; slot ``n`` of the scatter is offset ``n % bs``
of block ``n // bs``.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np

_ELEM_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}


@dataclass(frozen=True)
class CacheGeometry:
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str

    @property
    def x(self) -> int:
        return 16 // _ELEM_BYTES[self.dtype]

    @property
    def k_shape(self) -> Tuple[int, ...]:
        return (self.num_blocks, self.num_kv_heads, self.head_dim // self.x, self.block_size, self.x)

    @property
    def v_shape(self) -> Tuple[int, ...]:
        return (self.num_blocks, self.num_kv_heads, self.block_size // 4, self.head_dim, 4)

    def check(self) -> None:
        assert self.head_dim % self.x == 0, "head_dim must be a multiple of the 16-byte chunk"
        assert self.block_size % 4 == 0, "block_size must be a multiple of 4"


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of storage-form data (bf16 is held as uint16 bit patterns)."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def k_index(geo: CacheGeometry, b, g, o, d):
    """Index tuple of key element (block b, kv head g, offset o, dim d) in the 5-D K cache."""
    x = geo.x
    return (b, g, d // x, o, d % x)


def v_index(geo: CacheGeometry, b, g, o, d):
    """Index tuple of value element (block b, kv head g, offset o, dim d) in the 5-D V cache."""
    return (b, g, o // 4, d, o % 4)


def gather_kv(k_cache: np.ndarray, v_cache: np.ndarray, block_row: np.ndarray, length: int,
              geo: CacheGeometry) -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values of tokens 0..length-1 of one sequence, float64 ``[L, Hkv, D]`` each.

    Walks the sequence's block table: token t is offset t % bs of physical
    block block_row[t // bs].
    """
    geo.check()
    k5 = np.asarray(k_cache).reshape(geo.k_shape)
    v5 = np.asarray(v_cache).reshape(geo.v_shape)
    t = np.arange(length)
    blk = np.asarray(block_row, dtype=np.int64)[t // geo.block_size]
    off = t % geo.block_size
    g = np.arange(geo.num_kv_heads)
    d = np.arange(geo.head_dim)
    B = blk[:, None, None]
    O = off[:, None, None]
    G = g[None, :, None]
    Dd = d[None, None, :]
    k = k5[k_index(geo, B, G, O, Dd)]
    v = v5[v_index(geo, B, G, O, Dd)]
    return widen(k, geo.dtype), widen(v, geo.dtype)


def _scale64(scale: float) -> float:
    # The GPU receives the scale as a float32 argument; the oracle uses that exact value.
    return float(np.float64(np.float32(scale)))


def decode_sequence(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    return_weights: bool = False):
    """Attention of one sequence: q_rows [Hq, D] float64, k/v [L, Hkv, D] float64.

    For query head h with kv head g = h // G: z_t = scale * <q_h, k_t>;
    weights = exp(z - max z) / sum exp(z - max z); output = sum_t w_t v_t.
    """
    hq, dim = q_rows.shape
    length, hkv, _ = k.shape
    group = hq // hkv
    out = np.zeros((hq, dim), dtype=np.float64)
    weights = np.zeros((hq, length), dtype=np.float64)
    if length == 0:
        return (out, weights) if return_weights else out
    sigma = _scale64(scale)
    for h in range(hq):
        g = h // group
        z = sigma * (k[:, g, :] @ q_rows[h])
        e = np.exp(z - z.max())
        w = e / e.sum()
        weights[h] = w
        out[h] = w @ v[:, g, :]
    return (out, weights) if return_weights else out


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
           context_lens: np.ndarray, scale: float, geo: CacheGeometry,
           seqs: Optional[List[int]] = None, return_weights: bool = False):
    """Paged-attention decode of a batch; returns float64 ``[B, Hq, D]`` (rows of ``seqs`` only if given).

    q is storage-form ``[B, Hq, D]``; the caches are storage-form in the
    physical layout (any shape with the right number of elements).
    """
    b_total, hq, dim = q.shape
    assert dim == geo.head_dim and hq % geo.num_kv_heads == 0
    qf = widen(q, geo.dtype)
    rows = range(b_total) if seqs is None else seqs
    out = np.zeros((b_total, hq, dim), dtype=np.float64)
    weights = {}
    for s in rows:
        length = int(context_lens[s])
        k, v = gather_kv(k_cache, v_cache, block_tables[s], length, geo)
        res = decode_sequence(qf[s], k, v, scale, return_weights=return_weights)
        if return_weights:
            out[s], weights[s] = res
        else:
            out[s] = res
    return (out, weights) if return_weights else out


def store_kvcache(k_new: np.ndarray, v_new: np.ndarray, slot_mapping: np.ndarray,
                  k_cache: np.ndarray, v_cache: np.ndarray, geo: CacheGeometry):
    """Scatter of new tokens into the caches; returns updated copies (raw values, bit-exact).

    For token i with slot n = slot_mapping[i] >= 0, every (kv head g, dim d)
    of k_new[i] / v_new[i] is written to offset n % bs of block n // bs.
    Tokens with a negative slot are skipped.
    """
    geo.check()
    k5 = np.array(k_cache, copy=True).reshape(geo.k_shape)
    v5 = np.array(v_cache, copy=True).reshape(geo.v_shape)
    g = np.arange(geo.num_kv_heads)[:, None]
    d = np.arange(geo.head_dim)[None, :]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        b, o = int(slot) // geo.block_size, int(slot) % geo.block_size
        k5[k_index(geo, b, g, o, d)] = k_new[i]
        v5[v_index(geo, b, g, o, d)] = v_new[i]
    return k5.reshape(np.shape(k_cache)), v5.reshape(np.shape(v_cache))


def merge_partitions(lse: np.ndarray, parts: np.ndarray) -> np.ndarray:
    """Combine per-partition results of one (sequence, head).

    lse[p] is the natural-log sum of exp(z) over partition p (-inf if empty),
    parts[p] the partition's own normalised output. The full result is the
    average of the parts weighted by exp(lse[p]); computed relative to the
    largest lse so nothing overflows.
    """
    finite = np.isfinite(lse)
    if not finite.any():
        return np.zeros(parts.shape[1:], dtype=np.float64)
    m = lse[finite].max()
    w = np.where(finite, np.exp(np.where(finite, lse, m) - m), 0.0)
    return (w[:, None] * np.where(finite[:, None], parts, 0.0)).sum(axis=0) / w.sum()


def decode_split(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                 context_lens: np.ndarray, scale: float, geo: CacheGeometry, partition_size: int,
                 seqs: Optional[List[int]] = None):
    """Decode by context partitions of ``partition_size`` tokens, then merge.

    Returns (merged [B, Hq, D], lse list, parts list). Each partition is
    computed with the same dense definition as ``decode_sequence`` restricted
    to its tokens; the merge is ``merge_partitions``. In exact arithmetic the
    merged result equals ``decode``.
    """
    b_total, hq, dim = q.shape
    qf = widen(q, geo.dtype)
    sigma = _scale64(scale)
    group = hq // geo.num_kv_heads
    rows = range(b_total) if seqs is None else seqs
    out = np.zeros((b_total, hq, dim), dtype=np.float64)
    all_lse, all_parts = {}, {}
    for s in rows:
        length = int(context_lens[s])
        k, v = gather_kv(k_cache, v_cache, block_tables[s], length, geo)
        nparts = max(1, -(-length // partition_size))
        lse = np.full((hq, nparts), -np.inf)
        parts = np.zeros((hq, nparts, dim))
        for h in range(hq):
            g = h // group
            for p in range(nparts):
                lo, hi = p * partition_size, min(length, (p + 1) * partition_size)
                if hi <= lo:
                    continue
                z = sigma * (k[lo:hi, g, :] @ qf[s, h])
                m = z.max()
                e = np.exp(z - m)
                lse[h, p] = m + np.log(e.sum())
                parts[h, p] = (e / e.sum()) @ v[lo:hi, g, :]
            out[s, h] = merge_partitions(lse[h], parts[h])
        all_lse[s], all_parts[s] = lse, parts
    return out, all_lse, all_parts


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
            context_lens: np.ndarray, query_start: np.ndarray, scale: float, geo: CacheGeometry,
            seqs: Optional[List[int]] = None) -> np.ndarray:
    """Causal attention of each sequence's new tokens over its paged context; float64 ``[T, Hq, D]``.

    Sequence s owns query rows query_start[s] .. query_start[s+1]-1 of q
    (``[T, Hq, D]`` storage form). With n_s of them and L_s = context_lens[s]
    tokens in the cache (the new ones included), query i sits at position
    p = L_s - n_s + i and attends to tokens 0 .. p (flash-attention prefill of
    the miniVLLM docs, "What is miniVLLM?"; the standard materialised form of
    the hysenlabs MinivLLM review, prefilling-baseline section). n_s = 1 is
    the decode case.
    """
    t_total, hq, dim = q.shape
    qf = widen(q, geo.dtype)
    group = hq // geo.num_kv_heads
    sigma = _scale64(scale)
    out = np.zeros((t_total, hq, dim), dtype=np.float64)
    rows = range(len(context_lens)) if seqs is None else seqs
    for s in rows:
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        n, length = q1 - q0, int(context_lens[s])
        if n == 0:
            continue
        assert n <= length, "more new tokens than context"
        k, v = gather_kv(k_cache, v_cache, block_tables[s], length, geo)
        for i in range(n):
            p = length - n + i
            for h in range(hq):
                g = h // group
                z = sigma * (k[:p + 1, g, :] @ qf[q0 + i, h])
                e = np.exp(z - z.max())
                out[q0 + i, h] = (e / e.sum()) @ v[:p + 1, g, :]
    return out
