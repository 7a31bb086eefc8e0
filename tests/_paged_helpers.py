"""Test-side construction of paged caches from dense per-sequence K/V.

Places logical rows into the physical layout with numpy reshape/transpose (a
library routine), independently of the oracle's explicit index arithmetic, so
that the two can pin each other.
"""

from __future__ import annotations

import numpy as np

from workloads import to_storage

ELEM = {"fp32": 4, "fp16": 2, "bf16": 2}
STORE_NP = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}


def chunk_elems(dtype: str) -> int:
    return 16 // ELEM[dtype]


def logical_to_physical_k(k_log: np.ndarray, dtype: str) -> np.ndarray:
    """[NB, Hkv, bs, D] -> [NB, Hkv, D/x, bs, x]."""
    nb, hkv, bs, d = k_log.shape
    x = chunk_elems(dtype)
    return np.ascontiguousarray(k_log.reshape(nb, hkv, bs, d // x, x).transpose(0, 1, 3, 2, 4))


def logical_to_physical_v(v_log: np.ndarray) -> np.ndarray:
    """[NB, Hkv, bs, D] -> [NB, Hkv, bs/4, D, 4]."""
    nb, hkv, bs, d = v_log.shape
    return np.ascontiguousarray(v_log.reshape(nb, hkv, bs // 4, 4, d).transpose(0, 1, 2, 4, 3))


def physical_to_logical_k(k_phys: np.ndarray, nb, hkv, bs, d, dtype) -> np.ndarray:
    x = chunk_elems(dtype)
    return np.ascontiguousarray(k_phys.reshape(nb, hkv, d // x, bs, x).transpose(0, 1, 3, 2, 4).reshape(nb, hkv, bs, d))


def physical_to_logical_v(v_phys: np.ndarray, nb, hkv, bs, d) -> np.ndarray:
    return np.ascontiguousarray(v_phys.reshape(nb, hkv, bs // 4, d, 4).transpose(0, 1, 2, 4, 3).reshape(nb, hkv, bs, d))


def widen_np(a: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of storage-form data through torch's own conversions (bf16 patterns are
    uint16), independent of the oracle's widening."""
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return torch.from_numpy(a).to(torch.float64).numpy()


class PagedCase:
    """Dense per-sequence K/V plus the same data scattered into a shuffled block pool."""

    def __init__(self, rng, batch, hq, hkv, d, bs, lens, dtype="fp32", extra_blocks=3,
                 k_dense=None, v_dense=None, q=None):
        self.dtype, self.hq, self.hkv, self.d, self.bs = dtype, hq, hkv, d, bs
        self.lens = np.asarray(lens, dtype=np.int32)
        nblk = [-(-int(L) // bs) for L in lens]
        self.mb = max(1, max(nblk))
        self.nb = sum(nblk) + extra_blocks
        perm = rng.permutation(self.nb)
        self.tables = np.zeros((batch, self.mb), dtype=np.int32)
        k_log = to_storage(rng.standard_normal((self.nb, hkv, bs, d), dtype=np.float32), dtype)
        v_log = to_storage(rng.standard_normal((self.nb, hkv, bs, d), dtype=np.float32), dtype)
        self.k_dense, self.v_dense = [], []
        nxt = 0
        for s in range(batch):
            L = int(lens[s])
            blocks = perm[nxt:nxt + nblk[s]]
            nxt += nblk[s]
            self.tables[s, :len(blocks)] = blocks
            self.tables[s, len(blocks):] = perm[-1]
            if k_dense is not None:
                kd = np.asarray(k_dense[s])
                vd = np.asarray(v_dense[s])
            else:
                kd = np.empty((L, hkv, d), dtype=STORE_NP[dtype])
                vd = np.empty((L, hkv, d), dtype=STORE_NP[dtype])
                for t in range(L):
                    kd[t] = k_log[blocks[t // bs], :, t % bs, :]
                    vd[t] = v_log[blocks[t // bs], :, t % bs, :]
            for t in range(L):
                k_log[blocks[t // bs], :, t % bs, :] = kd[t]
                v_log[blocks[t // bs], :, t % bs, :] = vd[t]
            self.k_dense.append(kd)
            self.v_dense.append(vd)
        self.k_log, self.v_log = k_log, v_log
        self.k_cache = logical_to_physical_k(k_log, dtype)
        self.v_cache = logical_to_physical_v(v_log)
        if q is None:
            q = to_storage(rng.standard_normal((batch, hq, d), dtype=np.float32), dtype)
        self.q = np.asarray(q)

    def geometry(self):
        import oracle
        return oracle.CacheGeometry(self.nb, self.hkv, self.d, self.bs, self.dtype)


def sdpa_reference(q64: np.ndarray, k64: np.ndarray, v64: np.ndarray, scale: float) -> np.ndarray:
    """torch scaled_dot_product_attention in float64 on CPU; k/v [L, Hkv, D] repeated per query group."""
    import torch
    hq = q64.shape[0]
    L, hkv, d = k64.shape
    if L == 0:
        return np.zeros((hq, d))
    g = hq // hkv
    qt = torch.from_numpy(q64).reshape(1, hq, 1, d)
    kt = torch.from_numpy(k64).permute(1, 0, 2).repeat_interleave(g, dim=0).reshape(1, hq, L, d).contiguous()
    vt = torch.from_numpy(v64).permute(1, 0, 2).repeat_interleave(g, dim=0).reshape(1, hq, L, d).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return out.reshape(hq, d).numpy()
