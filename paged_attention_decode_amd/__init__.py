"""Python binding of libpagedattn (paged-attention decode for MI355X / gfx950).

Argument marshalling only: torch tensors are turned into device pointers,
sizes, strides and the current HIP stream, and every step runs in the HIP
kernels of ``libpagedattn.so``. There is no fallback: if the library is not
built, or a call fails, an exception is raised.

Entry points (same names as the C ABI in ``include/pagedattn.h``):

* ``store_kvcache(k, v, slot_mapping, k_cache, v_cache)``
* ``paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None, ...)``

Cache tensors use the library's physical layout; ``allocate_kv_cache`` creates
them and ``k_cache_shape`` / ``v_cache_shape`` give the shapes:

* K: ``[num_blocks, num_kv_heads, head_dim // x, block_size, x]`` with
  ``x = 16 // element_size``
* V: ``[num_blocks, num_kv_heads, block_size // 4, head_dim, 4]``
"""

from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional, Tuple

__all__ = [
    "PagedAttnError", "store_kvcache", "paged_attention_decode", "allocate_kv_cache",
    "k_cache_shape", "v_cache_shape", "decode_plan", "workspace_bytes", "version", "shutdown",
    "library_path", "load_library", "DTYPE_F32", "DTYPE_F16", "DTYPE_BF16", "BlockManager", "copy_blocks",
    "decode_step", "paged_prefill", "DEFAULT_CACHED_PREFIX_TOKENS", "paged_attention_decode_noalloc",
    "NOALLOC_SCRATCH_BYTES",
]

# Always the in-tree build next to this file: the binding loads no other library.
_LIB_PATH = Path(__file__).resolve().with_name("libpagedattn.so")
_lib = None

DTYPE_F32, DTYPE_F16, DTYPE_BF16 = 0, 1, 2
# PA_DEFAULT_CACHED_PREFIX_TOKENS: what cached_prefix_tokens = 0 selects.
DEFAULT_CACHED_PREFIX_TOKENS = 1024
# PA_NOALLOC_SCRATCH_BYTES: the fixed workspace of pa_paged_attention_decode_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20
_STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_DTYPE", 3: "PA_ERR_SHAPE", 4: "PA_ERR_UNSUPPORTED",
           5: "PA_ERR_WORKSPACE", 6: "PA_ERR_HIP", 7: "PA_ERR_CAPACITY"}


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_STATUS.get(code, code)}: {message}")
        self.code = code


class DecodeOpts(ctypes.Structure):
    _fields_ = [
        ("partition_size", ctypes.c_int32),
        ("cached_prefix_tokens", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("event_begin", ctypes.c_void_p),
        ("event_end", ctypes.c_void_p),
        ("shared_prefix", ctypes.c_int32),
    ]


def library_path() -> Path:
    return _LIB_PATH


def load_library():
    """Load libpagedattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m paged_attention_decode_amd.build`")
    lib = ctypes.CDLL(str(_LIB_PATH))
    c_int, c_i64, c_p, c_f = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.pa_store_kvcache.argtypes = [c_p, c_p, c_p, c_p, c_p, c_int, c_int, c_int, c_int, c_i64, c_i64, c_i64,
                                     c_int, c_p]
    lib.pa_store_kvcache.restype = c_int
    dec = [c_p, c_p, c_p, c_p, c_p, c_f, c_p, c_int, c_int, c_int, c_int, c_int, c_int, c_i64, c_i64, c_int, c_int]
    lib.pa_paged_attention_decode.argtypes = dec + [c_p]
    lib.pa_paged_attention_decode.restype = c_int
    lib.pa_paged_attention_decode_ex.argtypes = dec + [ctypes.POINTER(DecodeOpts), c_p]
    lib.pa_paged_attention_decode_ex.restype = c_int
    lib.pa_paged_attention_decode_noalloc.argtypes = dec + [ctypes.POINTER(DecodeOpts), c_p]
    lib.pa_paged_attention_decode_noalloc.restype = c_int
    lib.pa_decode_step.argtypes = [c_p, c_p, c_p, c_i64, c_i64, c_p, c_p, c_p, c_p, c_f, c_p, c_int, c_int, c_int,
                                   c_int, c_int, c_int, c_i64, c_i64, c_int, c_int, ctypes.POINTER(DecodeOpts), c_p]
    lib.pa_decode_step.restype = c_int
    lib.pa_paged_prefill.argtypes = [c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_f, c_p, c_int, c_int, c_int, c_int, c_int,
                                     c_int, c_int, c_i64, c_int, c_int, c_p]
    lib.pa_paged_prefill.restype = c_int
    lib.pa_decode_plan.argtypes = [c_int] * 9 + [ctypes.POINTER(c_i64), ctypes.POINTER(c_int),
                                                 ctypes.POINTER(c_int), ctypes.POINTER(ctypes.c_size_t)]
    lib.pa_decode_plan.restype = c_int
    lib.pa_decode_plan_ex.argtypes = [c_int] * 7 + [ctypes.POINTER(DecodeOpts), c_int, ctypes.POINTER(c_i64),
                                                    ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                                    ctypes.POINTER(c_int), ctypes.POINTER(ctypes.c_size_t)]
    lib.pa_decode_plan_ex.restype = c_int
    lib.pa_decode_workspace_bytes.argtypes = [c_int] * 8
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    lib.pa_shutdown.argtypes = []
    lib.pa_shutdown.restype = c_int
    lib.pa_copy_blocks.argtypes = [c_p, c_p, c_p, c_p, c_int, c_int, c_int, c_int, c_i64, c_int, c_p]
    lib.pa_copy_blocks.restype = c_int
    p_i32, p_i64 = ctypes.POINTER(c_int), ctypes.POINTER(c_i64)
    lib.pa_bm_create.argtypes = [c_int, c_int]
    lib.pa_bm_create.restype = c_p
    lib.pa_bm_destroy.argtypes = [c_p]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_add_sequence.argtypes = [c_p, c_i64, p_i32, c_int, p_i32]
    lib.pa_bm_append_token.argtypes = [c_p, c_i64, c_int, p_i32, p_i32, p_i32]
    lib.pa_bm_fork.argtypes = [c_p, c_i64, c_i64]
    lib.pa_bm_free_sequence.argtypes = [c_p, c_i64]
    lib.pa_bm_block_table.argtypes = [c_p, c_i64, p_i32, c_int, p_i32, p_i32]
    lib.pa_bm_slots.argtypes = [c_p, c_i64, c_int, c_int, p_i32]
    lib.pa_bm_stats.argtypes = [c_p, p_i32, p_i32, p_i64, p_i64, p_i64]
    lib.pa_bm_block_ref.argtypes = [c_p, c_int]
    lib.pa_bm_last_error.argtypes = []
    lib.pa_bm_last_error.restype = ctypes.c_char_p
    for f in (lib.pa_bm_add_sequence, lib.pa_bm_append_token, lib.pa_bm_fork, lib.pa_bm_free_sequence,
              lib.pa_bm_block_table, lib.pa_bm_slots, lib.pa_bm_stats, lib.pa_bm_block_ref):
        f.restype = c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise PagedAttnError(rc, load_library().pa_last_error().decode())


_DTYPE_CODES = None


def _dtype_code(dt) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16}
    code = _DTYPE_CODES.get(dt)
    if code is None:
        raise TypeError(f"unsupported dtype {dt}")
    return code


def _elem(dt) -> int:
    import torch
    return torch.empty((), dtype=dt).element_size()


def k_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int, dtype) -> Tuple[int, ...]:
    x = 16 // _elem(dtype)
    return (num_blocks, num_kv_heads, head_dim // x, block_size, x)


def v_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int, dtype=None) -> Tuple[int, ...]:
    return (num_blocks, num_kv_heads, block_size // 4, head_dim, 4)


def allocate_kv_cache(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int, dtype, device="cuda"):
    """Uninitialised (k_cache, v_cache) in the library's physical layout."""
    import torch
    k = torch.empty(k_cache_shape(num_blocks, num_kv_heads, head_dim, block_size, dtype), dtype=dtype, device=device)
    v = torch.empty(v_cache_shape(num_blocks, num_kv_heads, head_dim, block_size), dtype=dtype, device=device)
    return k, v


_raw_stream = None


def _stream_of(t) -> int:
    """Handle of the current stream of t's device (what torch's current_stream().cuda_stream gives,
    read without building a Stream object: about 0.1 us instead of 1.7 us per call)."""
    global _raw_stream
    if _raw_stream is None:
        import torch
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None) or \
            (lambda idx: torch.cuda.current_stream(idx).cuda_stream)
    return _raw_stream(t.get_device())


def _cache_geometry(k_cache, v_cache):
    ks, vs = k_cache.shape, v_cache.shape
    if len(ks) != 5 or len(vs) != 5:
        raise ValueError("k_cache and v_cache must be 5-D tensors in the library layout")
    nb, hkv, chunks, bs, x = ks
    if x != 16 // k_cache.element_size():
        raise ValueError(f"k_cache innermost dim {x} must be {16 // k_cache.element_size()}")
    d = chunks * x
    if vs != (nb, hkv, bs // 4, d, 4):
        raise ValueError(f"v_cache shape {tuple(vs)} does not match k_cache {tuple(ks)}")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache dtypes differ")
    return nb, hkv, d, bs


def _require_cuda(*ts):
    """All tensors on one GPU (get_device() is -1 for host tensors)."""
    dev = ts[0].get_device()
    if dev < 0:
        raise ValueError("all tensors must be on the same GPU")
    for t in ts:
        if t.get_device() != dev:
            raise ValueError("all tensors must be on the same GPU")


def store_kvcache(k, v, slot_mapping, k_cache, v_cache) -> None:
    """Write k[i], v[i] ([N, Hkv, D]) into slot slot_mapping[i] of the caches (slots < 0 skipped)."""
    import torch
    lib = _lib or load_library()
    _require_cuda(k, v, slot_mapping, k_cache, v_cache)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    ks = k.shape
    if len(ks) != 3 or ks[1:] != (hkv, d) or v.shape != ks:
        raise ValueError(f"k, v must be [N, {hkv}, {d}], got {tuple(k.shape)}, {tuple(v.shape)}")
    n = ks[0]
    if slot_mapping.shape != (n,):
        raise ValueError("k, v and slot_mapping disagree on the token count")
    if slot_mapping.dtype != torch.int32 or not slot_mapping.is_contiguous():
        raise TypeError("slot_mapping must be a contiguous int32 tensor")
    dt = k_cache.dtype
    if k.dtype != dt or v.dtype != dt:
        raise TypeError("k, v and the caches must share one dtype")
    kst, vst = k.stride(), v.stride()
    if kst[1:] != (d, 1) or vst[1:] != (d, 1):
        raise ValueError("k and v need contiguous [Hkv, D] rows")
    _check(lib.pa_store_kvcache(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
                                v_cache.data_ptr(), n, hkv, d, bs, nb, kst[0], vst[0],
                                _dtype_code(dt), _stream_of(k_cache)))


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out=None, *,
                           out_dtype=None, partition_size: int = 0, cached_prefix_tokens: int = 0,
                           workspace=None, events=None, shared_prefix: bool = False):
    """Decode attention; returns ``out`` ([B, Hq, D], fp32 or q's dtype).

    partition_size: 0 automatic (default: one pass when max_blocks_per_seq *
    block_size <= 512, else balanced split), -1 one pass per sequence, -2
    balanced split, -3 workgroup split (four wavefronts per (sequence, kv head),
    merged in LDS), >0 fixed ranges of that many tokens. cached_prefix_tokens: leading tokens
    of each context read with cached loads, the rest streamed (0 library
    default, -1 stream all; speed only). workspace: optional uint8 CUDA tensor
    (see ``workspace_bytes``). events: optional (begin, end) torch.cuda.Event
    pair recorded around the attention kernel itself. shared_prefix: read the
    leading blocks that neighbouring sequences share (same physical ids) once
    per group; found on the device, split modes only (see pa_decode_opts).
    """
    import torch
    lib = _lib or load_library()
    _require_cuda(q, k_cache, v_cache, block_tables, context_lens)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    qs, qst = q.shape, q.stride()
    if len(qs) != 3 or qs[2] != d or qst[1:] != (d, 1):
        raise ValueError(f"q must be [B, Hq, {d}] with contiguous head rows")
    bsz, hq = qs[0], qs[1]
    if q.dtype != k_cache.dtype:
        raise TypeError("q and the caches must share one dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    bts = block_tables.shape
    if len(bts) != 2 or bts[0] != bsz or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous [B, max_blocks] tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] tensor")
    if out is None:
        odt = out_dtype if out_dtype is not None else q.dtype
        out = torch.empty((bsz, hq, d), dtype=odt, device=q.device)
    elif out.shape != (bsz, hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, D] tensor")
    else:
        _require_cuda(q, out)
    opts = DecodeOpts()
    opts.partition_size = int(partition_size)
    opts.cached_prefix_tokens = int(cached_prefix_tokens)
    opts.shared_prefix = 1 if shared_prefix else 0
    if workspace is not None:
        _require_cuda(q, workspace)
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    if events is not None:
        for ev in events:
            if not ev.cuda_event:
                ev.record()  # a torch event gets its HIP handle on first record
        opts.event_begin = events[0].cuda_event
        opts.event_end = events[1].cuda_event
    _check(lib.pa_paged_attention_decode_ex(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        float(scale), out.data_ptr(), bsz, hq, hkv, d, bs, bts[1], nb, qst[0],
        _dtype_code(q.dtype), _dtype_code(out.dtype), ctypes.byref(opts), _stream_of(q)))
    return out


def paged_attention_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, out, *,
                                   partition_size: int = 0, cached_prefix_tokens: int = 0, events=None,
                                   shared_prefix: bool = False):
    """pa_paged_attention_decode_noalloc: paged_attention_decode into a caller-given ``out`` with
    the library's fixed scratch as workspace; the call allocates no device memory (raises
    PagedAttnError PA_ERR_WORKSPACE when the plan needs more than NOALLOC_SCRATCH_BYTES)."""
    import torch
    lib = _lib or load_library()
    _require_cuda(q, k_cache, v_cache, block_tables, context_lens, out)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    qs, qst = q.shape, q.stride()
    if len(qs) != 3 or qs[2] != d or qst[1:] != (d, 1):
        raise ValueError(f"q must be [B, Hq, {d}] with contiguous head rows")
    bsz, hq = qs[0], qs[1]
    if q.dtype != k_cache.dtype:
        raise TypeError("q and the caches must share one dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    bts = block_tables.shape
    if len(bts) != 2 or bts[0] != bsz or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous [B, max_blocks] tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] tensor")
    if out.shape != (bsz, hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, D] tensor")
    opts = DecodeOpts()
    opts.partition_size = int(partition_size)
    opts.cached_prefix_tokens = int(cached_prefix_tokens)
    opts.shared_prefix = 1 if shared_prefix else 0
    if events is not None:
        for ev in events:
            if not ev.cuda_event:
                ev.record()
        opts.event_begin = events[0].cuda_event
        opts.event_end = events[1].cuda_event
    _check(lib.pa_paged_attention_decode_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        float(scale), out.data_ptr(), bsz, hq, hkv, d, bs, bts[1], nb, qst[0],
        _dtype_code(q.dtype), _dtype_code(out.dtype), ctypes.byref(opts), _stream_of(q)))
    return out


def decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale: float, out=None, *,
                out_dtype=None, partition_size: int = 0, cached_prefix_tokens: int = 0, workspace=None,
                events=None, shared_prefix: bool = False):
    """Fused decode step: write k_new/v_new ([B, Hkv, D]) at position L-1 of each sequence and attend.

    Same result as store_kvcache (at each sequence's last position) followed by
    paged_attention_decode, in one kernel launch.
    """
    import torch
    lib = _lib or load_library()
    _require_cuda(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    qs, qst = q.shape, q.stride()
    if len(qs) != 3 or qs[2] != d or qst[1:] != (d, 1):
        raise ValueError(f"q must be [B, Hq, {d}] with contiguous head rows")
    bsz, hq = qs[0], qs[1]
    knst, vnst = k_new.stride(), v_new.stride()
    if k_new.shape != (bsz, hkv, d) or v_new.shape != (bsz, hkv, d) or knst[1:] != (d, 1) or vnst[1:] != (d, 1):
        raise ValueError(f"k_new, v_new must be [{bsz}, {hkv}, {d}] with contiguous head rows")
    if q.dtype != k_cache.dtype or k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("q, k_new, v_new and the caches must share one dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    bts = block_tables.shape
    if len(bts) != 2 or bts[0] != bsz or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous [B, max_blocks] tensor")
    if context_lens.shape != (bsz,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be a contiguous [B] tensor")
    if out is None:
        odt = out_dtype if out_dtype is not None else q.dtype
        out = torch.empty((bsz, hq, d), dtype=odt, device=q.device)
    elif out.shape != (bsz, hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, D] tensor")
    else:
        _require_cuda(q, out)
    opts = DecodeOpts()
    opts.partition_size = int(partition_size)
    opts.cached_prefix_tokens = int(cached_prefix_tokens)
    opts.shared_prefix = 1 if shared_prefix else 0
    if workspace is not None:
        _require_cuda(q, workspace)
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    if events is not None:
        for ev in events:
            if not ev.cuda_event:
                ev.record()
        opts.event_begin = events[0].cuda_event
        opts.event_end = events[1].cuda_event
    _check(lib.pa_decode_step(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), knst[0], vnst[0], k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), float(scale), out.data_ptr(), bsz, hq,
        hkv, d, bs, bts[1], nb, qst[0], _dtype_code(q.dtype), _dtype_code(out.dtype),
        ctypes.byref(opts), _stream_of(q)))
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float, out=None, *,
                  out_dtype=None):
    """Causal attention of each sequence's new tokens (q rows query_start[s]..query_start[s+1]-1,
    positions L-n..L-1) over its paged cache; returns out [num_tokens, Hq, D]."""
    import torch
    lib = load_library()
    _require_cuda(q, k_cache, v_cache, block_tables, context_lens, query_start)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    if q.dim() != 3 or q.shape[2] != d or q.stride(2) != 1 or q.stride(1) != d:
        raise ValueError(f"q must be [T, Hq, {d}] with contiguous head rows")
    t, hq = q.shape[0], q.shape[1]
    bsz = context_lens.shape[0]
    if q.dtype != k_cache.dtype:
        raise TypeError("q and the caches must share one dtype")
    for x, name in ((block_tables, "block_tables"), (context_lens, "context_lens"), (query_start, "query_start")):
        if x.dtype != torch.int32 or not x.is_contiguous():
            raise TypeError(f"{name} must be a contiguous int32 tensor")
    if block_tables.dim() != 2 or block_tables.shape[0] != bsz or query_start.shape != (bsz + 1,):
        raise ValueError("block_tables [B, MB], context_lens [B] and query_start [B+1] disagree")
    if out is None:
        odt = out_dtype if out_dtype is not None else q.dtype
        out = torch.empty((t, hq, d), dtype=odt, device=q.device)
    elif tuple(out.shape) != (t, hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, Hq, D] tensor")
    else:
        _require_cuda(q, out)
    _check(lib.pa_paged_prefill(q.data_ptr(), q.stride(0), k_cache.data_ptr(), v_cache.data_ptr(),
                                block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(),
                                float(scale), out.data_ptr(), bsz, t, hq, hkv, d, bs, block_tables.shape[1], nb,
                                _dtype_code(q.dtype), _dtype_code(out.dtype), _stream_of(q)))
    return out


def decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype_code,
                partition_size=0, num_cus=256, shared_prefix=False) -> dict:
    """Host-only launch plan (no device access when num_cus > 0)."""
    lib = load_library()
    waves = ctypes.c_int64()
    rng = ctypes.c_int32()
    red = ctypes.c_int32()
    win = ctypes.c_int32()
    ws = ctypes.c_size_t()
    opts = DecodeOpts()
    opts.partition_size = int(partition_size)
    opts.shared_prefix = 1 if shared_prefix else 0
    _check(lib.pa_decode_plan_ex(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                 dtype_code, ctypes.byref(opts), num_cus, ctypes.byref(waves), ctypes.byref(rng),
                                 ctypes.byref(red), ctypes.byref(win), ctypes.byref(ws)))
    return {"num_waves": waves.value, "range_tokens": rng.value, "uses_reduce": bool(red.value),
            "shared_prefix_window": win.value, "workspace_bytes": ws.value}


def workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype_code,
                    partition_size=0, shared_prefix=False) -> int:
    if shared_prefix:
        return decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype_code,
                           partition_size, 0, shared_prefix=True)["workspace_bytes"]
    return int(load_library().pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                       max_blocks_per_seq, dtype_code, partition_size))


def version() -> str:
    return load_library().pa_version().decode()


def shutdown() -> None:
    _check(load_library().pa_shutdown())


def copy_blocks(k_cache, v_cache, src, dst) -> None:
    """Bit-copy whole blocks src[i] -> dst[i] in both caches (copy-on-write); src/dst int32 CUDA tensors."""
    import torch
    lib = load_library()
    _require_cuda(k_cache, v_cache, src, dst)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.shape != dst.shape or src.dim() != 1:
        raise ValueError("src and dst must be 1-D int32 tensors of one length")
    src, dst = src.contiguous(), dst.contiguous()  # held until the launch is queued
    _check(lib.pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), src.data_ptr(),
                              dst.data_ptr(), src.shape[0], hkv, d, bs, nb,
                              _dtype_code(k_cache.dtype), _stream_of(k_cache)))


class BlockManager:
    """Prefix-caching KV block allocator (host C++; see pa_bm_* in pagedattn.h)."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = load_library()
        self.num_blocks, self.block_size = num_blocks, block_size
        self._m = self._lib.pa_bm_create(num_blocks, block_size)
        if not self._m:
            raise PagedAttnError(3, self._lib.pa_bm_last_error().decode())

    def _check(self, rc):
        if rc != 0:
            raise PagedAttnError(rc, self._lib.pa_bm_last_error().decode())

    def close(self):
        if self._m:
            self._lib.pa_bm_destroy(self._m)
            self._m = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq_id: int, tokens) -> int:
        """Allocate a prompt's blocks; returns the number of leading tokens already cached."""
        arr = (ctypes.c_int32 * max(1, len(tokens)))(*[int(t) for t in tokens])
        cached = ctypes.c_int32()
        self._check(self._lib.pa_bm_add_sequence(self._m, seq_id, arr, len(tokens), ctypes.byref(cached)))
        return cached.value

    def append_token(self, seq_id: int, token: int):
        """Slot for one new token, and the (src, dst) block copy to do first (or None)."""
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pa_bm_append_token(self._m, seq_id, int(token), ctypes.byref(slot),
                                                 ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, ((src.value, dst.value) if src.value >= 0 else None)

    def fork(self, parent_id: int, child_id: int) -> None:
        self._check(self._lib.pa_bm_fork(self._m, parent_id, child_id))

    def free_sequence(self, seq_id: int) -> None:
        self._check(self._lib.pa_bm_free_sequence(self._m, seq_id))

    def block_table(self, seq_id: int):
        n, t = ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pa_bm_block_table(self._m, seq_id, None, 0, ctypes.byref(n), ctypes.byref(t)))
        out = (ctypes.c_int32 * max(1, n.value))()
        self._check(self._lib.pa_bm_block_table(self._m, seq_id, out, n.value, None, None))
        return list(out[:n.value])

    def num_tokens(self, seq_id: int) -> int:
        n, t = ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pa_bm_block_table(self._m, seq_id, None, 0, ctypes.byref(n), ctypes.byref(t)))
        return t.value

    def slots(self, seq_id: int, first_token: int, count: int):
        out = (ctypes.c_int32 * max(1, count))()
        self._check(self._lib.pa_bm_slots(self._m, seq_id, first_token, count, out))
        return list(out[:count])

    def stats(self) -> dict:
        f, c = ctypes.c_int32(), ctypes.c_int32()
        h, m, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        self._check(self._lib.pa_bm_stats(self._m, ctypes.byref(f), ctypes.byref(c), ctypes.byref(h),
                                          ctypes.byref(m), ctypes.byref(e)))
        return {"free_blocks": f.value, "cached_blocks": c.value, "hits": h.value, "misses": m.value,
                "evictions": e.value}

    def block_ref(self, block: int) -> int:
        return self._lib.pa_bm_block_ref(self._m, block)
