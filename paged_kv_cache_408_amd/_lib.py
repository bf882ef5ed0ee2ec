"""ctypes binding of libpagedkv.so: the C ABI of include/pagedkv.h under the same names.

Argument marshalling only: tensors become (data pointer, sizes); the stream is torch's
current HIP stream; every step of the computation runs in the library's kernels.  Loading
fails loudly when the library has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_NO_BLOCKS, PA_ERR_DEVICE = 0, -1, -2, -3, -4
PA_DTYPE_F32, PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3, PA_DTYPE_MXFP4 = 0, 1, 2, 3

EXPORTED = [
    "pa_last_error", "pa_abi_version", "pa_kv_write", "pa_decode_workspace_bytes",
    "pa_decode_partition_tokens", "pa_decode_workspace_init", "pa_decode",
    "pa_copy_blocks", "pa_alloc_create", "pa_alloc_destroy", "pa_seq_add", "pa_seq_append",
    "pa_batch_append", "pa_seq_fork", "pa_seq_free", "pa_block_tables", "pa_alloc_stats",
    "pa_alloc_dump", "pa_alloc_set_host_blocks", "pa_swap_out", "pa_swap_in", "pa_seq_is_swapped",
    "pa_alloc_dump_host", "pa_swap_blocks", "pa_seq_add_prompt", "pa_seq_append_tokens", "pa_alloc_dump_cached",
    "pa_prefill", "pa_upload", "pa_probe_read", "pa_decode_noalloc", "pa_kv_write_t", "pa_decode_t", "pa_decode_append",
]


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class NoBlocksError(PagedKVError):
    """The allocator's free queue cannot cover the request (state unchanged)."""


class UnsupportedError(PagedKVError):
    pass


class pa_alloc_stats_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("free_blocks", "used_blocks", "total_refs", "exhaustion_events", "waste_slots", "num_seqs",
                 "host_free_blocks", "host_used_blocks", "swapped_seqs", "cached_blocks", "cache_hit_blocks",
                 "cache_evictions")]


class pa_tensor(ctypes.Structure):
    """Non-owning tensor view of include/pagedkv.h (shape and strides in elements)."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class pa_opts(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
                ("partition_tokens", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


PA_DTYPE_I32, PA_DTYPE_I64 = 4, 5

_lib = None


def load(path: str | None = None):
    """Load (once) and return the library handle; raises if it is missing.  `path` defaults to
    the module's LIB_PATH as it is when the library is first loaded."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_cache_408_amd._build` "
                          "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sig = {
        "pa_last_error": (ctypes.c_char_p, []),
        "pa_abi_version": (I32, []),
        "pa_kv_write": (ctypes.c_int, [P, P, P, I64, P, P, I64, I32, I32, I32, I32, I32, P, P, P]),
        "pa_decode_workspace_bytes": (I64, [I32, I32, I32, I32, I32, I32, I32, I32]),
        "pa_decode_partition_tokens": (I32, [I32, I32, I32, I32, I32, I32]),
        "pa_decode_workspace_init": (ctypes.c_int, [P, I64, P]),
        "pa_decode": (ctypes.c_int, [P, P, P, P, P, P, F32, I32, I32, I32, I32, I32, I64, I32, I32, I32, I32,
                                     P, P, P, I64, I32, P]),
        "pa_copy_blocks": (ctypes.c_int, [P, P, P, I32, I64, I32, I32, I32, I32, P]),
        "pa_alloc_create": (ctypes.c_int, [I32, I32, P, ctypes.POINTER(P)]),
        "pa_alloc_destroy": (None, [P]),
        "pa_seq_add": (ctypes.c_int, [P, I64]),
        "pa_seq_append": (ctypes.c_int, [P, I64, I32, P, P, P]),
        "pa_batch_append": (ctypes.c_int, [P, P, P, I32, P, P, P]),
        "pa_seq_fork": (ctypes.c_int, [P, I64, I64]),
        "pa_seq_free": (ctypes.c_int, [P, I64]),
        "pa_block_tables": (ctypes.c_int, [P, P, I32, I32, P, P]),
        "pa_alloc_stats": (ctypes.c_int, [P, ctypes.POINTER(pa_alloc_stats_t)]),
        "pa_alloc_dump": (ctypes.c_int, [P, P, P, P]),
        "pa_alloc_set_host_blocks": (ctypes.c_int, [P, I32]),
        "pa_swap_out": (ctypes.c_int, [P, P, I32, P, I32, P]),
        "pa_swap_in": (ctypes.c_int, [P, P, I32, P, I32, P]),
        "pa_seq_is_swapped": (ctypes.c_int, [P, I64]),
        "pa_alloc_dump_host": (ctypes.c_int, [P, P, P, P]),
        "pa_swap_blocks": (ctypes.c_int, [P, P, P, P, P, I32, I64, I64, I32, I32, I32, I32, P]),
        "pa_upload": (ctypes.c_int, [P, P, I64, P]),
        "pa_probe_read": (ctypes.c_int, [P, I64, I32, P, I64, P, I64, P]),
        "pa_decode_append": (ctypes.c_int, [P, P, P, P, P, P, P, P, F32, I32, I32, I32, I32, I32, I64, I32, I32, I32,
                                            I32, P, P, P, I64, I32, P]),
        "pa_kv_write_t": (ctypes.c_int, [ctypes.POINTER(pa_tensor)] * 5 + [ctypes.POINTER(pa_opts)]),
        "pa_decode_t": (ctypes.c_int, [ctypes.POINTER(pa_tensor)] * 6 + [F32, I32, ctypes.POINTER(pa_opts)]),
        "pa_decode_noalloc": (ctypes.c_int, [P, P, P, P, P, P, F32, I32, I32, I32, I32, I32, I64, I32, I32, I32,
                                             I32, P, P, I32, P]),
        "pa_seq_add_prompt": (ctypes.c_int, [P, I64, P, I32, P, P]),
        "pa_seq_append_tokens": (ctypes.c_int, [P, I64, P, I32, P, P, P]),
        "pa_alloc_dump_cached": (ctypes.c_int, [P, P]),
        "pa_prefill": (ctypes.c_int, [P, P, P, P, P, P, P, F32, I32, I32, I64, I32, I32, I32, I64, I32, I32, I32,
                                      I32, I32, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int):
    if rc == PA_OK:
        return
    msg = load().pa_last_error().decode()
    cls = NoBlocksError if rc == PA_ERR_NO_BLOCKS else UnsupportedError if rc == PA_ERR_UNSUPPORTED else PagedKVError
    raise cls(rc, msg)


# --------------------------------------------------------------------------- device ops

def _torch():
    import torch
    return torch


def _dtype_code(t, what):
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return PA_DTYPE_FP8_E4M3
    raise TypeError(f"{what}: unsupported dtype {t.dtype}")


def mx_row_bytes(head_dim: int) -> int:
    """Bytes per token row of an MXFP4 cache: head_dim / 2 of codes + head_dim / 32 of scales."""
    return head_dim // 2 + head_dim // 32


def mxfp4_cache(num_blocks, num_kv_heads, block_size, head_dim, device="cuda"):
    """A zeroed MXFP4 cache: uint8 [num_blocks, num_kv_heads, block_size, head_dim * 17 / 32]
    whose (block, head) tile holds the codes [block_size, head_dim / 2] and then the scales
    [block_size, head_dim / 32] (not interleaved per row: the last two dims only size it)."""
    torch = _torch()
    return torch.zeros((num_blocks, num_kv_heads, block_size, mx_row_bytes(head_dim)), dtype=torch.uint8,
                       device=device)


def _cache_geom(cache, what):
    """(num_blocks, num_kv_heads, block_size, head_dim, cache dtype code) of a cache tensor
    [N, Hkv, bs, head_dim] (f32 / bf16 / fp8 as uint8 or float8_e4m3fn) or an MXFP4 cache
    (uint8, last dim head_dim * 17 / 32: 34 or 68)."""
    torch = _torch()
    N, H, bs, last = cache.shape
    if cache.dtype == torch.uint8 and last in (mx_row_bytes(64), mx_row_bytes(128)):
        return N, H, bs, last * 32 // 17, PA_DTYPE_MXFP4
    return N, H, bs, last, _dtype_code(cache, what)


def _dev(t, what):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def pa_kv_write(k, v, slot_mapping, k_cache, v_cache, *, k_scale=None, v_scale=None, stream=None,
                validate=False):
    """Write new tokens' K/V rows (k, v: [T, Hkv, d]) into caches [N, Hkv, bs, d] at the
    int64 slots in slot_mapping (< 0 = skip)."""
    torch = _torch()
    T, H, d = k.shape
    N, Hc, bs, dc, cdt = _cache_geom(k_cache, "k_cache")
    if v.shape != k.shape or v_cache.shape != k_cache.shape or (Hc, dc) != (H, d):
        raise ValueError(f"shape mismatch: k {tuple(k.shape)} v {tuple(v.shape)} caches {tuple(k_cache.shape)}")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    if validate:
        s = slot_mapping.cpu().numpy()
        live = s[s >= 0]
        if live.size and (live.max() >= N * bs or len(np.unique(live)) != live.size):
            raise ValueError("slot_mapping holds out-of-range or duplicate slots")
    rc = load().pa_kv_write(_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping"), T,
                            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), N, H, d, bs,
                            _dtype_code(k, "k"), cdt,
                            _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _stream(stream))
    _check(rc)


def _code(cache_dtype):
    """A cache dtype code, or the code of a cache tensor (see _cache_geom)."""
    return cache_dtype if isinstance(cache_dtype, int) else _cache_geom(cache_dtype, "cache")[4]


def pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_tokens=0,
                              block_size=16, cache_dtype=PA_DTYPE_BF16) -> int:
    """cache_dtype: a PA_DTYPE_* code or the cache tensor itself."""
    n = load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                         partition_tokens, block_size, _code(cache_dtype))
    if n < 0:
        _check(int(n))
    return int(n)


def pa_decode_partition_tokens(num_seqs, num_kv_heads, max_seq_len, partition_tokens=0, block_size=16,
                               cache_dtype=PA_DTYPE_BF16) -> int:
    """Partition size (tokens) pa_decode uses for these sizes and cache type (a PA_DTYPE_*
    code or the cache tensor) on the current device."""
    n = load().pa_decode_partition_tokens(num_seqs, num_kv_heads, max_seq_len, partition_tokens, block_size,
                                          _code(cache_dtype))
    if n < 0:
        _check(int(n))
    return int(n)


def pa_decode_workspace_init(workspace, *, stream=None):
    """Zero a decode workspace (uint8 device tensor) on the stream."""
    rc = load().pa_decode_workspace_init(_dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                         _stream(stream))
    _check(rc)


def decode_workspace(nbytes, device, layout_key, *, stream=None):
    """A workspace of at least nbytes kept per device and grown on demand.  It is zeroed
    whenever the call's sizes (layout_key) differ from the previous call's, as the ticket
    counters require; callers using it on several streams at once must bring their own."""
    torch = _torch()
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    ws, last = _WORKSPACES.get(key, (None, None))
    if ws is None or ws.numel() < nbytes:
        n = (max(int(nbytes), 16) + 255) // 256 * 256
        ws, last = torch.empty(n, dtype=torch.uint8, device=device), None
    if last != layout_key:
        pa_decode_workspace_init(ws, stream=stream)
    _WORKSPACES[key] = (ws, layout_key)
    return ws


_WORKSPACES = {}


def pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale, block_size, *, max_seq_len=None,
              k_scale=None, v_scale=None, workspace=None, partition_tokens=0, stream=None, validate=False):
    """Decode attention: out[b, h] = softmax(scale * q[b, h] . K_b^T) . V_b through the block
    table.  q, out: [B, Hq, d]; caches [N, Hkv, bs, d]; block_tables int32 [B, max_blocks];
    seq_lens int32 [B].  max_seq_len defaults to the table capacity (no device sync).
    partition_tokens 0 lets the library choose the split-K partition size.  A zeroed
    workspace kept per device is used when none is given (it must not be shared by calls in
    flight on different streams); workspace=False runs every request as a single
    partition."""
    torch = _torch()
    B, Hq, d = q.shape
    N, Hkv, bs, dc, cdt = _cache_geom(k_cache, "k_cache")
    if out.shape != q.shape or v_cache.shape != k_cache.shape or dc != d or bs != block_size:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} out {tuple(out.shape)} cache {tuple(k_cache.shape)} "
                         f"block_size {block_size}")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [num_seqs]")
    max_blocks = block_tables.shape[1]
    if max_seq_len is None:
        max_seq_len = max_blocks * block_size
    if validate:
        lens = seq_lens.cpu().numpy()
        tab = block_tables.cpu().numpy()
        if lens.size and (lens.min() < 0 or lens.max() > max_seq_len):
            raise ValueError("seq_lens outside [0, max_seq_len]")
        for b, L in enumerate(lens):
            live = tab[b, : -(-int(L) // block_size)]
            if live.size and (live.min() < 0 or live.max() >= N):
                raise ValueError(f"block table row {b} holds an id outside [0, {N})")
    if workspace is None:
        nbytes = pa_decode_workspace_bytes(B, Hq, Hkv, d, max_seq_len, partition_tokens, block_size, cdt)
        key = (B, Hq, Hkv, d, int(max_seq_len), int(partition_tokens), block_size, cdt)
        workspace = decode_workspace(nbytes, q.device, key, stream=stream) if nbytes > 0 else None
    elif workspace is False:          # explicitly none: one partition per request
        workspace = None
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().pa_decode(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                          _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), float(scale),
                          block_size, B, Hq, Hkv, d, N, max_blocks, int(max_seq_len),
                          _dtype_code(q, "q"), cdt,
                          _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), ws_ptr, ws_bytes,
                          int(partition_tokens), _stream(stream))
    _check(rc)


def pa_decode_append(out, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, scale, block_size, *,
                     max_seq_len=None, k_scale=None, v_scale=None, workspace=None, partition_tokens=0, stream=None):
    """One launch: each request's new token (k_new, v_new: [B, Hkv, d], q's dtype) written at its
    position seq_lens[b] - 1 through the table, then the decode of pa_decode (see
    pa_decode_append in include/pagedkv.h).  The caches are modified."""
    torch = _torch()
    B, Hq, d = q.shape
    N, Hkv, bs, dc, cdt = _cache_geom(k_cache, "k_cache")
    if out.shape != q.shape or v_cache.shape != k_cache.shape or dc != d or bs != block_size:
        raise ValueError("shape mismatch")
    if k_new.shape != (B, Hkv, d) or v_new.shape != k_new.shape or k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise ValueError(f"k_new, v_new must be [{B}, {Hkv}, {d}] of q's dtype")
    max_blocks = block_tables.shape[1]
    if max_seq_len is None:
        max_seq_len = max_blocks * block_size
    if workspace is None:
        nbytes = pa_decode_workspace_bytes(B, Hq, Hkv, d, max_seq_len, partition_tokens, block_size, cdt)
        key = (B, Hq, Hkv, d, int(max_seq_len), int(partition_tokens), block_size, cdt)
        workspace = decode_workspace(nbytes, q.device, key, stream=stream) if nbytes > 0 else None
    elif workspace is False:
        workspace = None
    rc = load().pa_decode_append(_dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                 _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                                 _dev(seq_lens, "seq_lens"), float(scale), block_size, B, Hq, Hkv, d, N, max_blocks,
                                 int(max_seq_len), _dtype_code(q, "q"), cdt, _dev(k_scale, "k_scale"),
                                 _dev(v_scale, "v_scale"), _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                 int(partition_tokens), _stream(stream))
    _check(rc)


class PreparedDecodeAppend:
    """pa_decode_append with its arguments marshalled once (see PreparedDecode)."""

    def __init__(self, out, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, scale, block_size, *,
                 max_seq_len, workspace, k_scale=None, v_scale=None, partition_tokens=0, stream=None):
        B, Hq, d = q.shape
        N, Hkv, bs, dc, cdt = _cache_geom(k_cache, "k_cache")
        if out.shape != q.shape or v_cache.shape != k_cache.shape or dc != d or bs != block_size or \
                k_new.shape != (B, Hkv, d) or v_new.shape != k_new.shape:
            raise ValueError("shape mismatch")
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        self._keep = (out, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, workspace, k_scale, v_scale)
        self._args = (_dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                      _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                      _dev(seq_lens, "seq_lens"), ctypes.c_float(scale), block_size, B, Hq, Hkv, d, N,
                      block_tables.shape[1], int(max_seq_len), _dtype_code(q, "q"), cdt, _dev(k_scale, "k_scale"),
                      _dev(v_scale, "v_scale"), _dev(workspace, "workspace"), ws_bytes, int(partition_tokens),
                      _stream(stream))
        self._fn = load().pa_decode_append

    def __call__(self):
        rc = self._fn(*self._args)
        if rc:
            _check(rc)


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, scale, block_size, *, max_seq_len=None,
                      k_scale=None, v_scale=None, partition_tokens=0, stream=None):
    """pa_decode with the library's fixed device scratch instead of a workspace, for callers that
    cannot allocate (see pa_decode_noalloc in include/pagedkv.h): same arguments and results
    as pa_decode without `workspace`; calls that overlap on one device race on the scratch."""
    B, Hq, d = q.shape
    N, Hkv, bs, dc, cdt = _cache_geom(k_cache, "k_cache")
    if out.shape != q.shape or v_cache.shape != k_cache.shape or dc != d or bs != block_size:
        raise ValueError("shape mismatch")
    max_blocks = block_tables.shape[1]
    if max_seq_len is None:
        max_seq_len = max_blocks * block_size
    rc = load().pa_decode_noalloc(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                  _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), float(scale),
                                  block_size, B, Hq, Hkv, d, N, max_blocks, int(max_seq_len), _dtype_code(q, "q"), cdt,
                                  _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), int(partition_tokens),
                                  _stream(stream))
    _check(rc)


def pa_prefill(out, q, k_cache, v_cache, block_tables, seq_lens, query_start, scale, block_size, *,
               max_query_len=None, max_seq_len=None, k_scale=None, v_scale=None, stream=None):
    """Causal attention of each request's new tokens (q rows query_start[b]..query_start[b+1]-1,
    the request's last tokens, K/V already written) over its cached tokens; see pa_prefill in
    include/pagedkv.h.  The cache may be bf16, fp8 (k_scale / v_scale: float32 [num_kv_heads])
    or MXFP4.  max_query_len / max_seq_len default to the values read from the device tensors
    (a synchronising copy)."""
    T, Hq, d = q.shape
    N, Hkv, bs, _, cdt = _cache_geom(k_cache, "k_cache")
    B = seq_lens.shape[0]
    if query_start.shape[0] != B + 1:
        raise ValueError("query_start must hold num_seqs + 1 entries")
    if max_query_len is None:
        qs = query_start.cpu()
        max_query_len = int((qs[1:] - qs[:-1]).max()) if B else 0
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max()) if B else 0
    rc = load().pa_prefill(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"),
                           _dev(query_start, "query_start"), float(scale), int(block_size), B, T, Hq, Hkv, d, N,
                           block_tables.shape[1], int(max_query_len), int(max_seq_len),
                           _dtype_code(q, "q"), cdt, _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
                           _stream(stream))
    _check(rc)


PA_PROBE_GRID, PA_PROBE_RANGES, PA_PROBE_TILES = 0, 1, 2


def pa_probe_read(src, sink, *, pattern=PA_PROBE_GRID, tile_order=None, stream=None):
    """A plain streaming read of a contiguous device tensor in one of three patterns (see
    pa_probe_read in include/pagedkv.h): the references the decode's HBM rate is compared with."""
    nbytes = src.numel() * src.element_size()
    n_order = tile_order.numel() if tile_order is not None else 0
    rc = load().pa_probe_read(_dev(src, "src"), nbytes, int(pattern), _dev(tile_order, "tile_order"), n_order,
                              _dev(sink, "sink"), sink.numel() * sink.element_size(), _stream(stream))
    if rc:
        _check(rc)


def pa_upload(dst, src, *, stream=None):
    """Copy src (a pinned host tensor or a device tensor) into the device tensor dst, byte for
    byte, with one kernel on the stream (see pa_upload in include/pagedkv.h): a step's packed
    block-table rows, lengths and slots, with no copy engine involved.  src must stay unchanged
    until the stream has passed the call."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError(f"pa_upload: {nbytes} source bytes into a {dst.numel() * dst.element_size()}-byte destination")
    if not src.is_contiguous() or not (src.is_cuda or src.is_pinned()):
        raise ValueError("pa_upload: src must be a contiguous pinned host or device tensor")
    rc = load().pa_upload(_dev(dst, "dst"), ctypes.c_void_p(src.data_ptr()), nbytes, _stream(stream))
    _check(rc)


def tensor_view(t, dtype=None):
    """A pa_tensor view of a device tensor (dtype code from the tensor unless given; an MXFP4 cache
    is viewed with its logical head_dim and zero strides)."""
    torch = _torch()
    v = pa_tensor()
    v.data = t.data_ptr()
    if dtype is None:
        if t.dtype == torch.int32:
            dtype = PA_DTYPE_I32
        elif t.dtype == torch.int64:
            dtype = PA_DTYPE_I64
        elif t.dim() == 4:
            dtype = _cache_geom(t, "cache")[4]
        else:
            dtype = _dtype_code(t, "tensor")
    v.dtype, v.ndim = dtype, t.dim()
    shape = list(t.shape)
    if dtype == PA_DTYPE_MXFP4:
        shape[3] = _cache_geom(t, "cache")[3]
        strides = [0] * t.dim()
    else:
        strides = list(t.stride())
    for i in range(t.dim()):
        v.shape[i], v.stride[i] = shape[i], strides[i]
    return v


def pa_copy_blocks(k_cache, v_cache, src_dst, *, stream=None):
    """Copy whole blocks src -> dst (int64 [n, 2] device tensor) in both caches."""
    torch = _torch()
    N, Hkv, bs, d, cdt = _cache_geom(k_cache, "k_cache")
    if src_dst.dtype != torch.int64 or src_dst.dim() != 2 or src_dst.shape[1] != 2:
        raise ValueError("src_dst must be int64 [n, 2]")
    rc = load().pa_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(src_dst, "src_dst"),
                               src_dst.shape[0], N, Hkv, d, bs, cdt, _stream(stream))
    _check(rc)


def _dev_or_pinned(t, what):
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{what} must be a device tensor or a pinned host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def pa_swap_blocks(dst_k, dst_v, src_k, src_v, src_dst, *, stream=None):
    """Copy whole blocks src_k[s] -> dst_k[d] (and v) for each row (s, d) of src_dst (int64
    [n, 2]); each pool is a device tensor or a pinned host tensor of the cache layout."""
    torch = _torch()
    Ns, Hkv, bs, d, cdt = _cache_geom(src_k, "src_k")
    Nd = dst_k.shape[0]
    for t, n in ((dst_k, "dst_k"), (dst_v, "dst_v"), (src_v, "src_v")):
        if t.shape[1:] != src_k.shape[1:] or t.dtype != src_k.dtype:
            raise ValueError(f"{n} does not match src_k's block shape and dtype")
    if dst_v.shape[0] != Nd or src_v.shape[0] != Ns:
        raise ValueError("k and v pools differ in block count")
    if src_dst.dtype != torch.int64 or src_dst.dim() != 2 or src_dst.shape[1] != 2:
        raise ValueError("src_dst must be int64 [n, 2]")
    rc = load().pa_swap_blocks(_dev_or_pinned(dst_k, "dst_k"), _dev_or_pinned(dst_v, "dst_v"),
                               _dev_or_pinned(src_k, "src_k"), _dev_or_pinned(src_v, "src_v"),
                               _dev_or_pinned(src_dst, "src_dst"), src_dst.shape[0], Ns, Nd, Hkv, d, bs,
                               cdt, _stream(stream))
    _check(rc)


# --------------------------------------------------------------------------- host allocator

def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def pa_alloc_create(num_blocks, block_size, initial_free_order=None):
    h = ctypes.c_void_p()
    order = None
    if initial_free_order is not None:
        order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
    _check(load().pa_alloc_create(num_blocks, block_size, _p(order) if order is not None else None,
                                  ctypes.byref(h)))
    return h


def pa_alloc_destroy(h):
    load().pa_alloc_destroy(h)


def pa_seq_add(h, seq_id):
    _check(load().pa_seq_add(h, seq_id))


def pa_seq_append(h, seq_id, n_tokens):
    slots = np.empty(max(n_tokens, 1), dtype=np.int64)
    cow = np.empty(2, dtype=np.int64)
    ncow = np.zeros(1, dtype=np.int32)
    _check(load().pa_seq_append(h, seq_id, n_tokens, _p(slots), _p(cow), _p(ncow)))
    return slots[:n_tokens], [(int(cow[0]), int(cow[1]))] if ncow[0] else []


def pa_seq_append_tokens(h, seq_id, token_ids):
    toks = np.ascontiguousarray(token_ids, dtype=np.int32)
    n = len(toks)
    slots = np.empty(max(n, 1), dtype=np.int64)
    cow = np.empty(2, dtype=np.int64)
    ncow = np.zeros(1, dtype=np.int32)
    _check(load().pa_seq_append_tokens(h, seq_id, _p(toks), n, _p(slots), _p(cow), _p(ncow)))
    return slots[:n], [(int(cow[0]), int(cow[1]))] if ncow[0] else []


def pa_seq_add_prompt(h, seq_id, token_ids):
    """Returns (tokens found in the prefix cache, slots of the remaining tokens)."""
    toks = np.ascontiguousarray(token_ids, dtype=np.int32)
    slots = np.empty(max(len(toks), 1), dtype=np.int64)
    nc = np.zeros(1, dtype=np.int32)
    _check(load().pa_seq_add_prompt(h, seq_id, _p(toks), len(toks), _p(nc), _p(slots)))
    return int(nc[0]), slots[: len(toks) - int(nc[0])]


def pa_alloc_dump_cached(h, num_blocks):
    reg = np.empty(num_blocks, dtype=np.int32)
    _check(load().pa_alloc_dump_cached(h, _p(reg)))
    return reg


def pa_batch_append(h, seq_ids, n_tokens):
    ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    nt = np.ascontiguousarray(n_tokens, dtype=np.int32)
    slots = np.empty(max(int(nt.sum()), 1), dtype=np.int64)
    cow = np.empty(max(2 * len(ids), 2), dtype=np.int64)
    ncow = np.zeros(1, dtype=np.int32)
    _check(load().pa_batch_append(h, _p(ids), _p(nt), len(ids), _p(slots), _p(cow), _p(ncow)))
    return slots[: int(nt.sum())], [(int(cow[2 * i]), int(cow[2 * i + 1])) for i in range(int(ncow[0]))]


def pa_seq_fork(h, parent, child):
    _check(load().pa_seq_fork(h, parent, child))


def pa_seq_free(h, seq_id):
    _check(load().pa_seq_free(h, seq_id))


def pa_block_tables(h, seq_ids, max_blocks, tables_out=None, seq_lens_out=None):
    ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    tab = tables_out if tables_out is not None else np.empty((len(ids), max_blocks), dtype=np.int32)
    lens = seq_lens_out if seq_lens_out is not None else np.empty(len(ids), dtype=np.int32)
    assert tab.dtype == np.int32 and tab.flags.c_contiguous and tab.shape == (len(ids), max_blocks)
    assert lens.dtype == np.int32 and lens.shape == (len(ids),)
    _check(load().pa_block_tables(h, _p(ids), len(ids), max_blocks, _p(tab), _p(lens)))
    return tab, lens


def pa_alloc_stats(h) -> dict:
    st = pa_alloc_stats_t()
    _check(load().pa_alloc_stats(h, ctypes.byref(st)))
    return {n: int(getattr(st, n)) for n, _ in pa_alloc_stats_t._fields_}


def pa_alloc_dump(h, num_blocks):
    ref = np.empty(num_blocks, dtype=np.int32)
    free = np.empty(num_blocks, dtype=np.int32)
    nf = np.zeros(1, dtype=np.int32)
    _check(load().pa_alloc_dump(h, _p(ref), _p(free), _p(nf)))
    return ref, free[: int(nf[0])]


def pa_alloc_set_host_blocks(h, num_host_blocks):
    _check(load().pa_alloc_set_host_blocks(h, num_host_blocks))


def _swap(fn, h, seq_ids, max_pairs):
    ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    pairs = np.empty((max(max_pairs, 1), 2), dtype=np.int64)
    n = np.zeros(1, dtype=np.int32)
    _check(fn(h, _p(ids), len(ids), _p(pairs), max_pairs, _p(n)))
    return pairs[: int(n[0])].copy()


def pa_swap_out(h, seq_ids, max_pairs):
    """Returns the (device block, host block) pairs to copy, int64 [n, 2]."""
    return _swap(load().pa_swap_out, h, seq_ids, max_pairs)


def pa_swap_in(h, seq_ids, max_pairs):
    """Returns the (host block, device block) pairs to copy, int64 [n, 2]."""
    return _swap(load().pa_swap_in, h, seq_ids, max_pairs)


def pa_seq_is_swapped(h, seq_id) -> bool:
    rc = load().pa_seq_is_swapped(h, seq_id)
    if rc < 0:
        _check(rc)
    return rc == 1


def pa_alloc_dump_host(h, num_host_blocks):
    ref = np.empty(max(num_host_blocks, 1), dtype=np.int32)
    free = np.empty(max(num_host_blocks, 1), dtype=np.int32)
    nf = np.zeros(1, dtype=np.int32)
    _check(load().pa_alloc_dump_host(h, _p(ref), _p(free), _p(nf)))
    return ref[:num_host_blocks], free[: int(nf[0])]


class Allocator:
    """Owning wrapper of a pa_allocator handle (host only)."""

    def __init__(self, num_blocks, block_size, initial_free_order=None):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self._h = pa_alloc_create(self.num_blocks, self.block_size, initial_free_order)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h is not None and _lib is not None:
            pa_alloc_destroy(h)

    def add(self, seq_id):
        pa_seq_add(self._h, seq_id)

    def append(self, seq_id, n_tokens, token_ids=None):
        if token_ids is not None:
            if len(token_ids) != n_tokens:
                raise ValueError("token_ids must hold n_tokens ids")
            return pa_seq_append_tokens(self._h, seq_id, token_ids)
        return pa_seq_append(self._h, seq_id, n_tokens)

    def add_prompt(self, seq_id, token_ids):
        return pa_seq_add_prompt(self._h, seq_id, token_ids)

    def dump_cached(self):
        return pa_alloc_dump_cached(self._h, self.num_blocks)

    def batch_append(self, seq_ids, n_tokens):
        return pa_batch_append(self._h, seq_ids, n_tokens)

    def fork(self, parent, child):
        pa_seq_fork(self._h, parent, child)

    def free(self, seq_id):
        pa_seq_free(self._h, seq_id)

    def block_tables(self, seq_ids, max_blocks, tables_out=None, seq_lens_out=None):
        return pa_block_tables(self._h, seq_ids, max_blocks, tables_out, seq_lens_out)

    def stats(self):
        return pa_alloc_stats(self._h)

    def dump(self):
        return pa_alloc_dump(self._h, self.num_blocks)

    def set_host_blocks(self, num_host_blocks):
        pa_alloc_set_host_blocks(self._h, num_host_blocks)
        self.num_host_blocks = int(num_host_blocks)

    def swap_out(self, seq_ids):   # at most one pair per device block
        return pa_swap_out(self._h, seq_ids, self.num_blocks)

    def swap_in(self, seq_ids):    # at most one pair per host block
        return pa_swap_in(self._h, seq_ids, getattr(self, "num_host_blocks", 0))

    def is_swapped(self, seq_id):
        return pa_seq_is_swapped(self._h, seq_id)

    def dump_host(self):
        return pa_alloc_dump_host(self._h, getattr(self, "num_host_blocks", 0))


def blocks_for(seq_lens, block_size) -> int:
    return int(sum(math.ceil(int(L) / block_size) for L in seq_lens))


# --------------------------------------------------------------------------- prepared calls

class PreparedDecode:
    """pa_decode with its arguments checked and marshalled once; calling it enqueues the
    kernel with the same buffers (their contents may change between calls).  For loops
    where per-call Python overhead would otherwise show next to a ~50 us kernel."""

    def __init__(self, out, q, k_cache, v_cache, block_tables, seq_lens, scale, block_size, *, max_seq_len,
                 workspace, k_scale=None, v_scale=None, partition_tokens=0, stream=None):
        B, Hq, d = q.shape
        N, Hkv, bs, dc, cdt = _cache_geom(k_cache, "k_cache")
        if out.shape != q.shape or v_cache.shape != k_cache.shape or dc != d or bs != block_size:
            raise ValueError("shape mismatch")
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        self._keep = (out, q, k_cache, v_cache, block_tables, seq_lens, workspace, k_scale, v_scale)
        self._args = (_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                      _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), ctypes.c_float(scale),
                      block_size, B, Hq, Hkv, d, N, block_tables.shape[1], int(max_seq_len),
                      _dtype_code(q, "q"), cdt, _dev(k_scale, "k_scale"),
                      _dev(v_scale, "v_scale"), _dev(workspace, "workspace"), ws_bytes, int(partition_tokens),
                      _stream(stream))
        self._fn = load().pa_decode

    def __call__(self):
        rc = self._fn(*self._args)
        if rc:
            _check(rc)


class PreparedKVWrite:
    """pa_kv_write with its arguments marshalled once (see PreparedDecode)."""

    def __init__(self, k, v, slot_mapping, k_cache, v_cache, *, k_scale=None, v_scale=None, stream=None):
        T, H, d = k.shape
        N, Hc, bs, dc, cdt = _cache_geom(k_cache, "k_cache")
        if v.shape != k.shape or v_cache.shape != k_cache.shape or (Hc, dc) != (H, d) or slot_mapping.shape != (T,):
            raise ValueError("shape mismatch")
        self._keep = (k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale)
        self._args = (_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping"), T, _dev(k_cache, "k_cache"),
                      _dev(v_cache, "v_cache"), N, H, d, bs, _dtype_code(k, "k"), cdt,
                      _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _stream(stream))
        self._fn = load().pa_kv_write

    def __call__(self):
        rc = self._fn(*self._args)
        if rc:
            _check(rc)
