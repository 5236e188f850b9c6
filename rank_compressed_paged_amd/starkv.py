"""Thin ctypes binding over libstarkv (declared in include/starkv.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI.  Tensors are torch tensors on the GPU; this module
checks dtype, shape, contiguity and device, then passes ``data_ptr()`` and
the current HIP stream.  Importing it raises if the library is missing, and
nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("STARKV_LIB", os.path.join(_HERE, "libstarkv.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libstarkv.so not found at {LIB_PATH}; build it with "
        "`python -m rank_compressed_paged_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

STATUS = {
    0: "STARKV_OK", 1: "STARKV_ERR_NULL", 2: "STARKV_ERR_DIMS", 3: "STARKV_ERR_UNSUPPORTED",
    4: "STARKV_ERR_WORKSPACE", 5: "STARKV_ERR_ALIGN", 6: "STARKV_ERR_LAUNCH", 7: "STARKV_ERR_ARG",
}
EXPORTED = [
    "starkv_abi_version", "starkv_status_string", "starkv_shape_supported", "starkv_append",
    "starkv_append_workspace_size",
    "starkv_decode_workspace_size", "starkv_decode_attn", "starkv_prefill_workspace_size",
    "starkv_prefill_attn", "starkv_set_timing_events", "starkv_decode_plan",
    "starkv_util_stream_read", "starkv_util_event_create", "starkv_util_event_destroy",
    "starkv_util_event_elapsed_ms", "starkv_fit_workspace_size", "starkv_fit_bases",
    "starkv_append_fp8", "starkv_decode_attn_fp8", "starkv_prefill_attn_fp8",
    "starkv_decode_workspace_size_cfg", "starkv_decode_attn_cfg", "starkv_decode_attn_noalloc",
    "starkv_check_indices",
]
NOALLOC_SCRATCH_BYTES = 32 << 20


class Dims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rank_k", ctypes.c_int32), ("rank_v", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32)]


class DecodeConfig(ctypes.Structure):
    _fields_ = [("pages_per_split", ctypes.c_int32), ("merge_seqs", ctypes.c_int32),
                ("launches", ctypes.c_int32)]


class StarKVError(RuntimeError):
    def __init__(self, status, where):
        self.status = int(status)
        msg = _lib.starkv_status_string(int(status)).decode()
        super().__init__(f"{where}: {STATUS.get(int(status), status)} ({msg})")


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_lib.starkv_abi_version.restype = _i32
_lib.starkv_abi_version.argtypes = []
_lib.starkv_status_string.restype = ctypes.c_char_p
_lib.starkv_status_string.argtypes = [_i32]
_lib.starkv_shape_supported.restype = _i32
_lib.starkv_shape_supported.argtypes = [ctypes.POINTER(Dims)]
_lib.starkv_append.restype = _i32
_lib.starkv_append.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                               _sz, _vp]
_lib.starkv_append_workspace_size.restype = _i32
_lib.starkv_append_workspace_size.argtypes = [ctypes.POINTER(Dims), _i32, ctypes.POINTER(_sz)]
_lib.starkv_decode_workspace_size.restype = _i32
_lib.starkv_decode_workspace_size.argtypes = [ctypes.POINTER(Dims), _i32, _i32, ctypes.POINTER(_sz)]
_lib.starkv_decode_plan.restype = _i32
_lib.starkv_decode_plan.argtypes = [ctypes.POINTER(Dims), _i32, _i32, ctypes.POINTER(_i32),
                                    ctypes.POINTER(_i32)]
_lib.starkv_decode_attn.restype = _i32
_lib.starkv_decode_attn.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                    _i32, _i32, ctypes.c_float, _vp, _vp, _sz, _vp]
_lib.starkv_decode_workspace_size_cfg.restype = _i32
_lib.starkv_decode_workspace_size_cfg.argtypes = [ctypes.POINTER(Dims), _i32, _i32,
                                                  ctypes.POINTER(DecodeConfig), ctypes.POINTER(_sz)]
_lib.starkv_decode_attn_cfg.restype = _i32
_lib.starkv_decode_attn_cfg.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                        _vp, _i32, _i32, ctypes.c_float,
                                        ctypes.POINTER(DecodeConfig), _vp, _vp, _sz, _vp]
_lib.starkv_decode_attn_noalloc.restype = _i32
_lib.starkv_decode_attn_noalloc.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _vp, _vp, _vp, _vp,
                                            _i32, _vp, _i32, _i32, ctypes.c_float, _vp, _vp]
_lib.starkv_prefill_workspace_size.restype = _i32
_lib.starkv_prefill_workspace_size.argtypes = [ctypes.POINTER(Dims), _i32, _i32, _i32,
                                               ctypes.POINTER(_sz)]
_lib.starkv_prefill_attn.restype = _i32
_lib.starkv_prefill_attn.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                     _vp, _vp, _i32, _vp, _i32, _i32, ctypes.c_float, _vp, _vp,
                                     _sz, _vp]
_lib.starkv_check_indices.restype = _i32
_lib.starkv_check_indices.argtypes = [ctypes.POINTER(Dims), _vp, _i32, _vp, _i32, _i32, _vp, _i32,
                                      _vp, _vp]
_lib.starkv_util_stream_read.restype = _i32
_lib.starkv_util_stream_read.argtypes = [_vp, _sz, _vp, _vp]
_lib.starkv_util_event_create.restype = _i32
_lib.starkv_util_event_create.argtypes = [ctypes.POINTER(_vp)]
_lib.starkv_util_event_destroy.restype = _i32
_lib.starkv_util_event_destroy.argtypes = [_vp]
_lib.starkv_util_event_elapsed_ms.restype = _i32
_lib.starkv_util_event_elapsed_ms.argtypes = [_vp, _vp, ctypes.POINTER(ctypes.c_float)]
_lib.starkv_fit_workspace_size.restype = _i32
_lib.starkv_fit_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(_sz)]
_lib.starkv_fit_bases.restype = _i32
_lib.starkv_fit_bases.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp,
                                  _vp, _sz, _vp, _vp, _vp]
_f32 = ctypes.c_float
_lib.starkv_append_fp8.restype = _i32
_lib.starkv_append_fp8.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _vp, _vp, _vp, _i32, _f32, _f32,
                                   _vp, _vp, _vp, _sz, _vp]
_lib.starkv_decode_attn_fp8.restype = _i32
_lib.starkv_decode_attn_fp8.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                        _vp, _i32, _i32, _f32, _f32, _f32, _vp, _vp, _sz, _vp]
_lib.starkv_prefill_attn_fp8.restype = _i32
_lib.starkv_prefill_attn_fp8.argtypes = [ctypes.POINTER(Dims), _vp, _vp, _i32, _i32, _vp, _vp,
                                         _vp, _vp, _vp, _i32, _vp, _i32, _i32, _f32, _f32, _f32,
                                         _vp, _vp, _sz, _vp]
_lib.starkv_set_timing_events.restype = _i32
_lib.starkv_set_timing_events.argtypes = [_vp, _vp, _i32]

TIME_NONE, TIME_DECODE_SPLIT, TIME_PREFILL_ATTN, TIME_APPEND, TIME_FIT_GRAM, TIME_STREAM_READ = \
    0, 1, 2, 3, 4, 5


def lib():
    return _lib


def abi_version():
    return _lib.starkv_abi_version()


def _check(status, where):
    if status != 0:
        raise StarKVError(status, where)


def make_dims(H, d, r_k, r_v, num_blocks, block_size=16, num_kv_heads=0):
    return Dims(H, d, r_k, r_v, block_size, num_blocks, num_kv_heads)


def dims_of(k_cache, v_cache, U, W, num_heads=None):
    """Dims of a cache; num_heads = query heads (default: the cache's key/value
    heads, i.e. multi-head attention)."""
    NB, Hkv, bs, r_k = k_cache.shape
    d = U.shape[1]
    r_v = v_cache.shape[1]
    H = Hkv if num_heads is None else int(num_heads)
    return make_dims(H, d, r_k, r_v, NB, bs, 0 if H == Hkv else Hkv)


def shape_supported(dims):
    return bool(_lib.starkv_shape_supported(ctypes.byref(dims)))


def _dev(t, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return _vp(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _config(pages_per_split, merge_seqs, launches=0):
    """Plan override, or None for the library's plan."""
    if not pages_per_split and not merge_seqs and not launches:
        return None
    return DecodeConfig(int(pages_per_split or 0), int(merge_seqs or 0), int(launches or 0))


def decode_workspace_size(dims, batch, max_seq_len, pages_per_split=0, merge_seqs=0, launches=0):
    out = _sz(0)
    cfg = _config(pages_per_split, merge_seqs, launches)
    if cfg is None:
        _check(_lib.starkv_decode_workspace_size(ctypes.byref(dims), int(batch), int(max_seq_len),
                                                 ctypes.byref(out)), "starkv_decode_workspace_size")
    else:
        _check(_lib.starkv_decode_workspace_size_cfg(ctypes.byref(dims), int(batch),
                                                     int(max_seq_len), ctypes.byref(cfg),
                                                     ctypes.byref(out)),
               "starkv_decode_workspace_size_cfg")
    return int(out.value)


def decode_plan(dims, batch, max_seq_len):
    pps, ns = _i32(0), _i32(0)
    _check(_lib.starkv_decode_plan(ctypes.byref(dims), int(batch), int(max_seq_len),
                                   ctypes.byref(pps), ctypes.byref(ns)), "starkv_decode_plan")
    return int(pps.value), int(ns.value)


def prefill_workspace_size(dims, batch, total_q, max_seq_len):
    out = _sz(0)
    _check(_lib.starkv_prefill_workspace_size(ctypes.byref(dims), int(batch), int(total_q),
                                              int(max_seq_len), ctypes.byref(out)),
           "starkv_prefill_workspace_size")
    return int(out.value)


def alloc_workspace(nbytes, device):
    """A zero-filled workspace: its first 256 bytes (arrival counters of the
    few-token append) must start at zero, and every call leaves them zero."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def append_workspace_size(dims, num_tokens):
    out = _sz(0)
    _check(_lib.starkv_append_workspace_size(ctypes.byref(dims), int(num_tokens), ctypes.byref(out)),
           "starkv_append_workspace_size")
    return int(out.value)


def _append_workspace(dims, N, workspace, device):
    """(pointer, bytes) of the append workspace: the given one, or a new
    allocation when the call needs one and none was given."""
    need = append_workspace_size(dims, N)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = alloc_workspace(need, device)
    return _dev(workspace, torch.uint8, "workspace"), int(workspace.numel())


def append(k, v, U, W, slot_mapping, k_cache, v_cache, workspace=None, stream=None):
    """Project k, v [N, Hkv, d] to latents and write them to slot_mapping [N] (int64)."""
    dims = dims_of(k_cache, v_cache, U, W)
    N = k.shape[0]
    H, d = dims.num_heads, dims.head_dim
    ws, ws_bytes = _append_workspace(dims, N, workspace, k.device)
    st = _lib.starkv_append(
        ctypes.byref(dims), _dev(k, torch.float16, "k", (N, H, d)),
        _dev(v, torch.float16, "v", (N, H, d)), _dev(U, torch.float16, "U"),
        _dev(W, torch.float16, "W"), _dev(slot_mapping, torch.int64, "slot_mapping", (N,)),
        int(N), _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"),
        ws, ws_bytes, _stream(stream))
    _check(st, "starkv_append")


def append_fp8(k, v, U, W, slot_mapping, k_scale, v_scale, k_cache8, v_cache8, workspace=None,
               stream=None):
    """append() into FP8 E4M3 caches (uint8 codes, same layouts)."""
    dims = dims_of(k_cache8, v_cache8, U, W)
    N = k.shape[0]
    Hkv, d = dims.num_heads, dims.head_dim
    ws, ws_bytes = _append_workspace(dims, N, workspace, k.device)
    st = _lib.starkv_append_fp8(
        ctypes.byref(dims), _dev(k, torch.float16, "k", (N, Hkv, d)),
        _dev(v, torch.float16, "v", (N, Hkv, d)), _dev(U, torch.float16, "U"),
        _dev(W, torch.float16, "W"), _dev(slot_mapping, torch.int64, "slot_mapping", (N,)),
        int(N), float(k_scale), float(v_scale), _dev(k_cache8, torch.uint8, "k_cache8"),
        _dev(v_cache8, torch.uint8, "v_cache8"), ws, ws_bytes, _stream(stream))
    _check(st, "starkv_append_fp8")


def decode_attn_fp8(q, k_cache8, v_cache8, U, W, block_tables, seq_lens, max_seq_len, k_scale,
                    v_scale, scale=None, out=None, workspace=None, stream=None):
    """decode_attn() over FP8 E4M3 caches read as scale * value(code)."""
    dims = dims_of(k_cache8, v_cache8, U, W, num_heads=q.shape[1])
    B = q.shape[0]
    H, d = dims.num_heads, dims.head_dim
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float16, device=q.device)
    need = decode_workspace_size(dims, B, max_seq_len)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = _lib.starkv_decode_attn_fp8(
        ctypes.byref(dims), _dev(q, torch.float16, "q", (B, H, d)),
        _dev(k_cache8, torch.uint8, "k_cache8"), _dev(v_cache8, torch.uint8, "v_cache8"),
        _dev(U, torch.float16, "U"), _dev(W, torch.float16, "W"),
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens", (B,)), int(B), int(max_seq_len), float(scale),
        float(k_scale), float(v_scale), _dev(out, torch.float16, "out", (B, H, d)),
        _dev(workspace, torch.uint8, "workspace"), int(workspace.numel()), _stream(stream))
    _check(st, "starkv_decode_attn_fp8")
    return out


def decode_attn(q, k_cache, v_cache, U, W, block_tables, seq_lens, max_seq_len, scale=None,
                out=None, workspace=None, stream=None, pages_per_split=0, merge_seqs=0,
                launches=0):
    """Decode attention for q [B, H, d]; returns out [B, H, d] fp16.
    pages_per_split / merge_seqs / launches: a plan override (0 = the
    library's plan; launches 2 fuses the split pass and the merge, 3 keeps
    three kernels)."""
    dims = dims_of(k_cache, v_cache, U, W, num_heads=q.shape[1])
    B = q.shape[0]
    H, d = dims.num_heads, dims.head_dim
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float16, device=q.device)
    need = decode_workspace_size(dims, B, max_seq_len, pages_per_split, merge_seqs, launches)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    args = [ctypes.byref(dims), _dev(q, torch.float16, "q", (B, H, d)),
            _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"),
            _dev(U, torch.float16, "U"), _dev(W, torch.float16, "W"),
            _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
            _dev(seq_lens, torch.int32, "seq_lens", (B,)), int(B), int(max_seq_len), float(scale)]
    tail = [_dev(out, torch.float16, "out", (B, H, d)), _dev(workspace, torch.uint8, "workspace"),
            int(workspace.numel()), _stream(stream)]
    cfg = _config(pages_per_split, merge_seqs, launches)
    if cfg is None:
        _check(_lib.starkv_decode_attn(*args, *tail), "starkv_decode_attn")
    else:
        _check(_lib.starkv_decode_attn_cfg(*args, ctypes.byref(cfg), *tail),
               "starkv_decode_attn_cfg")
    return out


def decode_attn_noalloc(q, k_cache, v_cache, U, W, block_tables, seq_lens, max_seq_len, out,
                        scale=None, stream=None):
    """decode_attn() through the entry point that allocates nothing: the
    library's own scratch replaces the workspace; the caller passes out
    [B, H, d] fp16."""
    dims = dims_of(k_cache, v_cache, U, W, num_heads=q.shape[1])
    B = q.shape[0]
    H, d = dims.num_heads, dims.head_dim
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _lib.starkv_decode_attn_noalloc(
        ctypes.byref(dims), _dev(q, torch.float16, "q", (B, H, d)),
        _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"),
        _dev(U, torch.float16, "U"), _dev(W, torch.float16, "W"),
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens", (B,)), int(B), int(max_seq_len), float(scale),
        _dev(out, torch.float16, "out", (B, H, d)), _stream(stream))
    _check(st, "starkv_decode_attn_noalloc")
    return out


def prefill_attn(q, query_start_loc, max_query_len, k_cache, v_cache, U, W, block_tables,
                 seq_lens, max_seq_len, scale=None, out=None, workspace=None, stream=None):
    """Chunked-prefill attention for q [total_q, H, d]; returns out fp16."""
    dims = dims_of(k_cache, v_cache, U, W, num_heads=q.shape[1])
    T = q.shape[0]
    B = seq_lens.shape[0]
    H, d = dims.num_heads, dims.head_dim
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.float16, device=q.device)
    need = prefill_workspace_size(dims, B, T, max_seq_len)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = _lib.starkv_prefill_attn(
        ctypes.byref(dims), _dev(q, torch.float16, "q", (T, H, d)),
        _dev(query_start_loc, torch.int32, "query_start_loc", (B + 1,)), int(T),
        int(max_query_len), _dev(k_cache, torch.float16, "k_cache"),
        _dev(v_cache, torch.float16, "v_cache"), _dev(U, torch.float16, "U"),
        _dev(W, torch.float16, "W"), _dev(block_tables, torch.int32, "block_tables"),
        int(block_tables.shape[1]), _dev(seq_lens, torch.int32, "seq_lens", (B,)), int(B),
        int(max_seq_len), float(scale), _dev(out, torch.float16, "out", (T, H, d)),
        _dev(workspace, torch.uint8, "workspace"), int(workspace.numel()), _stream(stream))
    _check(st, "starkv_prefill_attn")
    return out


def fit_workspace_size(dims):
    out = _sz(0)
    _check(_lib.starkv_fit_workspace_size(ctypes.byref(dims), ctypes.byref(out)),
           "starkv_fit_workspace_size")
    return int(out.value)


def fit_bases(k, v, r_k, r_v, u0, w0, iters, U=None, W=None, workspace=None, info=None,
              residual=None, stream=None):
    """Bases U [H, d, r_k], W [H*d, r_v] (fp16) from samples k, v [N, H, d]
    (fp16), by subspace iteration from u0, w0 (fp32, same shapes).  `info`
    (int32 [1], optional) receives the count of non-positive pivots;
    `residual` (float32 [2], optional) the relative invariant-subspace
    residual of the returned key (largest over heads) and value bases."""
    N, H, d = k.shape
    dims = make_dims(H, d, r_k, r_v, 1)
    if U is None:
        U = torch.empty((H, d, r_k), dtype=torch.float16, device=k.device)
    if W is None:
        W = torch.empty((H * d, r_v), dtype=torch.float16, device=k.device)
    need = fit_workspace_size(dims)
    if workspace is None:
        workspace = alloc_workspace(need, k.device)
    st = _lib.starkv_fit_bases(
        ctypes.byref(dims), _dev(k, torch.float16, "k", (N, H, d)),
        _dev(v, torch.float16, "v", (N, H, d)), int(N),
        _dev(u0, torch.float32, "u0", (H, d, r_k)), _dev(w0, torch.float32, "w0", (H * d, r_v)),
        int(iters), _dev(U, torch.float16, "U", (H, d, r_k)),
        _dev(W, torch.float16, "W", (H * d, r_v)), _dev(workspace, torch.uint8, "workspace"),
        int(workspace.numel()), None if info is None else _dev(info, torch.int32, "info", (1,)),
        None if residual is None else _dev(residual, torch.float32, "residual", (2,)),
        _stream(stream))
    _check(st, "starkv_fit_bases")
    return U, W


def prefill_attn_fp8(q, query_start_loc, max_query_len, k_cache8, v_cache8, U, W, block_tables,
                     seq_lens, max_seq_len, k_scale, v_scale, scale=None, out=None,
                     workspace=None, stream=None):
    """prefill_attn() over FP8 E4M3 caches read as scale * value(code)."""
    dims = dims_of(k_cache8, v_cache8, U, W, num_heads=q.shape[1])
    T = q.shape[0]
    B = seq_lens.shape[0]
    H, d = dims.num_heads, dims.head_dim
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.float16, device=q.device)
    need = prefill_workspace_size(dims, B, T, max_seq_len)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = _lib.starkv_prefill_attn_fp8(
        ctypes.byref(dims), _dev(q, torch.float16, "q", (T, H, d)),
        _dev(query_start_loc, torch.int32, "query_start_loc", (B + 1,)), int(T),
        int(max_query_len), _dev(k_cache8, torch.uint8, "k_cache8"),
        _dev(v_cache8, torch.uint8, "v_cache8"), _dev(U, torch.float16, "U"),
        _dev(W, torch.float16, "W"), _dev(block_tables, torch.int32, "block_tables"),
        int(block_tables.shape[1]), _dev(seq_lens, torch.int32, "seq_lens", (B,)), int(B),
        int(max_seq_len), float(scale), float(k_scale), float(v_scale),
        _dev(out, torch.float16, "out", (T, H, d)), _dev(workspace, torch.uint8, "workspace"),
        int(workspace.numel()), _stream(stream))
    _check(st, "starkv_prefill_attn_fp8")
    return out


def check_indices(block_tables, seq_lens, max_seq_len, num_blocks, slot_mapping=None,
                  report=None, stream=None):
    """Index checks (debugging aid): returns the [4] device report of
    starkv_check_indices as int32 (flags; first sequence with a bad block id;
    first with a bad length; first token with a bad slot; -1, the uint32
    0xFFFFFFFF, for none)."""
    B = int(seq_lens.shape[0])
    dims = make_dims(1, 32, 8, 8, int(num_blocks))
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=seq_lens.device)
    n = 0 if slot_mapping is None else int(slot_mapping.shape[0])
    slots = None if slot_mapping is None else _dev(slot_mapping, torch.int64, "slot_mapping")
    _check(_lib.starkv_check_indices(
        ctypes.byref(dims), _dev(block_tables, torch.int32, "block_tables"),
        int(block_tables.shape[1]), _dev(seq_lens, torch.int32, "seq_lens", (B,)), B,
        int(max_seq_len), slots, n, _dev(report, torch.int32, "report", (4,)), _stream(stream)),
        "starkv_check_indices")
    return report


def stream_read(buf, sink, stream=None):
    """Measurement utility: stream-read a uint8 buffer (HBM ceiling)."""
    _check(_lib.starkv_util_stream_read(_dev(buf, torch.uint8, "buf"), int(buf.numel()),
                                        _dev(sink, torch.int32, "sink"), _stream(stream)),
           "starkv_util_stream_read")


class TimingEvent:
    """A library timing event (no system-scope fence when recorded)."""

    def __init__(self):
        h = _vp(None)
        _check(_lib.starkv_util_event_create(ctypes.byref(h)), "starkv_util_event_create")
        self.handle = h

    def elapsed_ms(self, stop):
        """Milliseconds from this event to `stop`; synchronise the device first."""
        ms = ctypes.c_float(0.0)
        _check(_lib.starkv_util_event_elapsed_ms(self.handle, stop.handle, ctypes.byref(ms)),
               "starkv_util_event_elapsed_ms")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _lib.starkv_util_event_destroy(self.handle)
            self.handle = None


def _event_handle(ev):
    if isinstance(ev, TimingEvent):
        return ev.handle
    return _vp(ev.cuda_event)      # a torch.cuda.Event


def set_timing_events(start_event, stop_event, which):
    """Time one kernel of later calls with two TimingEvent (or torch.cuda.Event)."""
    if which == TIME_NONE:
        _check(_lib.starkv_set_timing_events(None, None, 0), "starkv_set_timing_events")
        return
    _check(_lib.starkv_set_timing_events(_event_handle(start_event), _event_handle(stop_event),
                                         int(which)), "starkv_set_timing_events")
