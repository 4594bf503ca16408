"""ctypes binding of libpagedattn.so (argument marshalling only).

Each function takes torch tensors, checks what the C side cannot see (device,
dtype, contiguity, shape agreement), passes raw pointers and sizes to the C
entry point of the same name, and raises PagedAttnError on a non-zero status.
All compute runs in the library's HIP kernels; there is no fallback path:
if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpagedattn.so"

PA_F32, PA_BF16 = 0, 1
PA_PARTITION_BALANCED = -1  # pa_decode partition_size: equal work per resident wave
_STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED",
           3: "PA_ERR_WORKSPACE", 4: "PA_ERR_HIP"}


class PagedAttnError(RuntimeError):
    def __init__(self, func, status, message):
        self.status = status
        super().__init__(f"{func}: {_STATUS.get(status, status)}: {message}")


def library_path() -> str:
    return os.environ.get("PAGEDATTN_LIB", os.path.join(_HERE, _LIB_NAME))


_lib = None

_c_void_p, _i32, _i64, _f32, _size = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_float, ctypes.c_size_t)

_SIGNATURES = {
    "pa_store_kvcache": ([_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                          _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_decode_workspace_size": ([_i32, _i32, _i32, _i32, _i32], _size),
    "pa_decode_workspace_size_kv": ([_i32, _i32, _i32, _i32, _i32, _i32], _size),
    "pa_decode": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                   _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                   _c_void_p, _size, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_decode_noalloc": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                           ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_decode_hinted": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                          _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                          _c_void_p, _size, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_store_decode": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p,
                         _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                         _i32, _f32, _i32, _c_void_p, _size, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_store_decode_fp8": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _c_void_p,
                             _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                             _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                             _c_void_p, _size, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_prefill_chunk": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                          _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                          _f32, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_store_kvcache_fp8": ([_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                              _c_void_p], ctypes.c_int),
    "pa_decode_fp8": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                       _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                       _c_void_p, _size, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_prefill_chunk_fp8": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32,
                              _i32, _i32, _i32, _f32, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_mixed_batch": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                        _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                        _c_void_p, _size, ctypes.c_int, _c_void_p], ctypes.c_int),
    "pa_mixed_batch_fp8": ([_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32,
                            _i32, _i32, _i32, _i32, _f32, _c_void_p, _size, ctypes.c_int,
                            _c_void_p], ctypes.c_int),
    "pa_stream_read": ([_c_void_p, _size, _c_void_p, ctypes.POINTER(_size), _c_void_p], ctypes.c_int),
    "pa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "pa_last_error": ([], ctypes.c_char_p),
}


def load_library():
    """Load the built library once; raise if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build the HIP library first "
            f"(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(func, status):
    if status != 0:
        msg = load_library().pa_last_error().decode(errors="replace")
        raise PagedAttnError(func, status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(cond, what):
    if not cond:
        raise ValueError(what)


def _int32_device(t, name, device):
    _need(t.dtype == torch.int32, f"{name} must be int32")
    _need(t.device == device, f"{name} must be on {device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def pa_status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def pa_store_kvcache(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Scatter key/value rows [T][Hkv][D] into the pools by slot_mapping."""
    lib = load_library()
    T, Hkv, D = key.shape
    _need(value.shape == key.shape, "key and value shapes differ")
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "pools must be [NB][bs][Hkv][D]")
    NB, bs, Hkv2, D2 = k_cache.shape
    _need((Hkv2, D2) == (Hkv, D), "pool head shape does not match key")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "pools must be contiguous")
    for t in (key, value):
        _need(t.stride(2) == 1 and t.stride(1) == D, "key/value rows must be dense [Hkv][D]")
    _need(key.dtype == value.dtype == k_cache.dtype == v_cache.dtype, "dtypes differ")
    _int32_device(slot_mapping, "slot_mapping", k_cache.device)
    _need(slot_mapping.numel() == T, "slot_mapping length differs from key")
    st = lib.pa_store_kvcache(_ptr(key), _ptr(value), key.stride(0), value.stride(0),
                              _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, Hkv, D, bs, NB,
                              _dtype_code(key), _stream(stream))
    _check("pa_store_kvcache", st)


def pa_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size) -> int:
    """Workspace bytes a decode call needs whatever its KV head count."""
    return int(load_library().pa_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len,
                                                       partition_size))


def pa_decode_workspace_size_kv(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                partition_size) -> int:
    """Workspace bytes of a decode call with this KV head count (exact)."""
    return int(load_library().pa_decode_workspace_size_kv(num_seqs, num_heads, num_kv_heads, head_dim,
                                                          max_context_len, partition_size))


def decode_workspace(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                     partition_size, device):
    """A workspace of the size the decode calls need (None if 0); its
    contents do not matter."""
    n = pa_decode_workspace_size_kv(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                    partition_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def _shared_lens(t, num_seqs, device):
    """Pointer of the optional shared_lens hint (None stays NULL)."""
    if t is None:
        return None
    _int32_device(t, "shared_lens", device)
    _need(t.numel() == num_seqs, "shared_lens must have B entries")
    return _ptr(t)


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, workspace):
    """Checks shared by pa_decode and pa_decode_hinted; returns
    (B, Hq, Hkv, D, bs, NB, workspace pointer, workspace bytes)."""
    B, Hq, D = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "pools must be [NB][bs][Hkv][D]")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "pools must be contiguous")
    NB, bs, Hkv, D2 = k_cache.shape
    _need(D2 == D, "head_dim of pools and q differ")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "dtypes differ")
    _int32_device(block_tables, "block_tables", q.device)
    _int32_device(context_lens, "context_lens", q.device)
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B][max_blocks]")
    _need(context_lens.numel() == B, "context_lens must have B entries")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace.device == q.device and workspace.is_contiguous(), "bad workspace")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    return B, Hq, Hkv, D, bs, NB, ws_ptr, ws_bytes


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
              partition_size=0, workspace=None, stream=None):
    """Single-token decode; out and q are [B][Hq][D]."""
    lib = load_library()
    B, Hq, Hkv, D, bs, NB, ws_ptr, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                           context_lens, workspace)
    st = lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                       _ptr(context_lens), B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                       int(max_context_len), float(scale), int(partition_size), ws_ptr, ws_bytes,
                       _dtype_code(q), _stream(stream))
    _check("pa_decode", st)


PA_NOALLOC_SCRATCH_BYTES = 16 << 20  # the library's static scratch per GPU


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                      partition_size=0, stream=None):
    """pa_decode without a workspace: a split keeps its partial states in
    the library's static per-GPU scratch (calls on one GPU must not
    overlap); nothing is allocated."""
    lib = load_library()
    B, Hq, Hkv, D, bs, NB, _, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, None)
    st = lib.pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                               _ptr(context_lens), B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                               int(max_context_len), float(scale), int(partition_size), _dtype_code(q),
                               _stream(stream))
    _check("pa_decode_noalloc", st)


def pa_decode_hinted(out, q, k_cache, v_cache, block_tables, context_lens, shared_lens,
                     max_context_len, scale, partition_size=0, workspace=None, stream=None):
    """pa_decode with the shared-prefix load hint: shared_lens (int32 [B] or
    None) gives the leading context tokens of each sequence in blocks other
    sequences also read; the result is pa_decode's."""
    lib = load_library()
    B, Hq, Hkv, D, bs, NB, ws_ptr, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                           context_lens, workspace)
    sl = _shared_lens(shared_lens, B, q.device)
    st = lib.pa_decode_hinted(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                              _ptr(context_lens), sl, B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                              int(max_context_len), float(scale), int(partition_size), ws_ptr,
                              ws_bytes, _dtype_code(q), _stream(stream))
    _check("pa_decode_hinted", st)


def pa_store_decode(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens,
                    max_context_len, scale, partition_size=0, workspace=None, stream=None,
                    shared_lens=None):
    """Store each sequence's newest K/V row [B][Hkv][D] and decode, in one
    launch; the same as pa_store_kvcache followed by pa_decode (shared_lens
    as for pa_decode_hinted)."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "pools must be [NB][bs][Hkv][D]")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "pools must be contiguous")
    NB, bs, Hkv, D2 = k_cache.shape
    _need(D2 == D, "head_dim of pools and q differ")
    _need(key.shape == value.shape == (B, Hkv, D), "key/value must be [B][Hkv][D]")
    for t in (key, value):
        _need(t.stride(2) == 1 and t.stride(1) == D, "key/value rows must be dense [Hkv][D]")
    _need(q.dtype == k_cache.dtype == v_cache.dtype == key.dtype == value.dtype, "dtypes differ")
    for name, t in (("slot_mapping", slot_mapping), ("block_tables", block_tables),
                    ("context_lens", context_lens)):
        _int32_device(t, name, q.device)
    _need(slot_mapping.numel() == B, "slot_mapping must have B entries")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B][max_blocks]")
    _need(context_lens.numel() == B, "context_lens must have B entries")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace.device == q.device and workspace.is_contiguous(), "bad workspace")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    sl = _shared_lens(shared_lens, B, q.device)
    st = lib.pa_store_decode(_ptr(out), _ptr(q), _ptr(key), _ptr(value), key.stride(0), value.stride(0),
                             _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), _ptr(block_tables),
                             _ptr(context_lens), sl, B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                             int(max_context_len), float(scale), int(partition_size), ws_ptr, ws_bytes,
                             _dtype_code(q), _stream(stream))
    _check("pa_store_decode", st)


def pa_store_decode_fp8(out, q, key, value, k_cache, v_cache, k_scale, v_scale, slot_mapping,
                        block_tables, context_lens, max_context_len, scale, partition_size=0,
                        workspace=None, stream=None, shared_lens=None):
    """pa_store_decode over E4M3 pools: quantise each sequence's newest K/V
    row [B][Hkv][D] (the dtype of q) into its slot and decode, in one launch."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _e4m3_pools(k_cache, v_cache)
    NB, bs, Hkv, D2 = k_cache.shape
    _need(D2 == D, "head_dim of pools and q differ")
    _scales(k_scale, v_scale, Hkv, q.device)
    _need(key.shape == value.shape == (B, Hkv, D), "key/value must be [B][Hkv][D]")
    for t in (key, value):
        _need(t.stride(2) == 1 and t.stride(1) == D, "key/value rows must be dense [Hkv][D]")
        _need(t.dtype == q.dtype, "key/value must have the dtype of q")
    for name, t in (("slot_mapping", slot_mapping), ("block_tables", block_tables),
                    ("context_lens", context_lens)):
        _int32_device(t, name, q.device)
    _need(slot_mapping.numel() == B, "slot_mapping must have B entries")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B][max_blocks]")
    _need(context_lens.numel() == B, "context_lens must have B entries")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace.device == q.device and workspace.is_contiguous(), "bad workspace")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    sl = _shared_lens(shared_lens, B, q.device)
    st = lib.pa_store_decode_fp8(_ptr(out), _ptr(q), _ptr(key), _ptr(value), key.stride(0),
                                 value.stride(0), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                 _ptr(v_scale), _ptr(slot_mapping), _ptr(block_tables),
                                 _ptr(context_lens), sl, B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                                 int(max_context_len), float(scale), int(partition_size), ws_ptr,
                                 ws_bytes, _dtype_code(q), _stream(stream))
    _check("pa_store_decode_fp8", st)


def _e4m3_pools(k_cache, v_cache):
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "pools must be [NB][bs][Hkv][D]")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "pools must be contiguous")
    for t in (k_cache, v_cache):
        _need(t.dtype in (torch.uint8, torch.float8_e4m3fn), "E4M3 pools must be uint8 or float8_e4m3fn")


def _scales(k_scale, v_scale, num_kv_heads, device):
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t.dtype == torch.float32 and t.device == device and t.is_contiguous(),
              f"{name} must be a contiguous float32 tensor on {device}")
        _need(t.numel() == num_kv_heads, f"{name} must have num_kv_heads entries")


def pa_store_kvcache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream=None):
    """Quantise key/value rows [T][Hkv][D] (bf16 or fp32) to E4M3 codes with
    per-KV-head scales and scatter them into the uint8 pools by slot_mapping."""
    lib = load_library()
    T, Hkv, D = key.shape
    _need(value.shape == key.shape and value.dtype == key.dtype, "key and value differ")
    _e4m3_pools(k_cache, v_cache)
    NB, bs, Hkv2, D2 = k_cache.shape
    _need((Hkv2, D2) == (Hkv, D), "pool head shape does not match key")
    for t in (key, value):
        _need(t.stride(2) == 1 and t.stride(1) == D, "key/value rows must be dense [Hkv][D]")
    _int32_device(slot_mapping, "slot_mapping", k_cache.device)
    _need(slot_mapping.numel() == T, "slot_mapping length differs from key")
    _scales(k_scale, v_scale, Hkv, k_cache.device)
    st = lib.pa_store_kvcache_fp8(_ptr(key), _ptr(value), key.stride(0), value.stride(0),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), _ptr(k_scale),
                                  _ptr(v_scale), T, Hkv, D, bs, NB, _dtype_code(key), _stream(stream))
    _check("pa_store_kvcache_fp8", st)


def pa_decode_fp8(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                  max_context_len, scale, partition_size=0, workspace=None, stream=None,
                  shared_lens=None):
    """Single-token decode over E4M3 pools; out and q are [B][Hq][D] (bf16 or
    fp32), the workspace as for pa_decode, shared_lens as for
    pa_decode_hinted."""
    lib = load_library()
    B, Hq, D = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _e4m3_pools(k_cache, v_cache)
    NB, bs, Hkv, D2 = k_cache.shape
    _need(D2 == D, "head_dim of pools and q differ")
    _scales(k_scale, v_scale, Hkv, q.device)
    _int32_device(block_tables, "block_tables", q.device)
    _int32_device(context_lens, "context_lens", q.device)
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B][max_blocks]")
    _need(context_lens.numel() == B, "context_lens must have B entries")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace.device == q.device and workspace.is_contiguous(), "bad workspace")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    sl = _shared_lens(shared_lens, B, q.device)
    st = lib.pa_decode_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                           _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), sl, B, Hq, Hkv, D, bs,
                           NB, block_tables.shape[1], int(max_context_len), float(scale),
                           int(partition_size), ws_ptr, ws_bytes, _dtype_code(q), _stream(stream))
    _check("pa_decode_fp8", st)


def pa_prefill_chunk(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                     max_query_len, max_context_len, scale, stream=None):
    """Chunked causal prefill; out and q are [sum n_i][Hq][D]."""
    lib = load_library()
    T, Hq, D = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "pools must be [NB][bs][Hkv][D]")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "pools must be contiguous")
    NB, bs, Hkv, D2 = k_cache.shape
    _need(D2 == D, "head_dim of pools and q differ")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "dtypes differ")
    for name, t in (("block_tables", block_tables), ("query_start_loc", query_start_loc),
                    ("context_lens", context_lens)):
        _int32_device(t, name, q.device)
    B = context_lens.numel()
    _need(query_start_loc.numel() == B + 1, "query_start_loc must have B+1 entries")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B][max_blocks]")
    st = lib.pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                              _ptr(query_start_loc), _ptr(context_lens), B, Hq, Hkv, D, bs, NB,
                              block_tables.shape[1], int(max_query_len), int(max_context_len),
                              float(scale), _dtype_code(q), _stream(stream))
    _check("pa_prefill_chunk", st)


def pa_prefill_chunk_fp8(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, query_start_loc,
                         context_lens, max_query_len, max_context_len, scale, stream=None):
    """Chunked causal prefill over E4M3 pools; out and q are bf16
    [sum n_i][Hq][D], the pools uint8 codes, the scales fp32 [Hkv]."""
    lib = load_library()
    T, Hq, D = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _e4m3_pools(k_cache, v_cache)
    NB, bs, Hkv, D2 = k_cache.shape
    _need(D2 == D, "head_dim of pools and q differ")
    _scales(k_scale, v_scale, Hkv, q.device)
    for name, t in (("block_tables", block_tables), ("query_start_loc", query_start_loc),
                    ("context_lens", context_lens)):
        _int32_device(t, name, q.device)
    B = context_lens.numel()
    _need(query_start_loc.numel() == B + 1, "query_start_loc must have B+1 entries")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B][max_blocks]")
    st = lib.pa_prefill_chunk_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                  _ptr(v_scale), _ptr(block_tables), _ptr(query_start_loc),
                                  _ptr(context_lens), B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                                  int(max_query_len), int(max_context_len), float(scale),
                                  _dtype_code(q), _stream(stream))
    _check("pa_prefill_chunk_fp8", st)


# ---------------------------------------------------------------------------
# block manager (host only)
# ---------------------------------------------------------------------------

_BM_SIGNATURES = {
    "pa_bm_create": ([_i32, _i32, _c_void_p, ctypes.POINTER(_c_void_p)], ctypes.c_int),
    "pa_bm_destroy": ([_c_void_p], None),
    "pa_bm_allocate": ([_c_void_p, _c_void_p, _i32, _c_void_p, _i32, ctypes.POINTER(_i32),
                        ctypes.POINTER(_i32), _c_void_p], ctypes.c_int),
    "pa_bm_append": ([_c_void_p, _c_void_p, ctypes.POINTER(_i32), _i32, _i32, _i32,
                      ctypes.POINTER(_i32)], ctypes.c_int),
    "pa_bm_free": ([_c_void_p, _c_void_p, _i32], ctypes.c_int),
    "pa_bm_num_free": ([_c_void_p], _i32),
    "pa_bm_ref_count": ([_c_void_p, _i32], _i32),
    "pa_bm_shared_tokens": ([_c_void_p, _c_void_p, _i32, _i32], _i32),
    "pa_bm_last_error": ([], ctypes.c_char_p),
}
PA_ERR_OUT_OF_BLOCKS = 5


class OutOfBlocks(PagedAttnError):
    pass


def _bm_lib():
    lib = load_library()
    if not getattr(lib, "_bm_ready", False):
        for name, (args, res) in _BM_SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        lib._bm_ready = True
    return lib


def _bm_check(func, status):
    if status != 0:
        msg = _bm_lib().pa_bm_last_error().decode(errors="replace")
        cls = OutOfBlocks if status == PA_ERR_OUT_OF_BLOCKS else PagedAttnError
        raise cls(func, status, msg)


def _i32_array(values):
    import numpy as np
    return np.ascontiguousarray(np.asarray(values, dtype=np.int32))


class BlockManager:
    """The library's host-side block manager (pa_bm_*): block tables with
    prefix sharing, decode appends and reference-counted frees. Tables are
    numpy int32 arrays of the sequence's block ids."""

    def __init__(self, num_blocks, block_size, free_order=None):
        lib = _bm_lib()
        self.block_size = int(block_size)
        handle = _c_void_p()
        fo = None if free_order is None else _i32_array(free_order)
        _bm_check("pa_bm_create", lib.pa_bm_create(int(num_blocks), self.block_size,
                                                   None if fo is None else fo.ctypes.data,
                                                   ctypes.byref(handle)))
        self._h = handle
        self._lib = lib

    def close(self):
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def allocate(self, token_ids, with_slots=False):
        """(table, num_cached_tokens[, slots]) for a new sequence's prompt."""
        import numpy as np
        toks = _i32_array(token_ids)
        n = len(toks)
        cap = max(1, -(-n // self.block_size))
        table = np.empty(cap, dtype=np.int32)
        slots = np.empty(max(1, n), dtype=np.int32) if with_slots else None
        nb, cached = _i32(), _i32()
        _bm_check("pa_bm_allocate", self._lib.pa_bm_allocate(
            self._h, toks.ctypes.data if n else None, n, table.ctypes.data, cap, ctypes.byref(nb),
            ctypes.byref(cached), None if slots is None else slots.ctypes.data))
        table = table[:nb.value].copy()
        if with_slots:
            return table, cached.value, slots[:n].copy()
        return table, cached.value

    def append(self, table, num_tokens, token_id):
        """Append one token at position num_tokens; returns (table, slot), the
        table grown by one block when the last one was full."""
        import numpy as np
        nb = len(table)
        buf = np.empty(nb + 1, dtype=np.int32)
        buf[:nb] = table
        nbv, slot = _i32(nb), _i32()
        _bm_check("pa_bm_append", self._lib.pa_bm_append(self._h, buf.ctypes.data, ctypes.byref(nbv),
                                                         nb + 1, int(num_tokens), int(token_id),
                                                         ctypes.byref(slot)))
        return buf[:nbv.value].copy(), slot.value

    def free(self, table):
        t = _i32_array(table)
        _bm_check("pa_bm_free", self._lib.pa_bm_free(self._h, t.ctypes.data if len(t) else None, len(t)))

    def num_free(self):
        return int(self._lib.pa_bm_num_free(self._h))

    def ref_count(self, block_id):
        return int(self._lib.pa_bm_ref_count(self._h, int(block_id)))

    def shared_tokens(self, table, num_tokens):
        """Leading tokens of a sequence that lie in blocks other sequences
        also hold (its shared_lens entry for the decode calls)."""
        t = _i32_array(table)
        n = int(self._lib.pa_bm_shared_tokens(self._h, t.ctypes.data if len(t) else None, len(t),
                                              int(num_tokens)))
        if n < 0:
            raise ValueError("pa_bm_shared_tokens: invalid arguments")
        return n


def mixed_workspace(num_decode_seqs, num_heads, num_kv_heads, head_dim, max_context_len, device):
    """The workspace pa_mixed_batch needs (None when there is no decode row)."""
    if num_decode_seqs == 0:
        return None
    return decode_workspace(num_decode_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                            PA_PARTITION_BALANCED, device)


def pa_mixed_batch(out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                   num_decode_seqs, max_query_len, max_context_len, scale, workspace=None,
                   stream=None, shared_lens=None):
    """A continuous batch in one call: the first num_decode_seqs sequences are
    decode tokens (one row each), the rest prefill chunks; out and q are
    [T][Hq][D] bf16. shared_lens (int32 [B] or None): the decode rows'
    load-policy hint, as for pa_decode_hinted."""
    lib = load_library()
    T, Hq, D = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape, "pools must be [NB][bs][Hkv][D]")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "pools must be contiguous")
    NB, bs, Hkv, D2 = k_cache.shape
    _need(D2 == D, "head_dim of pools and q differ")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "dtypes differ")
    for name, t in (("block_tables", block_tables), ("query_start_loc", query_start_loc),
                    ("context_lens", context_lens)):
        _int32_device(t, name, q.device)
    B = context_lens.numel()
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B][max_blocks]")
    _need(query_start_loc.numel() == B + 1, "query_start_loc must have B+1 entries")
    _need(0 <= num_decode_seqs <= B and num_decode_seqs <= T, "num_decode_seqs out of range")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace.device == q.device and workspace.is_contiguous(), "bad workspace")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    sl = _shared_lens(shared_lens, B, q.device)
    st = lib.pa_mixed_batch(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                            _ptr(query_start_loc), _ptr(context_lens), sl, B, int(num_decode_seqs), Hq, Hkv,
                            D, bs, NB, block_tables.shape[1], int(max_query_len), int(max_context_len),
                            float(scale), ws_ptr, ws_bytes, _dtype_code(q), _stream(stream))
    _check("pa_mixed_batch", st)


def pa_mixed_batch_fp8(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, query_start_loc,
                       context_lens, num_decode_seqs, max_query_len, max_context_len, scale,
                       workspace=None, stream=None, shared_lens=None):
    """pa_mixed_batch over E4M3 pools (uint8 codes, fp32 per-head scales);
    out and q are [T][Hq][D] bf16, the workspace and shared_lens as for
    pa_mixed_batch."""
    lib = load_library()
    T, Hq, D = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _e4m3_pools(k_cache, v_cache)
    NB, bs, Hkv, D2 = k_cache.shape
    _need(D2 == D, "head_dim of pools and q differ")
    _scales(k_scale, v_scale, Hkv, q.device)
    for name, t in (("block_tables", block_tables), ("query_start_loc", query_start_loc),
                    ("context_lens", context_lens)):
        _int32_device(t, name, q.device)
    B = context_lens.numel()
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B][max_blocks]")
    _need(query_start_loc.numel() == B + 1, "query_start_loc must have B+1 entries")
    _need(0 <= num_decode_seqs <= B and num_decode_seqs <= T, "num_decode_seqs out of range")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace.device == q.device and workspace.is_contiguous(), "bad workspace")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    sl = _shared_lens(shared_lens, B, q.device)
    st = lib.pa_mixed_batch_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                _ptr(v_scale), _ptr(block_tables), _ptr(query_start_loc),
                                _ptr(context_lens), sl, B, int(num_decode_seqs), Hq, Hkv, D, bs, NB,
                                block_tables.shape[1], int(max_query_len), int(max_context_len),
                                float(scale), ws_ptr, ws_bytes, _dtype_code(q), _stream(stream))
    _check("pa_mixed_batch_fp8", st)


def pa_stream_read(buf, out, stream=None):
    """One streaming read of the device tensor buf (a measurement aid: the
    device's sustained read rate); out is a one-element int32 tensor on the
    same device. Returns the bytes the launch reads."""
    lib = load_library()
    _need(buf.is_cuda and buf.is_contiguous(), "buf must be a contiguous device tensor")
    _need(out.device == buf.device and out.dtype == torch.int32 and out.numel() >= 1,
          "out must be an int32 tensor on the device of buf")
    n = _size(0)
    st = lib.pa_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), ctypes.byref(n),
                            _stream(stream))
    _check("pa_stream_read", st)
    return int(n.value)

