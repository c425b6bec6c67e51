"""ctypes binding of libpa_mi355x.so (the C ABI of include/pa.h and include/pa_blocks.h).

Argument marshalling only: shapes become ints, tensors become device
pointers, the current torch stream becomes the hipStream_t.  Every step of
the computation runs in the library's kernels.  If the library has not been
built, loading raises ImportError -- there is no fallback path.

The functions carry the C names (pa_decode, pa_decode_noalloc, pa_decode_ex, pa_decode_path,
pa_decode_workspace_bytes, pa_reshape_and_cache, pa_copy_blocks,
pa_swap_blocks, pa_status_string, pa_abi_version); `BlockManager` wraps the
pa_bm_* calls of the host block manager.  `lib()` returns the raw ctypes
handle for callers that want to pass pointers themselves.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libpa_mi355x.so")
INCLUDE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_NO_BLOCKS = range(6)
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_LAYOUT_BHTD, PA_LAYOUT_BTHD = 0, 1
PA_KERNEL_AUTO, PA_KERNEL_VECTOR, PA_KERNEL_MFMA = 0, 1, 2
PA_PARTITION_AUTO, PA_PARTITION_SINGLE, PA_PARTITION_BALANCED = 0, -1, -2
PA_DECODE_SHARED_BLOCKS = 1
PA_NOALLOC_SCRATCH_BYTES = 32 << 20    # scratch of pa_decode_noalloc (include/pa.h)
STATUS_NAMES = {PA_OK: "PA_OK", PA_ERR_INVALID_ARG: "PA_ERR_INVALID_ARG", PA_ERR_UNSUPPORTED: "PA_ERR_UNSUPPORTED",
                PA_ERR_WORKSPACE: "PA_ERR_WORKSPACE", PA_ERR_HIP: "PA_ERR_HIP", PA_ERR_NO_BLOCKS: "PA_ERR_NO_BLOCKS"}
POOL_GPU, POOL_CPU = 0, 1

_lock = threading.Lock()
_lib = None


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({pa_status_string(status)})")


def declared_functions(include_dir: str = INCLUDE_DIR):
    """Names of the functions the headers under include/ declare."""
    names = set()
    for h in sorted(glob.glob(os.path.join(include_dir, "*.h"))):
        with open(h) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pa_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def lib():
    """Load the library (once).  Raises ImportError if it was never built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_405_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
            L.pa_decode.restype = i32
            L.pa_decode.argtypes = [vp] * 6 + [i32] * 6 + [f32, i32, vp, sz, vp]
            L.pa_decode_noalloc.restype = i32
            L.pa_decode_noalloc.argtypes = [vp] * 6 + [i32] * 6 + [f32, i32, vp]
            L.pa_decode_ex.restype = i32
            L.pa_decode_ex.argtypes = [vp] * 6 + [i32] * 7 + [f32, i32, i32, i32, i32, ctypes.c_uint32, vp, sz, vp]
            L.pa_decode_append.restype = i32
            L.pa_decode_append.argtypes = [vp] * 9 + [i32] * 7 + [f32, i32, i32, i32, i32, ctypes.c_uint32, vp, sz, vp]
            L.pa_decode_shared_prefix.restype = i32
            L.pa_decode_shared_prefix.argtypes = [vp] * 6 + [i32] * 8 + [f32, i32, i32, vp, sz, vp]
            L.pa_decode_shared_prefix_workspace_bytes.restype = i32
            L.pa_decode_shared_prefix_workspace_bytes.argtypes = [i32] * 8 + [ctypes.POINTER(sz)]
            L.pa_decode_workspace_bytes.restype = i32
            L.pa_decode_workspace_bytes.argtypes = [i32] * 8 + [ctypes.POINTER(sz)]
            L.pa_decode_path.restype = i32
            L.pa_decode_path.argtypes = [i32] * 9 + [ctypes.POINTER(i32), ctypes.POINTER(i32)]
            L.pa_reshape_and_cache.restype = i32
            L.pa_reshape_and_cache.argtypes = [vp] * 5 + [i32] * 7 + [vp]
            i64, pi32, pi64, vpp = ctypes.c_int64, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_int64), \
                ctypes.POINTER(vp)
            L.pa_copy_blocks.restype = i32
            L.pa_copy_blocks.argtypes = [vp, vp, vp] + [i32] * 6 + [vp]
            L.pa_swap_blocks.restype = i32
            L.pa_swap_blocks.argtypes = [vp] * 5 + [i32] * 7 + [vp]
            L.pa_bm_create.restype = i32
            L.pa_bm_create.argtypes = [i32, i32, i32, vpp]
            L.pa_bm_destroy.restype = None
            L.pa_bm_destroy.argtypes = [vp]
            L.pa_bm_add.restype = i32
            L.pa_bm_add.argtypes = [vp, i64]
            L.pa_bm_fork.restype = i32
            L.pa_bm_fork.argtypes = [vp, i64, i64]
            L.pa_bm_blocks_needed.restype = i32
            L.pa_bm_blocks_needed.argtypes = [vp, i64, i32, pi32]
            L.pa_bm_append.restype = i32
            L.pa_bm_append.argtypes = [vp, i64, i32, pi64, pi32, i32, pi32]
            L.pa_bm_free.restype = i32
            L.pa_bm_free.argtypes = [vp, i64]
            L.pa_bm_add_cached.restype = i32
            L.pa_bm_add_cached.argtypes = [vp, i64, pi32, i32, pi32]
            L.pa_bm_append_tokens.restype = i32
            L.pa_bm_append_tokens.argtypes = [vp, i64, pi32, i32, pi64, pi32, i32, pi32]
            L.pa_bm_cache_stats.restype = i32
            L.pa_bm_cache_stats.argtypes = [vp, pi32, pi32]
            for f in (L.pa_bm_swap_out, L.pa_bm_swap_in):
                f.restype = i32
                f.argtypes = [vp, i64, pi32, i32, pi32]
            L.pa_bm_block_tables.restype = i32
            L.pa_bm_block_tables.argtypes = [vp, pi64, i32, i32, pi32, pi32]
            L.pa_bm_num_free.restype = i32
            L.pa_bm_num_free.argtypes = [vp, i32, pi32]
            L.pa_bm_ref_count.restype = i32
            L.pa_bm_ref_count.argtypes = [vp, i32, i32, pi32]
            L.pa_bm_info.restype = i32
            L.pa_bm_info.argtypes = [vp, i64, pi64, pi32, pi32]
            L.pa_prefill.restype = i32
            L.pa_prefill.argtypes = [vp] * 7 + [i32] * 9 + [f32, i32, i32, ctypes.c_uint32, vp]
            L.pa_prefill_shared_prefix.restype = i32
            L.pa_prefill_shared_prefix.argtypes = [vp] * 7 + [i32] * 10 + [f32, i32, i32, vp, sz, vp]
            L.pa_prefill_shared_prefix_workspace_bytes.restype = i32
            L.pa_prefill_shared_prefix_workspace_bytes.argtypes = [i32] * 5 + [ctypes.POINTER(sz)]
            L.pa_status_string.restype = ctypes.c_char_p
            L.pa_probe_stream_read.restype = i32
            L.pa_probe_stream_read.argtypes = [vp, sz, vp, i32, i32, vp]
            L.pa_status_string.argtypes = [i32]
            L.pa_abi_version.restype = i32
            L.pa_abi_version.argtypes = []
            _lib = L
    return _lib


def pa_status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


def pa_abi_version() -> int:
    return int(lib().pa_abi_version())


# ---------------------------------------------------------------------------
# torch-tensor marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported element type {t.dtype}")
    return codes[t.dtype]


def _dev(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def cache_dims(k_cache, layout: int):
    """(num_blocks, block_size, num_kv_heads, head_dim) of a cache tensor in `layout`."""
    NB, a, b, D = k_cache.shape
    return (NB, b, a, D) if layout == PA_LAYOUT_BHTD else (NB, a, b, D)


def pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                              dtype_code, partition_tokens=0) -> int:
    out = ctypes.c_size_t(0)
    st = lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                         max_blocks_per_seq, dtype_code, partition_tokens, ctypes.byref(out))
    if st != PA_OK:
        raise PaError(st, "pa_decode_workspace_bytes")
    return int(out.value)


def pa_decode_path(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   dtype_code, partition_tokens=0, kernel=PA_KERNEL_AUTO) -> tuple[int, int]:
    """(partition, kernel) pa_decode_ex resolves these arguments to."""
    part, kern = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib().pa_decode_path(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                              dtype_code, partition_tokens, kernel, ctypes.byref(part), ctypes.byref(kern))
    if st != PA_OK:
        raise PaError(st, "pa_decode_path")
    return int(part.value), int(kern.value)


def _workspace(q, nbytes, workspace):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    return workspace, workspace.numel() * workspace.element_size()


def pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, scale, *, num_blocks=None,
                 layout=PA_LAYOUT_BHTD, partition_tokens=0, kernel=PA_KERNEL_AUTO, shared_blocks=False,
                 workspace=None, stream=None):
    """out[S, Hq, D] <- paged decode attention of q[S, Hq, D] over the caches.

    shared_blocks: some physical blocks are read by several sequences in this
    call (PA_DECODE_SHARED_BLOCKS): keep them in the caches."""
    torch = _torch()
    code = _dtype_code(q)
    S, Hq, D = q.shape
    NB, bs, Hkv, D2 = cache_dims(k_cache, layout)
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, out and the caches")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    MB = block_tables.shape[1]
    nbytes = pa_decode_workspace_bytes(S, Hq, Hkv, D, bs, MB, code, partition_tokens)
    ws, ws_bytes = _workspace(q, nbytes, workspace)
    st = lib().pa_decode_ex(
        _dev(out, "out", q.dtype), _dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        S, Hq, Hkv, D, bs, MB, NB if num_blocks is None else int(num_blocks), float(scale), code, int(layout),
        int(partition_tokens), int(kernel), PA_DECODE_SHARED_BLOCKS if shared_blocks else 0,
        None if ws is None else ws.data_ptr(), ws_bytes, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_ex")
    return out


def pa_decode_append(out, q, k_new, v_new, k_cache, v_cache, slot_mapping, block_tables, context_lens, scale, *,
                     num_blocks=None, layout=PA_LAYOUT_BHTD, partition_tokens=0, kernel=PA_KERNEL_AUTO,
                     shared_blocks=False, workspace=None, stream=None):
    """One decode step: sequence s's new K/V rows k_new/v_new[s] go to slot slot_mapping[s], then
    out[S, Hq, D] <- paged decode attention of q over the caches (context_lens count the new token)."""
    torch = _torch()
    code = _dtype_code(q)
    S, Hq, D = q.shape
    NB, bs, Hkv, D2 = cache_dims(k_cache, layout)
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, out and the caches")
    if tuple(k_new.shape) != (S, Hkv, D) or tuple(v_new.shape) != (S, Hkv, D) or tuple(slot_mapping.shape) != (S,):
        raise ValueError("k_new, v_new must be [S, Hkv, D] and slot_mapping [S]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    MB = block_tables.shape[1]
    nbytes = pa_decode_workspace_bytes(S, Hq, Hkv, D, bs, MB, code, partition_tokens)
    ws, ws_bytes = _workspace(q, nbytes, workspace)
    st = lib().pa_decode_append(
        _dev(out, "out", q.dtype), _dev(q, "q"), _dev(k_new, "k_new", q.dtype), _dev(v_new, "v_new", q.dtype),
        _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(slot_mapping, "slot_mapping", torch.int64), _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32),
        S, Hq, Hkv, D, bs, MB, NB if num_blocks is None else int(num_blocks), float(scale), code, int(layout),
        int(partition_tokens), int(kernel), PA_DECODE_SHARED_BLOCKS if shared_blocks else 0,
        None if ws is None else ws.data_ptr(), ws_bytes, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_append")
    return out


def pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                            max_blocks_per_seq, dtype_code, prefix_blocks):
    out = ctypes.c_size_t(0)
    st = lib().pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                       max_blocks_per_seq, dtype_code, prefix_blocks,
                                                       ctypes.byref(out))
    if st != PA_OK:
        raise PaError(st, "pa_decode_shared_prefix_workspace_bytes")
    return out.value


def pa_decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens, scale, prefix_blocks, *,
                            num_blocks=None, layout=PA_LAYOUT_BHTD, workspace=None, stream=None):
    """pa_decode_ex for tables that all start with the same prefix_blocks blocks (read once for the batch)."""
    torch = _torch()
    code = _dtype_code(q)
    S, Hq, D = q.shape
    NB, bs, Hkv, D2 = cache_dims(k_cache, layout)
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, out and the caches")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    MB = block_tables.shape[1]
    nbytes = pa_decode_shared_prefix_workspace_bytes(S, Hq, Hkv, D, bs, MB, code, int(prefix_blocks))
    ws, ws_bytes = _workspace(q, nbytes, workspace)
    st = lib().pa_decode_shared_prefix(
        _dev(out, "out", q.dtype), _dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        S, Hq, Hkv, D, bs, MB, NB if num_blocks is None else int(num_blocks), int(prefix_blocks), float(scale), code,
        int(layout), None if ws is None else ws.data_ptr(), ws_bytes, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_shared_prefix")
    return out


def pa_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len, scale, *,
               num_blocks=None, layout=PA_LAYOUT_BHTD, shared_blocks=False, stream=None):
    """out[total_q, Hq, D] <- causal paged attention of the q rows of every sequence (query_start [S + 1])."""
    torch = _torch()
    code = _dtype_code(q)
    TQ, Hq, D = q.shape
    NB, bs, Hkv, D2 = cache_dims(k_cache, layout)
    S = context_lens.shape[0]
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, out and the caches")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(query_start.shape) != (S + 1,):
        raise ValueError("block_tables must be [S, MB] and query_start [S + 1]")
    st = lib().pa_prefill(
        _dev(out, "out", q.dtype), _dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        _dev(query_start, "query_start", torch.int32), S, TQ, int(max_query_len), Hq, Hkv, D, bs,
        block_tables.shape[1], NB if num_blocks is None else int(num_blocks), float(scale), code, int(layout),
        PA_DECODE_SHARED_BLOCKS if shared_blocks else 0, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_prefill")
    return out


def pa_prefill_shared_prefix_workspace_bytes(total_q, num_q_heads, head_dim, block_size, prefix_blocks):
    out = ctypes.c_size_t(0)
    st = lib().pa_prefill_shared_prefix_workspace_bytes(total_q, num_q_heads, head_dim, block_size, prefix_blocks,
                                                        ctypes.byref(out))
    if st != PA_OK:
        raise PaError(st, "pa_prefill_shared_prefix_workspace_bytes")
    return out.value


def pa_prefill_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len,
                             scale, prefix_blocks, *, num_blocks=None, layout=PA_LAYOUT_BHTD, workspace=None,
                             stream=None):
    """pa_prefill for tables that all start with the same prefix_blocks blocks (their K/V read once for every
    sequence's rows)."""
    torch = _torch()
    code = _dtype_code(q)
    TQ, Hq, D = q.shape
    NB, bs, Hkv, D2 = cache_dims(k_cache, layout)
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, out and the caches")
    S = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(query_start.shape) != (S + 1,):
        raise ValueError("block_tables must be [S, MB], context_lens [S] and query_start [S + 1]")
    nbytes = pa_prefill_shared_prefix_workspace_bytes(TQ, Hq, D, bs, int(prefix_blocks))
    ws, ws_bytes = _workspace(q, nbytes, workspace)
    st = lib().pa_prefill_shared_prefix(
        _dev(out, "out", q.dtype), _dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        _dev(query_start, "query_start", torch.int32), S, TQ, int(max_query_len), Hq, Hkv, D, bs,
        block_tables.shape[1], NB if num_blocks is None else int(num_blocks), int(prefix_blocks), float(scale), code,
        int(layout), None if ws is None else ws.data_ptr(), ws_bytes, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_prefill_shared_prefix")
    return out


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, *, workspace=None, stream=None):
    """pa_decode: cache layout [NB, Hkv, bs, D], library-chosen partition, unchecked table entries."""
    torch = _torch()
    code = _dtype_code(q)
    S, Hq, D = q.shape
    NB, bs, Hkv, D2 = cache_dims(k_cache, PA_LAYOUT_BHTD)
    MB = block_tables.shape[1]
    nbytes = pa_decode_workspace_bytes(S, Hq, Hkv, D, bs, MB, code, 0)
    ws, ws_bytes = _workspace(q, nbytes, workspace)
    st = lib().pa_decode(
        _dev(out, "out", q.dtype), _dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        S, Hq, Hkv, D, bs, MB, float(scale), code, None if ws is None else ws.data_ptr(), ws_bytes,
        _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode")
    return out


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, *, stream=None):
    """pa_decode_noalloc: pa_decode with the library's own scratch instead of a workspace (allocates nothing)."""
    torch = _torch()
    code = _dtype_code(q)
    S, Hq, D = q.shape
    NB, bs, Hkv, D2 = cache_dims(k_cache, PA_LAYOUT_BHTD)
    st = lib().pa_decode_noalloc(
        _dev(out, "out", q.dtype), _dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        S, Hq, Hkv, D, bs, block_tables.shape[1], float(scale), code, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_noalloc")
    return out


def pa_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, *, layout=PA_LAYOUT_BHTD, stream=None):
    """Write k, v [T, Hkv, D] into their slots of the caches (in place)."""
    torch = _torch()
    code = _dtype_code(k)
    T, Hkv, D = k.shape
    NB, bs, Hkv2, D2 = cache_dims(k_cache, layout)
    if (Hkv2, D2) != (Hkv, D) or tuple(v.shape) != tuple(k.shape) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between k/v and the caches")
    if tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be [T]")
    st = lib().pa_reshape_and_cache(
        _dev(k, "k"), _dev(v, "v", k.dtype), _dev(k_cache, "k_cache", k.dtype), _dev(v_cache, "v_cache", k.dtype),
        _dev(slot_mapping, "slot_mapping", torch.int64), T, Hkv, D, bs, NB, code, int(layout), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_reshape_and_cache")
    return k_cache, v_cache


def pa_probe_stream_read(buf, sink, workgroups: int, mode: int = 0, *, stream=None):
    """Read the whole of `buf` (a device tensor) once; sink (uint32/int32, >= workgroups) gets one XOR per workgroup."""
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda or sink.numel() < workgroups:
        raise ValueError("buf and sink must be contiguous device tensors, sink holding one word per workgroup")
    st = lib().pa_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                    int(workgroups), int(mode), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_probe_stream_read")


def to_layout(cache_bthd, layout: int):
    """Rearrange a cache given in [NB, bs, Hkv, D] into `layout` (a copy for BHTD)."""
    if layout == PA_LAYOUT_BTHD:
        return cache_bthd.contiguous()
    return cache_bthd.permute(0, 2, 1, 3).contiguous()


def from_layout(cache, layout: int):
    """Inverse of to_layout: back to [NB, bs, Hkv, D]."""
    if layout == PA_LAYOUT_BTHD:
        return cache.contiguous()
    return cache.permute(0, 2, 1, 3).contiguous()


# ---------------------------------------------------------------------------
# block copies and the host block manager (include/pa_blocks.h)
# ---------------------------------------------------------------------------
def _pool(t, name, dtype):
    """A pool tensor: device memory, or pinned host memory the device can address."""
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _pairs(pairs):
    torch = _torch()
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [n, 2]")
    return _pool(pairs, "pairs", torch.int32), pairs.shape[0]


def copy_blocks(k_cache, v_cache, pairs, *, layout=PA_LAYOUT_BHTD, stream=None):
    """pa_copy_blocks: block pairs[i, 1] of both pools takes block pairs[i, 0]."""
    NB, bs, Hkv, D = cache_dims(k_cache, layout)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache differ in shape")
    ptr, n = _pairs(pairs)
    st = lib().pa_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache", k_cache.dtype), ptr, n, NB, bs, Hkv,
                              D, _dtype_code(k_cache), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_copy_blocks")


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs, *, layout=PA_LAYOUT_BHTD, stream=None):
    """pa_swap_blocks: block pairs[i, 1] of the destination pools takes block pairs[i, 0] of the source pools.
    Either pool pair may be device memory or pinned host memory."""
    NBd, bs, Hkv, D = cache_dims(dst_k, layout)
    NBs, bs2, Hkv2, D2 = cache_dims(src_k, layout)
    if (bs, Hkv, D) != (bs2, Hkv2, D2) or dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise ValueError("the pools differ in block shape")
    dt = dst_k.dtype
    ptr, n = _pairs(pairs)
    st = lib().pa_swap_blocks(_pool(dst_k, "dst_k", dt), _pool(dst_v, "dst_v", dt), _pool(src_k, "src_k", dt),
                              _pool(src_v, "src_v", dt), ptr, n, NBd, NBs, bs, Hkv, D, _dtype_code(dst_k),
                              _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_swap_blocks")


class BlockManager:
    """The host block manager (pa_bm_*): tables, reference counts and free blocks of a GPU and a CPU pool."""

    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int, block_size: int):
        h = ctypes.c_void_p()
        st = lib().pa_bm_create(num_gpu_blocks, num_cpu_blocks, block_size, ctypes.byref(h))
        if st != PA_OK:
            raise PaError(st, "pa_bm_create")
        self._h = h
        self.block_size = block_size

    def close(self):
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _call(self, name, *args):
        st = getattr(lib(), name)(self._h, *args)
        if st != PA_OK:
            raise PaError(st, name)

    def add(self, seq: int):
        self._call("pa_bm_add", seq)

    def fork(self, parent: int, child: int):
        self._call("pa_bm_fork", parent, child)

    def blocks_needed(self, seq: int, n: int) -> int:
        out = ctypes.c_int32(0)
        self._call("pa_bm_blocks_needed", seq, n, ctypes.byref(out))
        return out.value

    def append(self, seq: int, n: int):
        """(slot of each new token, [(src, dst)] block copies to run first)."""
        slots = (ctypes.c_int64 * max(n, 1))()
        copies = (ctypes.c_int32 * 2)()
        nc = ctypes.c_int32(0)
        self._call("pa_bm_append", seq, n, slots, copies, 1, ctypes.byref(nc))
        return list(slots[:n]), [(copies[2 * i], copies[2 * i + 1]) for i in range(nc.value)]

    @staticmethod
    def _tokens(tokens):
        import numpy as np
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).astype(np.int32)).reshape(-1)
        return t, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def append_tokens(self, seq: int, tokens):
        """append() with the token ids given, so that the blocks they fill can be cached."""
        import numpy as np
        keep, toks = self._tokens(tokens)
        n = keep.size
        slots = np.empty(max(n, 1), dtype=np.int64)
        copies = (ctypes.c_int32 * 2)()
        nc = ctypes.c_int32(0)
        self._call("pa_bm_append_tokens", seq, toks, n, slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                   copies, 1, ctypes.byref(nc))
        return slots[:n].tolist(), [(copies[2 * i], copies[2 * i + 1]) for i in range(nc.value)]

    def add_cached(self, seq: int, prompt) -> int:
        """A new request whose table starts with the cached blocks `prompt` begins
        with; returns the prompt tokens already cached."""
        keep, toks = self._tokens(prompt)
        hit = ctypes.c_int32(0)
        self._call("pa_bm_add_cached", seq, toks, keep.size, ctypes.byref(hit))
        return hit.value

    def cache_stats(self):
        """(cached GPU blocks, cached blocks no request holds)."""
        c, e = ctypes.c_int32(0), ctypes.c_int32(0)
        self._call("pa_bm_cache_stats", ctypes.byref(c), ctypes.byref(e))
        return c.value, e.value

    def free(self, seq: int):
        self._call("pa_bm_free", seq)

    def _move(self, name, seq):
        _, nb, _ = self.info(seq)
        pairs = (ctypes.c_int32 * max(2 * nb, 2))()
        n = ctypes.c_int32(0)
        self._call(name, seq, pairs, nb, ctypes.byref(n))
        return [(pairs[2 * i], pairs[2 * i + 1]) for i in range(n.value)]

    def swap_out(self, seq: int):
        """[(gpu block, cpu block)] to copy from the GPU pools to the CPU pools."""
        return self._move("pa_bm_swap_out", seq)

    def swap_in(self, seq: int):
        """[(cpu block, gpu block)] to copy from the CPU pools to the GPU pools."""
        return self._move("pa_bm_swap_in", seq)

    def block_tables(self, seqs, max_blocks: int):
        """(int32 [len(seqs), max_blocks] tables, -1 past the end; int32 [len(seqs)] lengths) as numpy arrays."""
        import numpy as np
        n = len(seqs)
        ids = (ctypes.c_int64 * max(n, 1))(*seqs)
        tables = np.empty((n, max_blocks), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        self._call("pa_bm_block_tables", ids, n, max_blocks,
                   tables.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                   lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
        return tables, lens

    def num_free(self, pool: int = POOL_GPU) -> int:
        out = ctypes.c_int32(0)
        self._call("pa_bm_num_free", pool, ctypes.byref(out))
        return out.value

    def ref_count(self, pool: int, block: int) -> int:
        out = ctypes.c_int32(0)
        self._call("pa_bm_ref_count", pool, block, ctypes.byref(out))
        return out.value

    def info(self, seq: int):
        """(tokens, blocks, on the GPU)."""
        t, b, g = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
        self._call("pa_bm_info", seq, ctypes.byref(t), ctypes.byref(b), ctypes.byref(g))
        return t.value, b.value, bool(g.value)
