"""ctypes loader for ``pa_oracle.c`` -- TEST INFRASTRUCTURE ONLY.

The C file holds the arithmetic (fp64 paged decode attention, exact element
decoders, round-to-nearest-even to a storage type, and the append scatter);
this module only builds it with gcc, loads it and marshals numpy arrays.

Element storage convention shared with the synthetic-input generators: f32
arrays are ``numpy.float32``, f16 arrays are ``numpy.float16``, bf16 arrays
are ``numpy.uint16`` holding the raw bfloat16 bit patterns (numpy has no
bfloat16 type).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32, F16, BF16 = 0, 1, 2
ORACLE_DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
_STORAGE = {F32: np.float32, F16: np.float16, BF16: np.uint16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "libpa_oracle.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile pa_oracle.c with gcc (IEEE arithmetic: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.orc_paged_decode.restype = i32
            lib.orc_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp] + [i32] * 7 + [dbl, i32]
            lib.orc_reshape_and_cache.restype = i32
            lib.orc_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp] + [i32] * 6
            lib.orc_round_array.restype = None
            lib.orc_round_array.argtypes = [vp, i64, i32]
            lib.orc_decode_array.restype = None
            lib.orc_decode_array.argtypes = [vp, vp, i64, i32]
            lib.orc_f16_to_f64.restype = dbl
            lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
            lib.orc_bf16_to_f64.restype = dbl
            lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
            lib.orc_num_threads.restype = i32
            _lib = lib
    return _lib


def _dtype_code(dtype) -> int:
    if isinstance(dtype, str):
        return ORACLE_DTYPES[dtype]
    return int(dtype)


def _check(arr: np.ndarray, code: int, name: str) -> np.ndarray:
    want = _STORAGE[code]
    if arr.dtype != want:
        raise TypeError(f"{name}: expected storage {np.dtype(want)}, got {arr.dtype}")
    return np.ascontiguousarray(arr)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype) -> np.ndarray:
    """fp64 softmax(scale * q K^T) V over each sequence's paged context.

    q: [S, Hq, D]; k_cache, v_cache: [NB, block_size, Hkv, D] (the pages' layout);
    block_tables: [S, MB] int32; context_lens: [S] int32; scale: the value the
    GPU receives (an fp32 number, widened exactly).  Returns [S, Hq, D] float64.
    """
    code = _dtype_code(dtype)
    q = _check(q, code, "q")
    k_cache = _check(k_cache, code, "k_cache")
    v_cache = _check(v_cache, code, "v_cache")
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    S, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or bt.shape[0] != S or cl.shape != (S,):
        raise ValueError("shape mismatch")
    MB = bt.shape[1] if bt.ndim == 2 else 0
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rc = _load().orc_paged_decode(
        out.ctypes.data, q.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data,
        bt.ctypes.data, cl.ctypes.data, S, Hq, Hkv, D, bs, max(MB, 1), NB,
        float(scale), code)
    if rc != 0:
        raise ValueError("oracle rejected the arguments (bad table entry, context length or shape)")
    return out


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, dtype) -> None:
    """In-place scatter of k, v [T, Hkv, D] into [NB, bs, Hkv, D] caches at their slots."""
    code = _dtype_code(dtype)
    k = _check(k, code, "k")
    v = _check(v, code, "v")
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        if c.dtype != _STORAGE[code] or not c.flags.c_contiguous:
            raise TypeError(f"{name} must be a C-contiguous {np.dtype(_STORAGE[code])} array")
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T, Hkv, D = k.shape
    NB, bs, Hkv2, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or v.shape != k.shape or v_cache.shape != k_cache.shape or sm.shape != (T,):
        raise ValueError("shape mismatch")
    rc = _load().orc_reshape_and_cache(
        k.ctypes.data, v.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data,
        sm.ctypes.data, T, Hkv, D, bs, NB, code)
    if rc != 0:
        raise ValueError("oracle rejected the arguments (slot past the pool)")


def round_to_dtype(x, dtype) -> np.ndarray:
    """Round float64 values to the storage type (nearest, ties to even); returns float64."""
    code = _dtype_code(dtype)
    y = np.array(x, dtype=np.float64, copy=True, order="C")
    _load().orc_round_array(y.ctypes.data, y.size, code)
    return y


def decode_elements(arr, dtype) -> np.ndarray:
    """Exact float64 values of stored elements (f32 / f16 / bf16 bit patterns)."""
    code = _dtype_code(dtype)
    a = _check(np.asarray(arr), code, "arr")
    out = np.empty(a.shape, dtype=np.float64)
    _load().orc_decode_array(out.ctypes.data, a.ctypes.data, a.size, code)
    return out


def f16_bits_to_f64(u: int) -> float:
    return float(_load().orc_f16_to_f64(int(u)))


def bf16_bits_to_f64(u: int) -> float:
    return float(_load().orc_bf16_to_f64(int(u)))
