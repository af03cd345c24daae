"""ctypes wrapper of the bulk value fill in ``fill.c`` (input generation only)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_tgfill.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile fill.c with gcc (OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               os.path.join(_HERE, "fill.c"), "-o", tmp])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise RuntimeError(f"{_SO} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_SO)
        lib.tg_fill.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.tg_fill.restype = None
        lib.tg_fill_rows.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int64]
        lib.tg_fill_rows.restype = None
        lib.tg_fill_fp8.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                    ctypes.c_float]
        lib.tg_fill_fp8.restype = None
        lib.tg_fill_rows_fp8.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_float]
        lib.tg_fill_rows_fp8.restype = None
        _lib = lib
    return _lib


def fill_ptr(ptr: int, key: int, e0: int, n: int) -> None:
    """Write n bf16 values (elements e0..e0+n of stream ``key``) at address ptr."""
    _load().tg_fill(ctypes.c_void_p(ptr), key, e0, n)


def fill_array(out: np.ndarray, key: int, e0: int = 0) -> None:
    assert out.dtype == np.uint16 and out.flags.c_contiguous
    fill_ptr(out.ctypes.data, key, e0, out.size)


def rows(key: int, positions, dim: int) -> np.ndarray:
    pos = np.ascontiguousarray(positions, dtype=np.int64).reshape(-1)
    out = np.empty((pos.shape[0], dim), dtype=np.uint16)
    _load().tg_fill_rows(ctypes.c_void_p(out.ctypes.data), key, ctypes.c_void_p(pos.ctypes.data),
                         pos.shape[0], dim)
    return out


def fill_ptr_fp8(ptr: int, key: int, e0: int, n: int, scale: float) -> None:
    """Write n FP8 E4M3 codes (elements e0..e0+n of stream ``key`` / scale) at ptr."""
    _load().tg_fill_fp8(ctypes.c_void_p(ptr), key, e0, n, scale)


def rows_fp8(key: int, positions, dim: int, scale: float) -> np.ndarray:
    pos = np.ascontiguousarray(positions, dtype=np.int64).reshape(-1)
    out = np.empty((pos.shape[0], dim), dtype=np.uint8)
    _load().tg_fill_rows_fp8(ctypes.c_void_p(out.ctypes.data), key, ctypes.c_void_p(pos.ctypes.data),
                             pos.shape[0], dim, scale)
    return out
