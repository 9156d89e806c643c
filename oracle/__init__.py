"""SplitZip CPU oracle -- test infrastructure only.

ctypes binding over ``splitzip_oracle.c``: a plain, slow, single-threaded
C definition of the SplitZip stream (gist.science summary page "SplitZip:
Ultra Fast Lossless KV Compression for Disaggregated LLM Serving", Method
section, encoding and decoding bullets).  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It shares no code with the HIP path and never imports
it.

Arrays are numpy: BF16 data as ``uint16``, E5M2 data as ``uint8``, streams
as ``uint8``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

BF16 = 0
E5M2 = 1

OK = 0
E_ARG = -1
E_DTYPE = -2
E_CAPACITY = -3
E_FORMAT = -5

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "splitzip_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (single-threaded, -O2) into liboracle.so."""
    stale = (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, _SRC]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    """The oracle library; SPLITZIP_ORACLE_LIB names another build of the
    same source to load instead (the sanitizer test's instrumented copy)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SPLITZIP_ORACLE_LIB") or build()
        L = ctypes.CDLL(path)
        u64, i64, vp, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.szo_encoded_size.argtypes = [i32, u64, u64]
        L.szo_encoded_size.restype = u64
        L.szo_histogram.argtypes = [i32, vp, u64, vp]
        L.szo_histogram.restype = i32
        L.szo_calibrate.argtypes = [i32, vp, u64, vp]
        L.szo_calibrate.restype = i32
        L.szo_count_escapes.argtypes = [i32, vp, u64, vp]
        L.szo_count_escapes.restype = u64
        L.szo_encode.argtypes = [i32, vp, u64, vp, vp, u64]
        L.szo_encode.restype = i64
        L.szo_validate.argtypes = [vp, u64, i32, u64]
        L.szo_validate.restype = i32
        L.szo_decode.argtypes = [vp, u64, i32, vp, u64]
        L.szo_decode.restype = i32
        L.szo_check_canonical.argtypes = [vp, u64, i32, u64]
        L.szo_check_canonical.restype = i32
        u32 = ctypes.c_uint32
        L.szo_encoded_size_variant.argtypes = [u32, u64, u64]
        L.szo_encoded_size_variant.restype = u64
        L.szo_count_escapes_variant.argtypes = [u32, vp, u64, vp]
        L.szo_count_escapes_variant.restype = u64
        L.szo_encode_variant.argtypes = [u32, vp, u64, vp, vp, u64]
        L.szo_encode_variant.restype = i64
        L.szo_validate_variant.argtypes = [u32, vp, u64, u64]
        L.szo_validate_variant.restype = i32
        L.szo_decode_variant.argtypes = [u32, vp, u64, vp, u64]
        L.szo_decode_variant.restype = i32
        _lib = L
    return _lib


def _elem_dtype(dtype: int):
    return np.uint16 if dtype == BF16 else np.uint8


def _as_input(data, dtype: int) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(data).reshape(-1))
    want = _elem_dtype(dtype)
    if a.dtype != want:
        a = a.view(want) if a.dtype.itemsize == np.dtype(want).itemsize else a.astype(want)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def encoded_size(dtype: int, n: int, n_escapes: int) -> int:
    return int(lib().szo_encoded_size(dtype, n, n_escapes))


def histogram(data, dtype: int) -> np.ndarray:
    a = _as_input(data, dtype)
    hist = np.zeros(256 if dtype == BF16 else 32, dtype=np.uint64)
    rc = lib().szo_histogram(dtype, _ptr(a), a.size, hist.ctypes.data_as(ctypes.c_void_p))
    if rc:
        raise ValueError("szo_histogram failed: %d" % rc)
    return hist


def calibrate(data, dtype: int) -> np.ndarray:
    a = _as_input(data, dtype)
    cb = np.zeros(16, dtype=np.uint8)
    rc = lib().szo_calibrate(dtype, _ptr(a), a.size, cb.ctypes.data_as(ctypes.c_void_p))
    if rc:
        raise ValueError("szo_calibrate failed: %d" % rc)
    return cb


def count_escapes(data, dtype: int, codebook) -> int:
    a = _as_input(data, dtype)
    cb = np.ascontiguousarray(codebook, dtype=np.uint8)
    return int(lib().szo_count_escapes(dtype, _ptr(a), a.size, cb.ctypes.data_as(ctypes.c_void_p)))


def encode(data, dtype: int, codebook, capacity: int | None = None) -> np.ndarray:
    """Encode; returns the stream (uint8 array of exactly the encoded size)."""
    a = _as_input(data, dtype)
    cb = np.ascontiguousarray(codebook, dtype=np.uint8)
    if cb.size != 16:
        raise ValueError("codebook must have 16 entries")
    if capacity is None:
        capacity = encoded_size(dtype, a.size, count_escapes(a, dtype, cb))
    out = np.empty(max(capacity, 1), dtype=np.uint8)
    size = lib().szo_encode(dtype, _ptr(a), a.size, cb.ctypes.data_as(ctypes.c_void_p),
                            out.ctypes.data_as(ctypes.c_void_p), capacity)
    if size < 0:
        raise ValueError("szo_encode failed: %d" % size)
    return out[:size]


def encode_rc(data, dtype: int, codebook, capacity: int) -> int:
    """Raw return code of szo_encode (size or negative error)."""
    a = _as_input(data, dtype)
    cb = np.ascontiguousarray(codebook, dtype=np.uint8)
    out = np.empty(max(capacity, 1), dtype=np.uint8)
    return int(lib().szo_encode(dtype, _ptr(a), a.size, cb.ctypes.data_as(ctypes.c_void_p),
                                out.ctypes.data_as(ctypes.c_void_p), capacity))


def decode_rc(stream, dtype: int, n: int):
    """Decode; returns (rc, values)."""
    s = np.ascontiguousarray(stream, dtype=np.uint8).reshape(-1)
    out = np.zeros(max(n, 1), dtype=_elem_dtype(dtype))
    rc = lib().szo_decode(_ptr(s), s.size, dtype, out.ctypes.data_as(ctypes.c_void_p), n)
    return int(rc), out[:n]


def decode(stream, dtype: int, n: int) -> np.ndarray:
    rc, out = decode_rc(stream, dtype, n)
    if rc:
        raise ValueError("szo_decode failed: %d" % rc)
    return out


def validate(stream, dtype: int, n: int) -> int:
    s = np.ascontiguousarray(stream, dtype=np.uint8).reshape(-1)
    return int(lib().szo_validate(_ptr(s), s.size, dtype, n))


def check_canonical(stream, dtype: int, n: int) -> int:
    s = np.ascontiguousarray(stream, dtype=np.uint8).reshape(-1)
    return int(lib().szo_check_canonical(_ptr(s), s.size, dtype, n))


# ---------------------------------------------------------------------------
# Ablation variants, BF16 only: version 2 = Top-8 (3-bit codes + position
# records), version 3 = Top-15 with code 15 as escape sentinel (exponent
# bytes, no positions).  Version 1 is the Top-16 format above.
# ---------------------------------------------------------------------------
TOP16, TOP8, TOP15S = 1, 2, 3
BOOK_ENTRIES = {TOP16: 16, TOP8: 8, TOP15S: 15}


def encoded_size_variant(version: int, n: int, n_escapes: int) -> int:
    return int(lib().szo_encoded_size_variant(version, n, n_escapes))


def count_escapes_variant(version: int, data, codebook) -> int:
    a = _as_input(data, BF16)
    cb = np.ascontiguousarray(codebook, dtype=np.uint8)
    return int(lib().szo_count_escapes_variant(version, _ptr(a), a.size, cb.ctypes.data_as(ctypes.c_void_p)))


def encode_variant(data, version: int, codebook, capacity: int | None = None) -> np.ndarray:
    """Encode BF16 bits in format `version`; returns the stream."""
    a = _as_input(data, BF16)
    cb = np.zeros(16, dtype=np.uint8)
    cb[:len(codebook)] = np.asarray(codebook, dtype=np.uint8)
    if capacity is None:
        capacity = encoded_size_variant(version, a.size, count_escapes_variant(version, a, cb))
    out = np.zeros(max(capacity, 1), dtype=np.uint8)
    rc = lib().szo_encode_variant(version, _ptr(a), a.size, cb.ctypes.data_as(ctypes.c_void_p),
                                  out.ctypes.data_as(ctypes.c_void_p), capacity)
    if rc < 0:
        raise ValueError("szo_encode_variant failed: %d" % rc)
    return out[:rc]


def validate_variant(stream, version: int, n: int) -> int:
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    return int(lib().szo_validate_variant(version, _ptr(s), s.size, n))


def decode_variant_rc(stream, version: int, n: int):
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    out = np.zeros(max(n, 1), dtype=np.uint16)
    rc = lib().szo_decode_variant(version, _ptr(s), s.size, out.ctypes.data_as(ctypes.c_void_p), n)
    return rc, out[:n]


def decode_variant(stream, version: int, n: int) -> np.ndarray:
    rc, out = decode_variant_rc(stream, version, n)
    if rc:
        raise ValueError("szo_decode_variant failed: %d" % rc)
    return out
