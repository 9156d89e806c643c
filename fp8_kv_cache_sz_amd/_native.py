"""ctypes binding of libsplitzip.so (the C ABI declared in include/splitzip.h).

Argument marshalling only: every step of the codec runs in the library.
PyTorch provides device memory and streams.  There is no fallback: if the
library is missing or cannot be loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so the library binds to the HIP runtime torch already uses

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.environ.get("SPLITZIP_LIB", os.path.join(HERE, "libsplitzip.so"))

if not os.path.exists(LIBRARY):
    raise ImportError(
        "libsplitzip.so not found at %s; build it with `python fp8_kv_cache_sz_amd/build.py` "
        "(or __graft_entry__.build())" % LIBRARY)

lib = ctypes.CDLL(LIBRARY)

SZ_BF16 = 0
SZ_FP8_E5M2 = 1

ERRORS = {
    0: "SZ_OK", -1: "SZ_E_ARG", -2: "SZ_E_DTYPE", -3: "SZ_E_CAPACITY", -4: "SZ_E_ALIGN",
    -5: "SZ_E_FORMAT", -6: "SZ_E_HIP", -7: "SZ_E_WORKSPACE", -8: "SZ_E_SCRATCH",
}


class sz_codebook(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_uint32), ("exp", ctypes.c_uint8 * 16)]


class sz_transfer_stats(ctypes.Structure):
    _fields_ = [("total_ms", ctypes.c_double), ("chunks", ctypes.c_uint64), ("raw_bytes", ctypes.c_uint64),
                ("wire_bytes", ctypes.c_uint64), ("escapes", ctypes.c_uint64), ("decode_status", ctypes.c_int32)]


class sz_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_uint64),
                ("total_ms", ctypes.c_double)]


_u64, _i32, _vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p

lib.sz_calibrate.argtypes = [_i32, _vp, _u64, ctypes.POINTER(sz_codebook)]
lib.sz_calibrate.restype = _i32
lib.sz_encoded_size.argtypes = [_i32, _u64, _u64]
lib.sz_encoded_size.restype = _u64
lib.sz_workspace_size.argtypes = [_i32, _u64]
lib.sz_workspace_size.restype = _u64
lib.sz_workspace_size_format.argtypes = [_i32, _i32, _u64]
lib.sz_workspace_size_format.restype = _u64
lib.sz_decode_workspace_size.argtypes = [_i32, _u64]
lib.sz_decode_workspace_size.restype = _u64
lib.sz_encode.argtypes = [_i32, _vp, _u64, ctypes.POINTER(sz_codebook), _vp, _u64, _vp, _u64, _vp]
lib.sz_encode.restype = _i32
lib.sz_encode_devcb.argtypes = [_i32, _vp, _u64, _vp, _vp, _u64, _vp, _u64, _vp]
lib.sz_encode_devcb.restype = _i32
lib.sz_calibrate_workspace_size.argtypes = [_i32]
lib.sz_calibrate_workspace_size.restype = _u64
lib.sz_calibrate_device.argtypes = [_i32, _vp, _u64, _u64, _vp, _vp, _vp, _u64, _vp]
lib.sz_calibrate_device.restype = _i32
lib.sz_encoded_size_format.argtypes = [_i32, _i32, _u64, _u64]
lib.sz_encoded_size_format.restype = _u64
lib.sz_encode_format.argtypes = [_i32, _i32, _vp, _u64, ctypes.POINTER(sz_codebook), _vp, _u64, _vp, _u64, _vp]
lib.sz_encode_format.restype = _i32
lib.sz_decode_format.argtypes = [_i32, _vp, _u64, _i32, _vp, _u64, _vp, _u64, _vp]
lib.sz_decode_format.restype = _i32
lib.sz_transfer_workspace_size.argtypes = [_i32, _u64, _i32]
lib.sz_transfer_workspace_size.restype = _u64
lib.sz_transfer_host_bytes.argtypes = [_i32, _u64, _u64, _i32]
lib.sz_transfer_host_bytes.restype = _u64
lib.sz_transfer.argtypes = [_i32, _vp, _u64, _u64, _vp, _i32, _i32, _vp, _u64, _vp, _vp, _u64, _vp,
                            ctypes.POINTER(sz_transfer_stats)]
lib.sz_transfer.restype = _i32
lib.sz_decode.argtypes = [_vp, _u64, _i32, _vp, _u64, _vp, _u64, _vp]
lib.sz_decode.restype = _i32
lib.sz_decode_noalloc_max_elems.argtypes = []
lib.sz_decode_noalloc_max_elems.restype = _u64
lib.sz_decode_noalloc.argtypes = [_vp, _u64, _i32, _vp, _u64, _vp, _vp]
lib.sz_decode_noalloc.restype = _i32
lib.sz_profile_enable.argtypes = [_i32]
lib.sz_profile_enable.restype = _i32
lib.sz_profile_collect.argtypes = [ctypes.POINTER(sz_kernel_stat), _i32]
lib.sz_profile_collect.restype = _i32
lib.sz_reference_copy.argtypes = [_vp, _vp, _u64, _vp]
lib.sz_reference_copy.restype = _i32
lib.sz_reference_split.argtypes = [_i32, _vp, _u64, _vp, _vp, _vp]
lib.sz_reference_split.restype = _i32
lib.sz_reference_join.argtypes = [_i32, _vp, _vp, _u64, _vp, _vp]
lib.sz_reference_join.restype = _i32

EXPORTS = ("sz_calibrate", "sz_encoded_size", "sz_workspace_size", "sz_workspace_size_format",
           "sz_decode_workspace_size", "sz_encode", "sz_encode_devcb",
           "sz_calibrate_workspace_size", "sz_calibrate_device", "sz_decode", "sz_encoded_size_format",
           "sz_encode_format", "sz_decode_format", "sz_transfer_workspace_size", "sz_transfer_host_bytes",
           "sz_transfer", "sz_profile_enable", "sz_profile_collect", "sz_reference_copy",
           "sz_reference_split", "sz_reference_join", "sz_decode_noalloc_max_elems", "sz_decode_noalloc")

SZ_FORMAT_TOP16 = 1
SZ_FORMAT_TOP8 = 2
SZ_FORMAT_TOP15_SENTINEL = 3


class SplitZipError(RuntimeError):
    def __init__(self, call, code):
        super().__init__("%s failed: %s (%d)" % (call, ERRORS.get(code, "?"), code))
        self.code = code


def check(call, rc):
    if rc < 0:
        raise SplitZipError(call, rc)
    return rc


def sz_calibrate(dtype: int, host_ptr: int, n: int) -> sz_codebook:
    cb = sz_codebook()
    check("sz_calibrate", lib.sz_calibrate(dtype, host_ptr, n, ctypes.byref(cb)))
    return cb


def sz_encoded_size(dtype: int, n: int, n_escapes: int) -> int:
    return int(lib.sz_encoded_size(dtype, n, n_escapes))


def sz_workspace_size(dtype: int, n: int) -> int:
    return int(lib.sz_workspace_size(dtype, n))


def sz_workspace_size_format(fmt: int, dtype: int, n: int) -> int:
    return int(lib.sz_workspace_size_format(fmt, dtype, n))


def sz_decode_workspace_size(dtype: int, n: int) -> int:
    return int(lib.sz_decode_workspace_size(dtype, n))


def sz_encode(dtype, d_in, n, cb, d_out, out_capacity, d_ws, ws_bytes, stream) -> int:
    return int(lib.sz_encode(dtype, d_in, n, ctypes.byref(cb), d_out, out_capacity, d_ws, ws_bytes,
                             stream))


def sz_encode_devcb(dtype, d_in, n, d_cb, d_out, out_capacity, d_ws, ws_bytes, stream) -> int:
    return int(lib.sz_encode_devcb(dtype, d_in, n, d_cb, d_out, out_capacity, d_ws, ws_bytes, stream))


def sz_calibrate_workspace_size(dtype: int) -> int:
    return int(lib.sz_calibrate_workspace_size(dtype))


def sz_calibrate_device(dtype, d_in, n, sample_every, d_cb, d_hist, d_ws, ws_bytes, stream) -> int:
    return int(lib.sz_calibrate_device(dtype, d_in, n, sample_every, d_cb, d_hist, d_ws, ws_bytes, stream))


def sz_encoded_size_format(fmt: int, dtype: int, n: int, n_escapes: int) -> int:
    return int(lib.sz_encoded_size_format(fmt, dtype, n, n_escapes))


def sz_encode_format(fmt, dtype, d_in, n, cb, d_out, out_capacity, d_ws, ws_bytes, stream) -> int:
    return int(lib.sz_encode_format(fmt, dtype, d_in, n, ctypes.byref(cb), d_out, out_capacity, d_ws, ws_bytes,
                                    stream))


def sz_decode_format(fmt, d_in, in_bytes, dtype, d_out, n, d_ws, ws_bytes, stream) -> int:
    return int(lib.sz_decode_format(fmt, d_in, in_bytes, dtype, d_out, n, d_ws, ws_bytes, stream))


def sz_transfer_workspace_size(dtype: int, chunk: int, depth: int) -> int:
    return int(lib.sz_transfer_workspace_size(dtype, chunk, depth))


def sz_transfer_host_bytes(dtype: int, n: int, chunk: int, depth: int) -> int:
    return int(lib.sz_transfer_host_bytes(dtype, n, chunk, depth))


def sz_transfer(dtype, d_src, n, chunk, cb, compress, depth, h_staging, h_bytes, d_dst, d_ws, ws_bytes, stream):
    """Returns (rc, sz_transfer_stats)."""
    stats = sz_transfer_stats()
    rc = lib.sz_transfer(dtype, d_src, n, chunk, ctypes.byref(cb) if cb is not None else None, compress, depth,
                         h_staging, h_bytes, d_dst, d_ws, ws_bytes, stream, ctypes.byref(stats))
    return int(rc), stats


def sz_decode(d_in, in_bytes, dtype, d_out, n, d_ws, ws_bytes, stream) -> int:
    return int(lib.sz_decode(d_in, in_bytes, dtype, d_out, n, d_ws, ws_bytes, stream))


def sz_decode_noalloc_max_elems() -> int:
    return int(lib.sz_decode_noalloc_max_elems())


def sz_decode_noalloc(d_in, in_bytes, dtype, d_out, n, d_status, stream) -> int:
    return int(lib.sz_decode_noalloc(d_in, in_bytes, dtype, d_out, n, d_status, stream))


def sz_reference_copy(d_src, d_dst, nbytes, stream) -> int:
    return int(lib.sz_reference_copy(d_src, d_dst, nbytes, stream))


def sz_reference_split(dtype, d_in, n, d_codes, d_sym, stream) -> int:
    return int(lib.sz_reference_split(dtype, d_in, n, d_codes, d_sym, stream))


def sz_reference_join(dtype, d_codes, d_sym, n, d_out, stream) -> int:
    return int(lib.sz_reference_join(dtype, d_codes, d_sym, n, d_out, stream))


def sz_profile_enable(on: bool) -> int:
    return int(lib.sz_profile_enable(1 if on else 0))


def sz_profile_collect(max_stats: int = 32):
    stats = (sz_kernel_stat * max_stats)()
    count = check("sz_profile_collect", lib.sz_profile_collect(stats, max_stats))
    return {stats[i].name.decode(): (int(stats[i].launches), float(stats[i].total_ms))
            for i in range(count)}
