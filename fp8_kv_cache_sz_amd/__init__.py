"""SplitZip lossless KV-cache codec for MI355X (gfx950).

Thin Python layer over the C ABI of ``libsplitzip.so`` (include/splitzip.h):
it only moves pointers, sizes and streams; calibration, encode and decode all
run in the library.  Tensors:

* BF16 data: ``torch.bfloat16`` (or ``int16``) tensors.
* FP8 E5M2 data: ``torch.float8_e5m2`` or ``uint8`` tensors of raw bytes.
* Streams: ``uint8`` device tensors.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _native
from ._native import (SZ_BF16, SZ_FP8_E5M2, SZ_FORMAT_TOP16, SZ_FORMAT_TOP8, SZ_FORMAT_TOP15_SENTINEL,
                      SplitZipError)

BF16 = SZ_BF16
E5M2 = SZ_FP8_E5M2
# stream formats: the page's Top-16 design and its two ablation alternatives (BF16 only)
TOP16 = SZ_FORMAT_TOP16
TOP8 = SZ_FORMAT_TOP8
TOP15S = SZ_FORMAT_TOP15_SENTINEL

__all__ = ["BF16", "E5M2", "TOP16", "TOP8", "TOP15S", "Codebook", "SplitZipError", "calibrate", "calibrate_device",
           "codebook_from_device", "encoded_size", "workspace_size", "workspace", "decode_workspace_size",
           "decode_workspace", "encode", "decode",
           "read_escape_count", "transfer", "transfer_buffers", "reference_copy", "reference_split",
           "reference_join", "profile_enable",
           "profile_collect"]

# An sz_codebook in device memory: u32 dtype, 16 exponent bytes (20 bytes,
# padded to 32 so that the tensor size keeps 16-byte multiples).
DEVICE_CODEBOOK_BYTES = 32


@dataclass(frozen=True)
class Codebook:
    """Top-16 exponent codebook: ``exps[c]`` is the exponent coded as ``c``."""
    dtype: int
    exps: tuple

    def to_c(self) -> _native.sz_codebook:
        cb = _native.sz_codebook()
        cb.dtype = self.dtype
        for c, e in enumerate(self.exps):
            cb.exp[c] = int(e)
        return cb


def dtype_of(t: torch.Tensor) -> int:
    if t.dtype in (torch.bfloat16, torch.int16):
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e5m2):
        return E5M2
    raise TypeError("SplitZip codes BF16 (bfloat16/int16) or FP8 E5M2 (float8_e5m2/uint8) tensors, "
                    "got %s" % t.dtype)


def _elem_size(dtype: int) -> int:
    return 2 if dtype == BF16 else 1


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _side_stream(stream, device):
    """The caller's stream when it is not the current one, else None.  On a
    side stream the tensors this layer allocates are marked as used by it
    (record_stream), and host reads of results wait for it first."""
    if stream is None or stream == torch.cuda.current_stream(device):
        return None
    return stream


def _adopt(side, device, tensors) -> None:
    """Before a launch on a side stream: memory this layer just took from the
    current stream's pool may still be in use by work queued there, so the
    side stream waits for that work."""
    if side is not None and any(t is not None for t in tensors):
        side.wait_stream(torch.cuda.current_stream(device))


def _owned_by(side, *tensors) -> None:
    if side is not None:
        for t in tensors:
            if t is not None:
                t.record_stream(side)


def _before_host_read(side) -> None:
    if side is not None:
        side.synchronize()


def calibrate(t: torch.Tensor) -> Codebook:
    """Offline Top-16 calibration on the host (sz_calibrate)."""
    dtype = dtype_of(t)
    h = t.detach().reshape(-1).contiguous().cpu()
    cb = _native.sz_calibrate(dtype, h.data_ptr() if h.numel() else None, h.numel())
    return Codebook(dtype, tuple(int(x) for x in cb.exp))


def calibrate_device(t: torch.Tensor, sample_every: int = 1, out: torch.Tensor | None = None,
                     hist: bool = False, ws: torch.Tensor | None = None, stream=None):
    """On-device Top-16 calibration (sz_calibrate_device) over the 64K blocks
    0, s, 2s, ... of a device tensor.  Returns the codebook as a uint8 device
    tensor in sz_codebook layout, usable by ``encode`` without a host round
    trip; with ``hist=True`` returns ``(codebook, uint64 counts)``."""
    dtype = dtype_of(t)
    t = t.reshape(-1)
    if not t.is_contiguous():
        raise ValueError("calibrate_device needs a contiguous tensor")
    n = t.numel()
    side = _side_stream(stream, t.device)
    owned = []
    if out is None:
        out = torch.zeros(DEVICE_CODEBOOK_BYTES, dtype=torch.uint8, device=t.device)
        owned.append(out)
    h = torch.empty(256 if dtype == BF16 else 32, dtype=torch.int64, device=t.device) if hist else None
    owned.append(h)
    if ws is None:
        ws = torch.empty(_native.sz_calibrate_workspace_size(dtype), dtype=torch.uint8, device=t.device)
        owned.append(ws)
    _adopt(side, t.device, owned)       # also orders the zero fill of `out`
    rc = _native.sz_calibrate_device(dtype, t.data_ptr() if n else None, n, sample_every, out.data_ptr(),
                                     h.data_ptr() if h is not None else None, ws.data_ptr(), ws.numel(),
                                     _stream_handle(stream, t.device))
    _native.check("sz_calibrate_device", rc)
    _owned_by(side, *owned)
    return (out, h) if hist else out


def codebook_from_device(d_cb: torch.Tensor) -> Codebook:
    """Reads a device codebook (sz_codebook layout) back to the host."""
    raw = d_cb[:20].cpu()
    return Codebook(int(raw[:4].view(torch.int32)[0]), tuple(int(x) for x in raw[4:20]))


def encoded_size(dtype: int, n: int, n_escapes: int, fmt: int = TOP16) -> int:
    if fmt == TOP16:
        return _native.sz_encoded_size(dtype, n, n_escapes)
    return _native.sz_encoded_size_format(fmt, dtype, n, n_escapes)


def workspace_size(dtype: int, n: int, fmt: int = TOP16) -> int:
    """Bytes of encode workspace (sz_workspace_size / sz_workspace_size_format)."""
    if fmt == TOP16:
        return _native.sz_workspace_size(dtype, n)
    return _native.sz_workspace_size_format(fmt, dtype, n)


def decode_workspace_size(dtype: int, n: int) -> int:
    """Bytes of decode workspace (sz_decode_workspace_size)."""
    return _native.sz_decode_workspace_size(dtype, n)


def workspace(dtype: int, n: int, device="cuda", fmt: int = TOP16) -> torch.Tensor:
    """An encode workspace (also large enough for decode)."""
    return torch.empty(workspace_size(dtype, n, fmt), dtype=torch.uint8, device=device)


def decode_workspace(dtype: int, n: int, device="cuda") -> torch.Tensor:
    return torch.empty(decode_workspace_size(dtype, n), dtype=torch.uint8, device=device)


def read_escape_count(buf: torch.Tensor) -> int:
    """E from a finished stream's header (u64 at byte 16); synchronises on the copy."""
    return int(buf[16:24].cpu().view(torch.int64)[0])


def encode(x: torch.Tensor, cb, out: torch.Tensor | None = None,
           ws: torch.Tensor | None = None, stream=None, sync: bool = True, fmt: int = TOP16):
    """Encode a device tensor with a host ``Codebook`` (sz_encode) or a device
    codebook tensor from ``calibrate_device`` (sz_encode_devcb).  Returns
    ``(buf, size, escapes)``; with ``sync=False`` the call only enqueues the
    kernels and returns ``(buf, None, None)`` (the size is known once the
    stream has run).  ``fmt`` selects an ablation format (TOP8, TOP15S; BF16
    with a host codebook only)."""
    dtype = dtype_of(x)
    on_device = isinstance(cb, torch.Tensor)
    if fmt != TOP16 and on_device:
        raise ValueError("the ablation formats take a host Codebook")
    if not on_device and cb.dtype != dtype:
        raise SplitZipError("sz_encode", -2)
    x = x.reshape(-1)
    if not x.is_contiguous():
        raise ValueError("encode needs a contiguous tensor")
    n = x.numel()
    cap = encoded_size(dtype, n, n, fmt)
    side = _side_stream(stream, x.device)
    owned = []
    if out is None:
        out = torch.empty(max(cap, 1), dtype=torch.uint8, device=x.device)
        owned.append(out)
    if ws is None:
        ws = workspace(dtype, n, x.device, fmt)
        owned.append(ws)
    _adopt(side, x.device, owned)
    if fmt != TOP16:
        rc = _native.sz_encode_format(fmt, dtype, x.data_ptr() if n else None, n, cb.to_c(), out.data_ptr(),
                                      out.numel(), ws.data_ptr(), ws.numel(), _stream_handle(stream, x.device))
        _native.check("sz_encode_format", rc)
    elif on_device:
        rc = _native.sz_encode_devcb(dtype, x.data_ptr() if n else None, n, cb.data_ptr(), out.data_ptr(),
                                     out.numel(), ws.data_ptr(), ws.numel(), _stream_handle(stream, x.device))
        _native.check("sz_encode_devcb", rc)
    else:
        rc = _native.sz_encode(dtype, x.data_ptr() if n else None, n, cb.to_c(), out.data_ptr(),
                               out.numel(), ws.data_ptr(), ws.numel(), _stream_handle(stream, x.device))
        _native.check("sz_encode", rc)
    _owned_by(side, *owned)
    if not sync:
        return out, None, None
    _before_host_read(side)
    if on_device:
        status = int(ws[:4].cpu().view(torch.int32)[0])
        if status != 0:
            raise SplitZipError("sz_encode_devcb (device codebook check)", status)
    escapes = read_escape_count(out)
    return out, encoded_size(dtype, n, escapes, fmt), escapes


def decode(buf: torch.Tensor, dtype: int, n: int, out: torch.Tensor | None = None,
           ws: torch.Tensor | None = None, stream=None, check: bool = True,
           in_bytes: int | None = None, fmt: int = TOP16) -> torch.Tensor:
    """Decode a device stream into ``n`` values.  With ``check`` the call
    synchronises and raises if the device-side validation failed."""
    side = _side_stream(stream, buf.device)
    owned = []
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16 if dtype == BF16 else torch.uint8, device=buf.device)
        owned.append(out)
    if out.numel() * out.element_size() < n * _elem_size(dtype):
        raise ValueError("output tensor too small")
    if ws is None:
        ws = decode_workspace(dtype, n, buf.device)
        owned.append(ws)
    _adopt(side, buf.device, owned)
    nbytes = buf.numel() if in_bytes is None else in_bytes
    if fmt != TOP16:
        rc = _native.sz_decode_format(fmt, buf.data_ptr(), nbytes, dtype, out.data_ptr() if n else None, n,
                                      ws.data_ptr(), ws.numel(), _stream_handle(stream, buf.device))
        _native.check("sz_decode_format", rc)
    else:
        rc = _native.sz_decode(buf.data_ptr(), nbytes, dtype, out.data_ptr() if n else None, n,
                               ws.data_ptr(), ws.numel(), _stream_handle(stream, buf.device))
        _native.check("sz_decode", rc)
    _owned_by(side, *owned)
    if check:
        _before_host_read(side)
        status = int(ws[:4].cpu().view(torch.int32)[0])
        if status != 0:
            raise SplitZipError("sz_decode (device check)", status)
    return out


def transfer_buffers(dtype: int, n: int, chunk: int, depth: int = 3, device="cuda"):
    """Pinned host staging and device workspace for ``transfer``."""
    h = torch.empty(_native.sz_transfer_host_bytes(dtype, n, chunk, depth), dtype=torch.uint8, pin_memory=True)
    ws = torch.empty(_native.sz_transfer_workspace_size(dtype, chunk, depth), dtype=torch.uint8, device=device)
    return h, ws


def transfer(x: torch.Tensor, chunk: int, cb: Codebook | None = None, depth: int = 3,
             out: torch.Tensor | None = None, staging=None, stream=None):
    """Send a device tensor through pinned host memory in chunks of ``chunk``
    values (sz_transfer): SplitZip-compressed with ``cb``, or raw when ``cb``
    is None.  Synchronous.  Returns ``(out, stats)`` with stats a dict of the
    library's sz_transfer_stats."""
    dtype = dtype_of(x)
    x = x.reshape(-1)
    n = x.numel()
    if out is None:
        out = torch.empty_like(x)
    if staging is None:
        staging = transfer_buffers(dtype, n, chunk, depth, x.device)
    h, ws = staging
    rc, st = _native.sz_transfer(dtype, x.data_ptr() if n else None, n, chunk,
                                 cb.to_c() if cb is not None else None, 1 if cb is not None else 0, depth,
                                 h.data_ptr(), h.numel(), out.data_ptr() if n else None, ws.data_ptr(), ws.numel(),
                                 _stream_handle(stream, x.device))
    _native.check("sz_transfer", rc)
    stats = {k: getattr(st, k) for k, _ in st._fields_}
    if stats["decode_status"] != 0:
        raise SplitZipError("sz_transfer (chunk decode)", stats["decode_status"])
    return out, stats


def reference_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """The library's plain streaming copy (sz_reference_copy) of a contiguous
    device tensor into another of the same byte size; not part of the codec,
    it times the practical streaming ceiling."""
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("reference_copy needs contiguous tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("reference_copy needs tensors of the same byte size")
    rc = _native.sz_reference_copy(src.data_ptr() if nbytes else None, dst.data_ptr() if nbytes else None,
                                   nbytes, _stream_handle(stream, src.device))
    _native.check("sz_reference_copy", rc)
    return dst


def reference_split(x: torch.Tensor, stream=None):
    """The library's reference of the dense encoders' memory pattern
    (sz_reference_split) on a contiguous BF16 or E5M2-byte device tensor of
    whole 16K-element tiles; not part of the codec, it times the practical
    ceiling of the encoders' stream mix.  Returns (codes, sym) byte tensors."""
    dtype = dtype_of(x)
    if not x.is_contiguous():
        raise ValueError("reference_split needs a contiguous tensor")
    n = x.numel()
    codes = torch.empty(n // 2, dtype=torch.uint8, device=x.device)
    sym = torch.empty(n if dtype == SZ_BF16 else 3 * n // 8, dtype=torch.uint8, device=x.device)
    rc = _native.sz_reference_split(dtype, x.data_ptr() if n else None, n, codes.data_ptr() if n else None,
                                    sym.data_ptr() if n else None, _stream_handle(stream, x.device))
    _native.check("sz_reference_split", rc)
    return codes, sym


def reference_join(codes: torch.Tensor, sym: torch.Tensor, dtype: int, n: int, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """The library's reference of the span decoders' memory pattern
    (sz_reference_join): reads the code and sign/mantissa byte tensors of n
    elements (whole 16K tiles) and writes n elements; not part of the codec,
    it times the practical ceiling of the decoders' stream mix."""
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16 if dtype == BF16 else torch.uint8, device=codes.device)
    rc = _native.sz_reference_join(dtype, codes.data_ptr() if n else None, sym.data_ptr() if n else None, n,
                                   out.data_ptr() if n else None, _stream_handle(stream, codes.device))
    _native.check("sz_reference_join", rc)
    return out


def profile_enable(on: bool = True) -> None:
    _native.check("sz_profile_enable", _native.sz_profile_enable(on))


def profile_collect() -> dict:
    """{kernel name: (launches, total ms)} since the last collect/enable."""
    return _native.sz_profile_collect()
