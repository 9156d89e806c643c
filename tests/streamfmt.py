"""Test-side reader for the v1 SplitZip stream layout.

Reads fields out of a stream (numpy uint8) so tests can check invariants.  It
is independent of both the oracle and the HIP library: it only knows where
the format puts each section.
"""
from __future__ import annotations

import numpy as np

BLOCK = 65536


def _a256(x: int) -> int:
    return (x + 255) // 256 * 256


def layout(dtype: int, n: int) -> dict:
    nb = (n + BLOCK - 1) // BLOCK
    off_nib = _a256(64 + 4 * nb)
    nib_bytes = (n + 1) // 2
    off_sm = off_nib + _a256(nib_bytes)
    sm_bytes = n if dtype == 0 else 3 * ((n + 7) // 8)
    off_esc = off_sm + _a256(sm_bytes)
    return dict(nb=nb, off_nib=off_nib, nib_bytes=nib_bytes, off_sm=off_sm,
                sm_bytes=sm_bytes, off_esc=off_esc)


def header(stream: np.ndarray) -> dict:
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    return dict(
        magic=int(s[0:4].view("<u4")[0]),
        version=int(s[4:6].view("<u2")[0]),
        dtype=int(s[6]),
        log2_block=int(s[7]),
        n=int(s[8:16].view("<u8")[0]),
        escapes=int(s[16:24].view("<u8")[0]),
        nb=int(s[24:28].view("<u4")[0]),
        reserved=int(s[28:32].view("<u4")[0]),
        codebook=s[32:48].copy(),
        zero48=s[48:64].copy(),
    )


def sections(stream: np.ndarray) -> dict:
    """All sections of a stream as numpy arrays."""
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    h = header(s)
    L = layout(h["dtype"], h["n"])
    n, e = h["n"], h["escapes"]
    counts = s[64:64 + 4 * L["nb"]].view("<u4").astype(np.int64)
    nib = s[L["off_nib"]:L["off_nib"] + L["nib_bytes"]]
    codes = np.empty(2 * nib.size, dtype=np.uint8)
    codes[0::2] = nib & 0xF
    codes[1::2] = nib >> 4
    sm_raw = s[L["off_sm"]:L["off_sm"] + L["sm_bytes"]]
    if h["dtype"] == 0:
        sm = sm_raw.copy()
    else:
        groups = sm_raw.reshape(-1, 3).astype(np.uint32)
        v = groups[:, 0] | (groups[:, 1] << 8) | (groups[:, 2] << 16)
        sm = ((v[:, None] >> (3 * np.arange(8, dtype=np.uint32))[None, :]) & 7).astype(np.uint8)
        sm = sm.reshape(-1)
    rec = s[L["off_esc"]:L["off_esc"] + 3 * e].reshape(-1, 3).astype(np.int64)
    pos = rec[:, 0] | (rec[:, 1] << 8)
    exp = rec[:, 2]
    return dict(header=h, layout=L, counts=counts, codes=codes[:n], tail_code=codes[n:],
                sm=sm[:n], sm_tail=sm[n:], pos=pos, exp=exp, size=L["off_esc"] + 3 * e)


def padding_ranges(stream: np.ndarray):
    """(start, end) byte ranges the format requires to be zero."""
    h = header(stream)
    L = layout(h["dtype"], h["n"])
    ranges = [(28, 32), (48, 64), (64 + 4 * L["nb"], L["off_nib"]),
              (L["off_nib"] + L["nib_bytes"], L["off_sm"]),
              (L["off_sm"] + L["sm_bytes"], L["off_esc"])]
    return [(a, b) for a, b in ranges if b > a]
