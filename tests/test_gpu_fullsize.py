"""Full-size parity on the published workloads, through the same C-ABI calls
and launch configuration that bench.py times.

At these sizes the whole encoded stream is compared byte for byte with the
CPU oracle's stream of the whole tensor (the page's claim is bit-exact
reconstruction, and the format makes the stream a pure function of the input
and the codebook).  The GPU stream comes back to the host in slices, so host
memory holds the input, the oracle's stream and one slice.  Around that the
test keeps (1) a bit-exact decode back to the input and (2) properties
computed with plain torch ops, not the HIP path (escape count from the
exponent histogram, per-block escape counts).  On a mismatch the message
names the first differing byte, its section and its 64K block.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import streamfmt

pytestmark = pytest.mark.gpu

BLOCK = 65536
SLICE = 1 << 28          # bytes of the GPU stream brought to the host at a time


def _exponents(x, dtype):
    if dtype == 0:
        v = x.view(torch.int16).to(torch.int32) & 0xFFFF
        return (v >> 7) & 0xFF
    return (x.view(torch.uint8).to(torch.int32) >> 2) & 0x1F


def _where(dtype, n, counts, off):
    """Section, element or record, and block of byte `off` of a stream."""
    L = streamfmt.layout(dtype, n)
    if off < 64:
        return "header byte %d" % off
    if off < L["off_nib"]:
        return "block count %d" % ((off - 64) // 4)
    if off < L["off_sm"]:
        i = 2 * (off - L["off_nib"])
        return "code byte of elements %d-%d (block %d)" % (i, i + 1, i // BLOCK)
    if off < L["off_esc"]:
        i = off - L["off_sm"] if dtype == 0 else 8 * ((off - L["off_sm"]) // 3)
        return "sign/mantissa byte of element %d (block %d)" % (i, i // BLOCK)
    r = (off - L["off_esc"]) // 3
    b = int(np.searchsorted(np.cumsum(counts), r, side="right"))
    return "escape record %d (block %d)" % (r, b)


def assert_stream_equals_oracle(buf_dev, size, expect, dtype, n, counts):
    """buf_dev[:size] (device) == expect (host numpy), byte for byte."""
    assert size == expect.size, "stream size %d, oracle %d" % (size, expect.size)
    for lo in range(0, size, SLICE):
        hi = min(size, lo + SLICE)
        got = buf_dev[lo:hi].cpu().numpy()
        ref = expect[lo:hi]
        if not np.array_equal(got, ref):
            off = lo + int(np.flatnonzero(got != ref)[0])
            pytest.fail("stream differs from the oracle at byte %d (%s): GPU %d, oracle %d"
                        % (off, _where(dtype, n, counts, off), int(buf_dev[off]), int(expect[off])))


WORKLOADS = [
    ("kv1m", (0.0, 0.004)),
    ("llama3_8b_kv", (0.001, 0.003)),
    ("longctx_kv", (0.0003, 0.003)),
    ("stress_t3", (0.015, 0.05)),
    ("stress_oneexp", (0.0, 0.0)),
    ("stress_random", (0.93, 0.945)),
    ("llama3_8b_kv_e5m2", (0.0003, 0.004)),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,band", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_full_size_workload(name, band):
    import fp8_kv_cache_sz_amd as sz
    torch.cuda.empty_cache()
    print("full-size workload", name, flush=True)
    x, dtype = synth.workload(name, device="cuda")
    cal = synth.calibration_tensor(name)
    cb = sz.calibrate(cal)
    cbn = np.array(cb.exps, dtype=np.uint8)
    assert np.array_equal(cbn, oracle.calibrate(synth.as_bits_numpy(cal), dtype))
    n = x.numel()
    buf, size, escapes = sz.encode(x, cb)
    print("  n=%d escapes=%d rate=%.5f ratio=%.5f" % (n, escapes, escapes / n, n * (2 - dtype) / size),
          flush=True)
    # (1) bit-exact round trip
    y = sz.decode(buf[:size], dtype, n)
    assert torch.equal(y.view(torch.uint8), x.view(torch.uint8))
    del y
    # (2) properties computed with torch
    expo = _exponents(x, dtype)
    in_cb = torch.isin(expo, torch.tensor(cbn.astype(np.int32), device="cuda"))
    del expo
    escaped = (~in_cb).to(torch.int32)
    del in_cb
    assert escapes == int(escaped.sum())
    lo_rate, hi_rate = band
    assert lo_rate <= escapes / n <= hi_rate
    nb = (n + BLOCK - 1) // BLOCK
    per_block = torch.zeros(nb * BLOCK, dtype=torch.int32, device="cuda")
    per_block[:n] = escaped
    per_block = per_block.view(nb, BLOCK).sum(dim=1)
    del escaped
    counts_dev = buf[64:64 + 4 * nb].view(torch.int32)
    assert torch.equal(counts_dev, per_block)
    counts = per_block.cpu().numpy().astype(np.int64)
    del per_block
    hdr = streamfmt.header(buf[:64].cpu().numpy())
    assert (hdr["magic"], hdr["n"], hdr["escapes"], hdr["nb"]) == (0x50495A53, n, escapes, nb)
    assert size == oracle.encoded_size(dtype, n, escapes)
    # (3) the whole stream against the oracle's stream of the whole tensor
    bits = synth.as_bits_numpy(x)
    del x
    torch.cuda.empty_cache()
    print("  oracle encode of %d elements" % n, flush=True)
    expect = oracle.encode(bits, dtype, list(cb.exps))
    del bits
    print("  comparing %d stream bytes" % size, flush=True)
    assert_stream_equals_oracle(buf, size, expect, dtype, n, counts)
    del buf, expect
    torch.cuda.empty_cache()
