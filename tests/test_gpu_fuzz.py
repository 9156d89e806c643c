"""Seeded random cases through the C ABI against the oracle: sizes around
tile (16K) and block (64K) edges, escape densities from none to all,
random codebooks, both element types and all three formats.  Every case is
byte-exact on the stream and bit-exact on the decode."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

EDGES = [1, 7, 8, 9, 4095, 4096, 4097, 16383, 16384, 16385, 65535, 65536, 65537, 131071, 131073]


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = 0 if rng.random() < 0.6 else 1
    fmt = 1 if dtype == 1 else int(rng.choice([1, 1, 2, 3]))
    n = int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 300000))
    symbols = 256 if dtype == 0 else 32
    # exponents concentrated on a window, with a chosen share drawn from anywhere
    density = float(rng.choice([0.0, 1e-4, 1e-3, 0.02, 0.3, 0.9, 1.0]))
    centre = int(rng.integers(8, symbols - 8))
    width = int(rng.integers(2, 12))
    e = np.clip(rng.integers(centre - width, centre + width + 1, n), 0, symbols - 1)
    wild = rng.random(n) < density
    e[wild] = rng.integers(0, symbols, int(wild.sum()))
    if dtype == 0:
        bits = ((rng.integers(0, 2, n) << 15) | (e << 7) | rng.integers(0, 128, n)).astype(np.uint16)
    else:
        bits = ((rng.integers(0, 2, n) << 7) | (e << 2) | rng.integers(0, 4, n)).astype(np.uint8)
    # codebook: calibrated, or a random permutation prefix
    if rng.random() < 0.5:
        cb = list(oracle.calibrate(bits, dtype))
    else:
        cb = list(rng.permutation(symbols)[:16])
    return dtype, fmt, bits, cb


@pytest.mark.parametrize("seed", range(48))
def test_fuzz_roundtrip(seed):
    import fp8_kv_cache_sz_amd as sz
    dtype, fmt, bits, cb = _case(seed)
    n = bits.size
    print("fuzz seed=%d dtype=%d fmt=%d n=%d" % (seed, dtype, fmt, n), flush=True)
    if fmt == 1:
        expect = oracle.encode(bits, dtype, cb)
    else:
        expect = oracle.encode_variant(bits, fmt, cb[:oracle.BOOK_ENTRIES[fmt]])
    x = torch.from_numpy(bits.copy())
    x = (x.view(torch.int16).view(torch.bfloat16) if dtype == 0 else x).cuda()
    book = sz.Codebook(dtype, tuple(int(v) for v in cb))
    if fmt != 1:
        k = oracle.BOOK_ENTRIES[fmt]
        book = sz.Codebook(dtype, tuple(int(v) for v in cb[:k]) + (0,) * (16 - k))
    cap = sz.encoded_size(dtype, n, n, fmt)
    out = torch.full((cap,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = torch.full((sz.workspace_size(dtype, n),), 0xA5, dtype=torch.uint8, device="cuda")
    buf, size, esc = sz.encode(x, book, out=out, ws=ws, fmt=fmt)
    assert size == expect.size
    got = buf[:size].cpu().numpy()
    assert np.array_equal(got, expect), np.nonzero(got != expect)[0][:8]
    y = sz.decode(buf[:size], dtype, n, fmt=fmt)
    assert np.array_equal(y.view(torch.uint8).cpu().numpy().view(bits.dtype), bits)
