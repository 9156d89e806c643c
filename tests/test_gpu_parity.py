"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Encoded streams must equal the oracle's byte for byte over [0, size);
decoded tensors must equal the input bit for bit (tolerance 0: everything
is integer work).  Output buffers are poison-filled (0xA5) before each call
so bytes the kernels never write show up.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import streamfmt

pytestmark = pytest.mark.gpu

POISON = 0xA5


def _sz():
    import fp8_kv_cache_sz_amd as sz
    return sz


def _dev_input(bits_np, dtype):
    t = torch.from_numpy(bits_np.copy())
    if dtype == 0:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def _encode_gpu(x, cb_exps, dtype):
    sz = _sz()
    n = x.numel()
    cap = sz.encoded_size(dtype, n, n)
    out = torch.full((cap,), POISON, dtype=torch.uint8, device="cuda")
    ws = torch.full((sz.workspace_size(dtype, n),), POISON, dtype=torch.uint8, device="cuda")
    buf, size, esc = sz.encode(x, sz.Codebook(dtype, tuple(int(v) for v in cb_exps)), out=out, ws=ws)
    return buf, size, esc


def _decode_gpu(stream_dev, dtype, n, in_bytes=None, check=True):
    sz = _sz()
    out = torch.full((max(n, 1) * (2 if dtype == 0 else 1),), POISON, dtype=torch.uint8, device="cuda")
    # exactly the decode workspace: the kernels must stay inside it
    ws = torch.full((sz.decode_workspace_size(dtype, n),), POISON, dtype=torch.uint8, device="cuda")
    view = out.view(torch.bfloat16) if dtype == 0 else out
    sz.decode(stream_dev, dtype, n, out=view[:n] if n else view[:0], ws=ws, check=check, in_bytes=in_bytes)
    return out, ws


def _bits_of(out_u8, dtype, n):
    a = out_u8.cpu().numpy()
    return a[:2 * n].view(np.uint16) if dtype == 0 else a[:n]


def roundtrip_check(bits, dtype, cb):
    """Full byte-for-byte encode parity and bit-exact decode (oracle and GPU streams)."""
    print("roundtrip n=%d dtype=%d" % (bits.size, dtype), flush=True)
    expect = oracle.encode(bits, dtype, cb)
    x = _dev_input(bits, dtype)
    buf, size, esc = _encode_gpu(x, cb, dtype)
    assert size == expect.size
    got = buf[:size].cpu().numpy()
    if not np.array_equal(got, expect):
        bad = np.nonzero(got != expect)[0]
        raise AssertionError("stream differs at %d bytes, first %s (got %02x want %02x)"
                             % (bad.size, bad[:8], got[bad[0]], expect[bad[0]]))
    # decode the GPU stream and, separately, the oracle's stream
    out, _ = _decode_gpu(buf[:size], dtype, bits.size)
    assert np.array_equal(_bits_of(out, dtype, bits.size), bits)
    out2, _ = _decode_gpu(torch.from_numpy(expect).cuda(), dtype, bits.size)
    assert np.array_equal(_bits_of(out2, dtype, bits.size), bits)
    # no byte past the decoded values was touched
    tail = out[bits.size * (2 if dtype == 0 else 1):].cpu().numpy()
    assert np.all(tail == POISON)
    return expect


# Escape-free 64K blocks put in front of a test case: 0 keeps the stream
# small (one-wave decode scan, 4096-element BF16 spans), 256 moves it to
# 8192-element BF16 spans, 1024 past the one-wave scan's 1024 blocks to the
# one-workgroup scan.
PAD_BLOCKS = [0, 256, 1024]


def _pad_front(bits, pad_blocks, fill):
    return np.concatenate([np.full(pad_blocks * 65536, fill, dtype=bits.dtype), bits])


EDGE_SIZES = [0, 1, 2, 3, 7, 8, 9, 15, 16, 17, 511, 512, 513, 4095, 4096, 4097, 16383, 16384,
              16385, 65535, 65536, 65537, 3 * 65536 + 1003]


@pytest.mark.parametrize("n", EDGE_SIZES)
@pytest.mark.parametrize("dtype", [0, 1])
def test_edge_sizes_random_bits(n, dtype):
    rng = np.random.default_rng(n + 17)
    if dtype == 0:
        bits = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
        cb = rng.permutation(256)[:16].astype(np.uint8)
    else:
        bits = rng.integers(0, 256, n, dtype=np.uint32).astype(np.uint8)
        cb = rng.permutation(32)[:16].astype(np.uint8)
    roundtrip_check(bits, dtype, cb)


@pytest.mark.parametrize("n", [1, 9, 31, 33, 4097, 65537, 200000])
@pytest.mark.parametrize("dtype", [0, 1])
def test_edge_sizes_kv_like(n, dtype):
    """Narrow exponent distribution (few escapes), calibrated codebook."""
    rng = np.random.default_rng(n)
    if dtype == 0:
        e = np.clip(np.rint(rng.normal(126, 2.5, n)), 0, 255).astype(np.uint16)
        bits = ((rng.integers(0, 256, n).astype(np.uint16) & 0x80) << 8) | (e << 7) | rng.integers(0, 128, n).astype(np.uint16)
        bits = bits.astype(np.uint16)
    else:
        e = np.clip(np.rint(rng.normal(14, 2.0, n)), 0, 31).astype(np.uint8)
        bits = ((rng.integers(0, 2, n).astype(np.uint8) << 7) | (e << 2) | rng.integers(0, 4, n).astype(np.uint8)).astype(np.uint8)
    cb = oracle.calibrate(bits, dtype)
    roundtrip_check(bits, dtype, cb)


# Streams up to 2048 tiles (32M elements) are ordered by one compaction launch
# that sums the tile counts itself, larger ones through the scan; streams up
# to 1024 blocks (64M elements) are decoded by workgroups that sum the block
# counts themselves, larger ones after the scan.  Sizes at and just past the
# encode limit and at the decode limit, so the fused paths and the mixed
# case (scan encode, fused decode) are checked against the oracle byte for
# byte; the full-size workloads take both scans.
PATH_SIZES = [2048 * 16384, 2048 * 16384 + 1, 1024 * 65536]


@pytest.mark.parametrize("n", PATH_SIZES)
@pytest.mark.parametrize("dtype", [0, 1])
def test_prefix_path_limits(n, dtype):
    # exponents from a sum of small uniform terms (a bell over 18 or 20
    # values, so the Top-16 leaves a few per cent of escapes); integer draws
    # keep 64M elements quick
    r = np.random.default_rng(n % 1000 + 7).integers(0, 2 ** 32, n, dtype=np.uint32)
    if dtype == 0:
        e = 120 + (r & 7) + ((r >> 3) & 7) + ((r >> 6) & 3)
        bits = (((r >> 16) & 0x807F) | (e << 7)).astype(np.uint16)
    else:
        e = 8 + (r & 3) + ((r >> 2) & 3) + ((r >> 4) & 3) + ((r >> 6) & 3) + ((r >> 8) & 7)
        bits = (((r >> 16) & 0x83) | (e << 2)).astype(np.uint8)
    cb = oracle.calibrate(bits, dtype)
    roundtrip_check(bits, dtype, cb)


def test_all_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    roundtrip_check(bits, 0, oracle.calibrate(bits, 0))


def test_all_e5m2_patterns():
    bits = np.arange(256, dtype=np.uint32).astype(np.uint8)
    roundtrip_check(bits, 1, oracle.calibrate(bits, 1))
    # every pattern 300 times, in a shuffled order over several blocks
    rng = np.random.default_rng(2)
    many = rng.permutation(np.tile(bits, 300))
    roundtrip_check(many, 1, oracle.calibrate(many, 1))


def test_every_element_escapes():
    """Two full blocks and a tail where no exponent is in the codebook."""
    n = 2 * 65536 + 77
    rng = np.random.default_rng(5)
    e = rng.integers(16, 256, n).astype(np.uint16)
    bits = ((rng.integers(0, 2, n).astype(np.uint16) << 15) | (e << 7) | rng.integers(0, 128, n).astype(np.uint16)).astype(np.uint16)
    cb = np.arange(16, dtype=np.uint8)
    expect = roundtrip_check(bits, 0, cb)
    assert streamfmt.header(expect)["escapes"] == n


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("n", [16 * 65536, 40 * 65536 + 1234, 2049 * 16384 + 1234])
def test_escape_heavy_compaction_paths(dtype, n):
    """Random bits (escape-heavy tiles mixed with light ones) at sizes whose
    dense encoders stage every tile, copied by 1024 lanes per block (16
    blocks) or by one wave per block (40 blocks), and at one past 2,048
    tiles, whose compaction re-derives the heavy tiles from the input."""
    rng = np.random.default_rng(17)
    if dtype == 0:
        bits = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
        bits[((bits >> 7) & 0xFF) == 0xFF] &= 0x807F             # no NaN/Inf exponent
        cb = np.arange(120, 136, dtype=np.uint8)
    else:
        bits = rng.integers(0, 256, n, dtype=np.uint32).astype(np.uint8)
        cb = np.arange(8, 24, dtype=np.uint8)
    # a light stretch: one block of in-book exponents
    light = slice(65536, 2 * 65536)
    if dtype == 0:
        bits[light] = (bits[light] & 0x807F) | (np.uint16(127) << 7)
    else:
        bits[light] = (bits[light] & 0x83) | (np.uint8(15) << 2)
    expect = roundtrip_check(bits, dtype, cb)
    counts = streamfmt.sections(expect)["counts"]
    assert counts[1] == 0 and max(counts) > 16384


# Escapes per 16K tile around the encoders' staging limits: a row's direct
# records (up to 32 per chunk row) against its LDS segments, the E5M2 tile
# buffer (2,058 records), and the re-derivation above 4,096 records.
TILE_ESCAPES = [0, 1, 31, 32, 33, 200, 500, 2057, 2058, 2059, 3000, 4095, 4096, 4097, 9000, 16384]


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("clustered", [False, True])
def test_tile_escape_counts_around_staging_limits(dtype, clustered):
    """A stream past 2,048 tiles (where the limits apply) whose tiles carry
    the escape counts of TILE_ESCAPES in turn, spread over the tile or in one
    run at a random place; the other tiles have none."""
    rng = np.random.default_rng(31 + dtype + 2 * clustered)
    tiles = 2049 + len(TILE_ESCAPES)
    n = tiles * 16384 - 77
    if dtype == 0:
        bits = np.full(n, 0x3F80, dtype=np.uint16)            # exponent 127
        esc_val = lambda m: (0x0080 | (rng.integers(0, 2, m) << 15) | rng.integers(0, 128, m)).astype(np.uint16)
        cb = np.array([127] + list(range(100, 115)), dtype=np.uint8)
    else:
        bits = np.full(n, 0x3C, dtype=np.uint8)               # exponent 15
        esc_val = lambda m: (0x04 | (rng.integers(0, 2, m) << 7) | rng.integers(0, 4, m)).astype(np.uint8)
        cb = np.array([15] + list(range(16, 31)), dtype=np.uint8)
    want = np.zeros(tiles, dtype=np.int64)
    for i, k in enumerate(TILE_ESCAPES):
        t = 5 + 97 * i                                        # tiles spread over the stream
        lo, hi = t * 16384, min((t + 1) * 16384, n)
        k = min(k, hi - lo)
        if clustered:
            start = lo + int(rng.integers(0, hi - lo - k + 1))
            idx = np.arange(start, start + k)
        else:
            idx = lo + rng.choice(hi - lo, size=k, replace=False)
        bits[idx] = esc_val(k)
        want[t] = k
    expect = roundtrip_check(bits, dtype, cb)
    assert streamfmt.header(expect)["escapes"] == int(want.sum())


# Record counts around the compaction's copy limits: 256 (8-lane groups, two
# blocks per wave), 1,024 (16-lane groups) and 4,096 (staging; a heavier
# tile is re-derived from the input).
PAIR_COUNTS = [1, 255, 256, 257, 1024, 1025, 4096, 4097]


def _escape_stream(dtype, n, rng):
    """A stream of n escape-free values, a value generator for escapes and
    the codebook that makes them so."""
    if dtype == 0:
        bits = np.full(n, 0x3F80, dtype=np.uint16)            # exponent 127
        esc_val = lambda m: (0x0080 | (rng.integers(0, 2, m) << 15) | rng.integers(0, 128, m)).astype(np.uint16)
        cb = np.array([127] + list(range(100, 115)), dtype=np.uint8)
    else:
        bits = np.full(n, 0x3C, dtype=np.uint8)               # exponent 15
        esc_val = lambda m: (0x04 | (rng.integers(0, 2, m) << 7) | rng.integers(0, 4, m)).astype(np.uint8)
        cb = np.array([15] + list(range(16, 31)), dtype=np.uint8)
    return bits, esc_val, cb


def _set_tile_escapes(bits, fill, esc_val, rng, tile, k):
    """Tile `tile` gets exactly k escapes (at random places) and no others."""
    lo, hi = tile * 16384, min((tile + 1) * 16384, bits.size)
    bits[lo:hi] = fill
    k = min(k, hi - lo)
    bits[lo + rng.choice(hi - lo, size=k, replace=False)] = esc_val(k)


@pytest.mark.parametrize("dtype", [0, 1])
def test_paired_block_copies(dtype):
    """A stream above 4,096 blocks, where a compaction wave copies the staged
    records of blocks b and b + 4,096 at once (512 workgroups of eight
    waves): every tile holds a few escapes, and tiles with the record counts
    of PAIR_COUNTS sit in the first block of a pair, in the second, in both,
    and in blocks without a partner."""
    rng = np.random.default_rng(71 + dtype)
    nb = 4096 + 300
    n = nb * 65536 - 4321
    bits, esc_val, cb = _escape_stream(dtype, n, rng)
    fill = bits[0]
    nt = (n + 16383) // 16384
    for t in range(nt):                                       # light records everywhere
        _set_tile_escapes(bits, fill, esc_val, rng, t, 3)
    heavy = {}
    for i, k in enumerate(PAIR_COUNTS):
        for b in (5 + 9 * i,                                  # first block of a pair
                  4096 + 100 + 9 * i,                         # second block of a pair
                  200 + 9 * i, 4096 + 200 + 9 * i,            # both blocks of one pair
                  1000 + 37 * i):                             # no partner (b + 4096 >= nb)
            heavy[4 * b + i % 4] = k
    for t, k in heavy.items():
        _set_tile_escapes(bits, fill, esc_val, rng, t, k)
    expect = roundtrip_check(bits, dtype, cb)
    escaped = bits != fill
    assert streamfmt.header(expect)["escapes"] == int(np.count_nonzero(escaped))
    per_block = np.add.reduceat(escaped, np.arange(0, n, 65536))
    assert np.array_equal(streamfmt.sections(expect)["counts"], per_block)


@pytest.mark.parametrize("where,nb", [("first", 8216), ("last", 8216), ("last", 8193)])
def test_one_flagged_tile_past_8192_blocks(where, nb):
    """Above 8,192 blocks the scan runs in two workgroups (the second one
    holding a single block at 8,193); a single tile heavy enough to be
    re-derived, the stream's first or its last, must still make the
    compaction re-derive it (the scan's flagged-tile words)."""
    rng = np.random.default_rng(nb + (5 if where == "first" else 6))
    n = nb * 65536 - 999
    bits, esc_val, cb = _escape_stream(0, n, rng)
    fill = bits[0]
    nt = (n + 16383) // 16384
    tile = 0 if where == "first" else nt - 1
    _set_tile_escapes(bits, fill, esc_val, rng, tile, 9000)
    _set_tile_escapes(bits, fill, esc_val, rng, nt // 2, 17)     # one light tile elsewhere
    expect = roundtrip_check(bits, 0, cb)
    assert streamfmt.header(expect)["escapes"] == 9000 + 17


# Streams above 128 blocks decode BF16 with eight workgroups per block: a
# block of at most 2048 records in strided 2048-element sub-spans (workgroup
# r: sub-spans r, r + 8, r + 16, r + 24, one wave per sub-span's records), a
# heavier one in contiguous 8192-element spans; the last block gets only as
# many workgroups as it has sub-spans (up to 8).  E5M2 decodes them in
# contiguous 16384-element spans (four workgroups per block, fewer in the
# last).  Last blocks of every length class around the sub-span, row and
# span edges.
WIDE_TAILS = [1, 2047, 2048, 2049, 8191, 8192, 8193, 8 * 2048 + 1, 30001, 65535, 65536]
WIDE_TAILS_E5M2 = [1, 31, 33, 2047, 2049, 16383, 16384, 16385, 32769, 49153, 65535, 65536]


@pytest.mark.parametrize("dtype,tail", [(0, t) for t in WIDE_TAILS] + [(1, t) for t in WIDE_TAILS_E5M2])
def test_wide_decode_block_tails(dtype, tail):
    """Escapes on both sides of every 2048-element edge (first block, last
    full block, last block); blocks of 2,048 and 2,049 scattered escapes (the
    two layouts' limit), 3,500 scattered and 65,536 (every element); a run
    of 1,500 across two sub-spans (strided: the per-wave windows miss it and
    the per-wave search finds it) and a run of 5,000 across a span edge
    (contiguous: the same for the workgroup's window)."""
    rng = np.random.default_rng(tail + 101)
    full = 130
    n = full * 65536 + tail
    if dtype == 0:
        fill = 0x3F80                                         # exponent 127, in the book
        bits = np.full(n, fill, dtype=np.uint16)
        esc_val = lambda m: (0x0080 | (rng.integers(0, 2, m) << 15) | rng.integers(0, 128, m)).astype(np.uint16)
        cb = np.array([127] + list(range(100, 115)), dtype=np.uint8)
    else:
        fill = 0x3C                                           # exponent 15, in the book
        bits = np.full(n, fill, dtype=np.uint8)
        esc_val = lambda m: (0x04 | (rng.integers(0, 2, m) << 7) | rng.integers(0, 4, m)).astype(np.uint8)
        cb = np.array([15] + list(range(16, 31)), dtype=np.uint8)
    last0 = full * 65536                                      # first element of the last block
    edges = []
    for b0 in (0, (full - 1) * 65536, full * 65536):
        for m in range(33):
            for p in (b0 + 2048 * m - 1, b0 + 2048 * m):
                if b0 <= p < min(b0 + 65536, n):
                    edges.append(p)
    edges = np.array(sorted(set(edges)))
    bits[edges] = esc_val(edges.size)
    bits[5 * 65536:6 * 65536] = esc_val(65536)
    for blk, m in ((7, 3500), (8, 2048), (11, 2049)):
        where = blk * 65536 + rng.choice(65536, m, replace=False)
        bits[where] = esc_val(m)
    run = 9 * 65536 + 8192 - 2000
    bits[run:run + 5000] = esc_val(5000)
    run = 10 * 65536 + 5 * 2048 - 700
    bits[run:run + 1500] = esc_val(1500)
    tail_hits = last0 + rng.choice(n - last0, min(n - last0, 300), replace=False)
    bits[tail_hits] = esc_val(tail_hits.size)
    expect = roundtrip_check(bits, dtype, cb)
    counts = streamfmt.sections(expect)["counts"]
    assert [int(counts[b]) for b in (5, 7, 8, 9, 10, 11)] == [65536, 3500, 2048, 5000, 1500, 2049]
    assert streamfmt.header(expect)["escapes"] == int(np.count_nonzero(bits != fill))


def test_single_escapes_at_block_edges():
    n = 3 * 65536
    bits = np.full(n, 0x3F80, dtype=np.uint16)
    for i in (0, 65535, 65536, 2 * 65536 + 7, n - 1):
        bits[i] = 0x0080 | 0x8000            # exponent 1, negative
    cb = np.array([127] + list(range(100, 115)), dtype=np.uint8)
    expect = roundtrip_check(bits, 0, cb)
    sec = streamfmt.sections(expect)
    assert list(sec["counts"]) == [2, 1, 2]
    assert list(sec["pos"]) == [0, 65535, 0, 7, 65535]


@pytest.mark.parametrize("pad_blocks", PAD_BLOCKS)
@pytest.mark.parametrize("dtype", [0, 1])
def test_clustered_escapes(dtype, pad_blocks):
    """Escapes bunched into one run per block (a few hundred to a few thousand
    records, at a random place, some across span and block edges), so that
    a span's records are far from where evenly spread escapes would put them."""
    rng = np.random.default_rng(13)
    nblk = 6
    n = nblk * 65536 - 1234
    if dtype == 0:
        bits = np.full(n, 0x3F80, dtype=np.uint16)            # exponent 127
        esc_val = lambda m: (0x0080 | (rng.integers(0, 2, m) << 15) | rng.integers(0, 128, m)).astype(np.uint16)
        cb = np.array([127] + list(range(100, 115)), dtype=np.uint8)
    else:
        bits = np.full(n, 0x3C, dtype=np.uint8)               # exponent 15
        esc_val = lambda m: (0x04 | (rng.integers(0, 2, m) << 7) | rng.integers(0, 4, m)).astype(np.uint8)
        cb = np.array([15] + list(range(16, 31)), dtype=np.uint8)
    for b, m in enumerate([300, 1500, 5000, 9000, 20000, 700]):
        start = b * 65536 + int(rng.integers(0, 65536 - m))
        if b == 2:
            start = 3 * 65536 - m // 2                        # run across a block edge
        end = min(start + m, n)
        bits[start:end] = esc_val(end - start)
    bits = _pad_front(bits, pad_blocks, bits[0])
    expect = roundtrip_check(bits, dtype, cb)
    assert streamfmt.header(expect)["escapes"] > 30000


def test_no_escapes_single_exponent():
    bits = synth.as_bits_numpy(synth.single_exponent(41, 300000, 127))
    cb = oracle.calibrate(synth.as_bits_numpy(synth.calibration_tensor("kv1m")), 0)
    expect = roundtrip_check(bits, 0, cb)
    assert streamfmt.header(expect)["escapes"] == 0


@pytest.mark.parametrize("name", ["kv1m", "llama3_8b_kv", "longctx_kv", "stress_t3", "stress_oneexp",
                                  "stress_random", "llama3_8b_kv_e5m2"])
def test_workloads_small(name):
    x, dtype = synth.workload(name, size="small")
    cb = oracle.calibrate(synth.as_bits_numpy(synth.calibration_tensor(name)), dtype)
    roundtrip_check(synth.as_bits_numpy(x), dtype, cb)


def test_gpu_calibration_matches_oracle():
    sz = _sz()
    for name in ("kv1m", "llama3_8b_kv"):
        cal = synth.calibration_tensor(name)
        assert list(sz.calibrate(cal).exps) == list(oracle.calibrate(synth.as_bits_numpy(cal), 0))


def test_encode_is_deterministic_and_stream_order_safe():
    sz = _sz()
    x, dtype = synth.workload("stress_t3", size="small")
    cb = sz.calibrate(synth.calibration_tensor("kv1m"))
    xd = x.cuda()
    a, size_a, _ = sz.encode(xd, cb)
    b, size_b, _ = sz.encode(xd, cb)
    assert size_a == size_b
    assert torch.equal(a[:size_a], b[:size_b])
    # two encodes in flight on one stream with distinct workspaces, then decodes
    y = torch.flip(xd, [0]).contiguous()
    s1, _, _ = sz.encode(xd, cb, sync=False)
    s2, _, _ = sz.encode(y, cb, sync=False)
    torch.cuda.synchronize()
    d1 = sz.decode(s1, dtype, xd.numel())
    d2 = sz.decode(s2, dtype, y.numel())
    assert torch.equal(d1.view(torch.int16), xd.view(torch.int16))
    assert torch.equal(d2.view(torch.int16), y.view(torch.int16))


def test_concurrent_streams_with_own_workspaces():
    """Round trips on two streams at once, each with its own buffers and
    workspaces: the library keeps no state between calls, so both streams
    equal the oracle's byte for byte and both decodes are exact."""
    sz = _sz()
    cb = sz.calibrate(synth.calibration_tensor("kv1m"))
    xs = [synth.workload("stress_t3", size="small")[0].cuda(),
          synth.workload("llama3_8b_kv", size="small")[0].cuda()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    runs = []
    for x, s in zip(xs, streams):
        n = x.numel()
        buf = torch.empty(sz.encoded_size(0, n, n), dtype=torch.uint8, device="cuda")
        ws_enc, ws_dec = sz.workspace(0, n), sz.workspace(0, n)
        y = torch.empty_like(x)
        runs.append((x, s, buf, ws_enc, ws_dec, y))
    torch.cuda.synchronize()
    for _ in range(3):                       # interleave the two streams' launches
        for x, s, buf, ws_enc, ws_dec, y in runs:
            sz.encode(x, cb, out=buf, ws=ws_enc, stream=s, sync=False)
            sz.decode(buf, 0, x.numel(), out=y, ws=ws_dec, stream=s, check=False)
    torch.cuda.synchronize()
    for x, s, buf, ws_enc, ws_dec, y in runs:
        bits = synth.as_bits_numpy(x)
        expect = oracle.encode(bits, 0, list(cb.exps))
        size = sz.encoded_size(0, x.numel(), sz.read_escape_count(buf))
        assert size == expect.size
        assert np.array_equal(buf[:size].cpu().numpy(), expect)
        assert int(ws_dec[:4].cpu().view(torch.int32)[0]) == 0
        assert torch.equal(y.view(torch.int16), x.view(torch.int16))


def test_side_stream_with_library_allocations():
    """encode / decode on a side stream with their default host reads
    (size, escape count, decode status) and buffers the Python layer
    allocates itself: the reads wait for the side stream, and memory taken
    from the current stream's pool is not reused while the side stream
    still works on it."""
    sz = _sz()
    cb = sz.calibrate(synth.calibration_tensor("kv1m"))
    s = torch.cuda.Stream()
    for name in ("stress_t3", "llama3_8b_kv"):
        x = synth.workload(name, size="small")[0].cuda()
        n = x.numel()
        expect = oracle.encode(synth.as_bits_numpy(x), 0, list(cb.exps))
        junk = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        junk.fill_(7)                      # current-stream work queued ahead of the side stream
        del junk
        buf, size, esc = sz.encode(x, cb, stream=s)
        assert size == expect.size and esc == int(expect[16:24].view(np.uint64)[0])
        y = sz.decode(buf[:size], 0, n, stream=s)
        s.synchronize()
        assert np.array_equal(buf[:size].cpu().numpy(), expect)
        assert torch.equal(y.view(torch.int16), x.view(torch.int16))


def _corrupt_cases(stream, n):
    L = streamfmt.layout(0, n)
    first = L["off_esc"]
    yield "magic", lambda t: t.__setitem__(0, 0)
    yield "version", lambda t: t.__setitem__(4, 2)
    yield "n", lambda t: t.__setitem__(8, (int(t[8]) + 1) % 256)
    yield "escapes", lambda t: t.__setitem__(16, int(t[16]) + 1)
    yield "count", lambda t: t.__setitem__(64, int(t[64]) + 1)
    yield "pos_repeat", lambda t: t.__setitem__(slice(first + 3, first + 5), t[first:first + 2].copy())
    yield "pos_range", lambda t: t.__setitem__(slice(first + 6 * 3, first + 6 * 3 + 2), [0xFF, 0xFF])
    yield "cb_range", lambda t: t.__setitem__(32, 255)          # fine for BF16: stays valid


@pytest.mark.parametrize("pad_blocks", PAD_BLOCKS)
def test_device_validation_matches_oracle(pad_blocks):
    rng = np.random.default_rng(9)
    bits = np.full(70000, 0x3F80, dtype=np.uint16)
    idx = np.sort(rng.choice(bits.size - 1, 40, replace=False))
    bits[idx] = 0x0001
    bits = _pad_front(bits, pad_blocks, 0x3F80)
    n = bits.size
    cb = np.array([127] + list(range(100, 115)), dtype=np.uint8)
    good = oracle.encode(bits, 0, cb)
    for name, mutate in _corrupt_cases(good, n):
        t = good.copy()
        mutate(t)
        want = oracle.validate(t, 0, n)
        _, ws = _decode_gpu(torch.from_numpy(t).cuda(), 0, n, check=False)
        status = int(ws[:4].cpu().view(torch.int32)[0])
        print(name, want, status, flush=True)
        assert status == want, name
    # a BF16 stream handed to the E5M2 decoder
    _, ws = _decode_gpu(torch.from_numpy(good).cuda(), 1, n, check=False)
    assert int(ws[:4].cpu().view(torch.int32)[0]) == oracle.validate(good, 1, n) == oracle.E_DTYPE
    # the untouched stream passes
    _, ws = _decode_gpu(torch.from_numpy(good).cuda(), 0, n, check=False)
    assert int(ws[:4].cpu().view(torch.int32)[0]) == 0
    # truncated: records past in_bytes
    _, ws = _decode_gpu(torch.from_numpy(good).cuda(), 0, n, in_bytes=good.size - 1, check=False)
    assert int(ws[:4].cpu().view(torch.int32)[0]) == oracle.E_FORMAT


def test_profile_hooks_record_kernels():
    sz = _sz()
    x = synth.kv_layer(0).cuda()
    cb = sz.calibrate(synth.calibration_tensor("kv1m"))
    sz.profile_enable(True)
    buf, size, _ = sz.encode(x, cb)
    sz.decode(buf[:size], 0, x.numel())
    stats = sz.profile_collect()
    sz.profile_enable(False)
    assert stats["sz_enc_dense_bf16"][0] == 1 and stats["sz_dec_bf16_span"][0] == 1
    assert all(ms >= 0 for _, ms in stats.values())


@pytest.mark.parametrize("pad_blocks", PAD_BLOCKS)
def test_e5m2_device_validation(pad_blocks):
    bits = np.full(5000, 0x3C, dtype=np.uint8)               # 1.0: exponent 15
    bits[[10, 20, 4000]] = 0x01                              # exponent 0
    bits = _pad_front(bits, pad_blocks, 0x3C)
    n = bits.size
    cb = np.array([15] + list(range(1, 15)) + [16], dtype=np.uint8)
    good = oracle.encode(bits, 1, cb)
    first = streamfmt.layout(1, n)["off_esc"]
    for name, mutate in [("exp_range", lambda t: t.__setitem__(first + 2, 32)),
                         ("pos_order", lambda t: t.__setitem__(slice(first + 3, first + 5), [5, 0])),
                         ("pos_range", lambda t: t.__setitem__(slice(first + 6, first + 8), [0x88, 0x13]))]:
        t = good.copy()
        mutate(t)
        want = oracle.validate(t, 1, n)
        _, ws = _decode_gpu(torch.from_numpy(t).cuda(), 1, n, check=False)
        assert int(ws[:4].cpu().view(torch.int32)[0]) == want == oracle.E_FORMAT, name


@pytest.mark.parametrize("pad_blocks", PAD_BLOCKS)
@pytest.mark.parametrize("dtype", [0, 1])
def test_device_validation_heavy_blocks(dtype, pad_blocks):
    """Malformed records inside blocks where most values escape (each span
    then takes more records than its light window holds and goes through the
    exponent plane) are reported like the light ones."""
    n = 65536 + 20000
    rng = np.random.default_rng(11)
    if dtype == 0:
        e = rng.integers(16, 256, n).astype(np.uint16)
        bits = ((rng.integers(0, 2, n).astype(np.uint16) << 15) | (e << 7) | rng.integers(0, 128, n).astype(np.uint16)).astype(np.uint16)
    else:
        e = rng.integers(16, 32, n).astype(np.uint8)
        bits = ((rng.integers(0, 2, n).astype(np.uint8) << 7) | (e << 2) | rng.integers(0, 4, n).astype(np.uint8)).astype(np.uint8)
    # padding value: exponent 1, inside the book [0..15]
    bits = _pad_front(bits, pad_blocks, 0x0080 if dtype == 0 else 0x04)
    n = bits.size
    cb = np.arange(16, dtype=np.uint8)
    good = oracle.encode(bits, dtype, cb)
    assert streamfmt.sections(good)["counts"][pad_blocks] > 8192
    first = streamfmt.layout(dtype, n)["off_esc"]
    second_block = first + 3 * 65536
    cases = [("repeat", lambda t: t.__setitem__(slice(first + 3000, first + 3002), t[first + 2997:first + 2999].copy())),
             ("descend", lambda t: t.__setitem__(slice(first + 3, first + 5), [0, 0])),
             ("range_last_block", lambda t: t.__setitem__(slice(second_block + 3 * 19999, second_block + 3 * 19999 + 2), [0x30, 0x75]))]
    if dtype == 1:
        cases.append(("exp_range", lambda t: t.__setitem__(first + 3 * 500 + 2, 40)))
    for name, mutate in cases:
        t = good.copy()
        mutate(t)
        want = oracle.validate(t, dtype, n)
        assert want == oracle.E_FORMAT, name
        _, ws = _decode_gpu(torch.from_numpy(t).cuda(), dtype, n, check=False)
        assert int(ws[:4].cpu().view(torch.int32)[0]) == want, name
    out, ws = _decode_gpu(torch.from_numpy(good).cuda(), dtype, n, check=False)
    assert int(ws[:4].cpu().view(torch.int32)[0]) == 0
    assert np.array_equal(_bits_of(out, dtype, n), bits)
