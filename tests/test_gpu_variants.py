"""GPU parity of the ablation formats (BF16 only): version 2, Top-8, and
version 3, Top-15 with code 15 as escape sentinel, through the C ABI
(sz_encode_format / sz_decode_format), against the CPU oracle.

Streams must equal the oracle's byte for byte; decoding must give the input
back bit for bit, both from the GPU stream and from the oracle's stream.
Output buffers are poison-filled so unwritten bytes show up.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

POISON = 0xA5
BLOCK = 65536
FORMATS = [2, 3]


def _sz():
    import fp8_kv_cache_sz_amd as sz
    return sz


def _dev(bits):
    return torch.from_numpy(bits.copy()).view(torch.int16).view(torch.bfloat16).cuda()


def _encode(bits, fmt, book):
    sz = _sz()
    n = bits.size
    cap = sz.encoded_size(0, n, n, fmt)
    out = torch.full((max(cap, 1),), POISON, dtype=torch.uint8, device="cuda")
    ws = torch.full((sz.workspace_size(0, n),), POISON, dtype=torch.uint8, device="cuda")
    cb = sz.Codebook(0, tuple(int(v) for v in book) + (0,) * (16 - len(book)))
    return sz.encode(_dev(bits), cb, out=out, ws=ws, fmt=fmt)


def _decode(stream_dev, fmt, n, check=True):
    sz = _sz()
    out = torch.full((max(n, 1) * 2,), POISON, dtype=torch.uint8, device="cuda")
    ws = torch.full((sz.workspace_size(0, n),), POISON, dtype=torch.uint8, device="cuda")
    sz.decode(stream_dev, 0, n, out=out.view(torch.bfloat16)[:n], ws=ws, check=check, fmt=fmt)
    return out, ws


def roundtrip(bits, fmt, book):
    print("variant roundtrip fmt=%d n=%d" % (fmt, bits.size), flush=True)
    book = list(book)[:oracle.BOOK_ENTRIES[fmt]]
    expect = oracle.encode_variant(bits, fmt, book)
    buf, size, esc = _encode(bits, fmt, book)
    assert size == expect.size
    got = buf[:size].cpu().numpy()
    if not np.array_equal(got, expect):
        bad = np.nonzero(got != expect)[0]
        raise AssertionError("stream differs at %d bytes, first %s" % (bad.size, bad[:8]))
    n = bits.size
    for src in (buf[:size], torch.from_numpy(expect).cuda()):
        out, _ = _decode(src, fmt, n)
        a = out.cpu().numpy()
        assert np.array_equal(a[:2 * n].view(np.uint16), bits)
        assert np.all(a[2 * n:] == POISON)
    return expect


SIZES = [0, 1, 7, 8, 9, 511, 4095, 4097, 16385, 65535, 65536, 65537, 3 * 65536 + 1003]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_random_bits(n, fmt):
    bits = synth.as_bits_numpy(synth.random_bits(500 + n % 101, n, 0))
    roundtrip(bits, fmt, range(118, 134))


@pytest.mark.parametrize("n", [1, 33, 4097, 65537, 200000])
@pytest.mark.parametrize("fmt", FORMATS)
def test_kv_like(n, fmt):
    x = synth.kv_layer(7, tokens=(n + 1023) // 1024 + 1)
    bits = synth.as_bits_numpy(x)[:n]
    roundtrip(bits, fmt, oracle.calibrate(synth.as_bits_numpy(synth.calibration_tensor("kv1m")), 0))


@pytest.mark.parametrize("fmt", FORMATS)
def test_all_bf16_patterns(fmt):
    roundtrip(np.arange(65536, dtype=np.uint32).astype(np.uint16), fmt, range(16))


@pytest.mark.parametrize("name", ["llama3_8b_kv", "stress_t3", "stress_random", "stress_oneexp"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_workloads_small(name, fmt):
    x, dtype = synth.workload(name, size="small")
    book = oracle.calibrate(synth.as_bits_numpy(synth.calibration_tensor(name)), 0)
    roundtrip(synth.as_bits_numpy(x), fmt, book)


@pytest.mark.parametrize("fmt", FORMATS)
def test_device_validation_matches_oracle(fmt):
    """Corrupted streams: the device verdict equals the oracle's."""
    sz = _sz()
    x, _ = synth.workload("stress_t3", size="small")
    bits = synth.as_bits_numpy(x)[:2 * BLOCK + 999]
    n = bits.size
    book = list(range(118, 118 + oracle.BOOK_ENTRIES[fmt]))
    s = oracle.encode_variant(bits, fmt, book)
    cases = []
    t = s.copy(); t[4] = 1; cases.append(t)                          # another version
    t = s.copy(); t[6] = 1; cases.append(t)                          # E5M2 dtype
    t = s.copy(); t[47] = 3; cases.append(t)                         # unused book byte
    t = s.copy(); t[64] += 1; cases.append(t)                        # counts no longer sum to E
    t = s.copy(); t[64] -= 1; t[68] += 1; cases.append(t)            # counts sum to E, blocks disagree
    cases.append(s[:-1].copy())                                      # truncated
    for t in cases:
        want = oracle.validate_variant(t, fmt, n)
        assert want != 0
        out = torch.full((2 * n,), POISON, dtype=torch.uint8, device="cuda")
        ws = torch.zeros(sz.workspace_size(0, n), dtype=torch.uint8, device="cuda")
        try:
            sz.decode(torch.from_numpy(t).cuda(), 0, n, out=out.view(torch.bfloat16), ws=ws, fmt=fmt)
            got = 0
        except sz.SplitZipError as e:
            got = e.code
        assert got == want, (fmt, got, want)


@pytest.mark.parametrize("fmt", FORMATS)
def test_full_size_llama3_kv(fmt):
    """The 1 GiB Llama-3-8B KV cache: round trip bit-exact, E equal to the
    escape count torch computes from the exponent field, sampled blocks equal
    to the oracle's encoding of the same block."""
    sz = _sz()
    torch.cuda.empty_cache()
    x, _ = synth.workload("llama3_8b_kv", device="cuda")
    n = x.numel()
    book = list(oracle.calibrate(synth.as_bits_numpy(synth.calibration_tensor("llama3_8b_kv")), 0))
    book = book[:oracle.BOOK_ENTRIES[fmt]]
    cb = sz.Codebook(0, tuple(book) + (0,) * (16 - len(book)))
    buf, size, esc = sz.encode(x, cb, fmt=fmt)
    print("full-size fmt=%d escapes=%d rate=%.5f ratio=%.5f" % (fmt, esc, esc / n, 2 * n / size), flush=True)
    expo = (x.view(torch.int16).to(torch.int32) >> 7) & 0xFF
    in_book = torch.isin(expo, torch.tensor(book, dtype=torch.int32, device="cuda"))
    assert esc == int((~in_book).sum())
    del expo, in_book
    y = sz.decode(buf[:size], 0, n, fmt=fmt)
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))
    del y
    # sampled blocks: the oracle encodes each block alone; its code and
    # sign/mantissa bytes must equal the GPU stream's bytes for that block
    nb = (n + BLOCK - 1) // BLOCK
    per = 3 * BLOCK // 8 if fmt == 2 else BLOCK // 2
    off_code = (64 + 4 * nb + 255) // 256 * 256
    off_sm = off_code + ((n * 3 // 8 if fmt == 2 else n // 2) + 255) // 256 * 256
    counts = buf[64:64 + 4 * nb].view(torch.int32).cpu().numpy()
    for b in [0, 1, nb // 2, nb - 1]:
        bits = synth.as_bits_numpy(x[b * BLOCK:(b + 1) * BLOCK])
        ref = oracle.encode_variant(bits, fmt, book)
        r_code = (64 + 4 + 255) // 256 * 256
        assert np.array_equal(buf[off_code + b * per:off_code + (b + 1) * per].cpu().numpy(), ref[r_code:r_code + per])
        r_sm = r_code + (per + 255) // 256 * 256
        assert np.array_equal(buf[off_sm + b * BLOCK:off_sm + (b + 1) * BLOCK].cpu().numpy(), ref[r_sm:r_sm + BLOCK])
        assert counts[b] == int(ref[64:68].view(np.uint32)[0])
    del x, buf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pad_blocks", [0, 256])
@pytest.mark.parametrize("heavy", [False, True])
def test_top8_record_validation(heavy, pad_blocks):
    """Malformed position records of the Top-8 format, in blocks with a few
    records and in blocks where most values escape, behind 0 or 256 blocks of
    escape-free padding (the narrow and the wide span shapes): the device
    verdict equals the oracle's, and the untouched stream decodes."""
    rng = np.random.default_rng(21)
    n = BLOCK + 20000
    if heavy:
        e = rng.integers(100, 140, n)                       # about 80 % outside the book
    else:
        e = np.full(n, 124)
        e[rng.choice(n, 60, replace=False)] = 90
    bits = ((rng.integers(0, 2, n) << 15) | (e << 7) | rng.integers(0, 128, n)).astype(np.uint16)
    bits = np.concatenate([np.full(pad_blocks * BLOCK, 124 << 7, dtype=np.uint16), bits])
    n = bits.size
    good = oracle.encode_variant(bits, 2, range(120, 128))
    e_total = int(good[16:24].view(np.uint64)[0])
    first = good.size - 3 * e_total
    cases = [("repeat", lambda t: t.__setitem__(slice(first + 3, first + 5), t[first:first + 2].copy())),
             ("middle_range", lambda t: t.__setitem__(slice(first + 3 * (e_total // 2), first + 3 * (e_total // 2) + 2),
                                                      [0xFF, 0xFF])),
             ("range_last_block", lambda t: t.__setitem__(slice(good.size - 3, good.size - 1), [0x30, 0x75]))]
    for name, mutate in cases:
        print("top8 record case", name, "heavy", heavy, "pad", pad_blocks, flush=True)
        t = good.copy()
        mutate(t)
        want = oracle.validate_variant(t, 2, n)
        assert want == oracle.E_FORMAT, name
        _, ws = _decode(torch.from_numpy(t).cuda(), 2, n, check=False)
        assert int(ws[:4].cpu().view(torch.int32)[0]) == want, name
    out, ws = _decode(torch.from_numpy(good).cuda(), 2, n, check=False)
    assert int(ws[:4].cpu().view(torch.int32)[0]) == 0
    assert np.array_equal(out.cpu().numpy()[:2 * n].view(np.uint16), bits)
