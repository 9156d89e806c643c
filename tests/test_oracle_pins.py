"""Pins for the CPU oracle, checked against facts that do not come from the
oracle itself: hand-worked streams, closed forms, brute force over every bit
pattern, float decompositions from math.frexp, numpy bincount/lexsort
counts, and the rules the SplitZip page states (gist.science summary of
"SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
Serving", Method and Results sections).
"""
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import synth
from tests import streamfmt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_golden(name):
    fields = {}
    chunks = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "bytes":
                parts = rest.split()
                chunks.append((int(parts[0]), bytes(int(x, 16) for x in parts[1:])))
            else:
                fields[key] = rest.split()
    size = int(fields["size"][0])
    expect = bytearray(size)
    for off, blob in chunks:
        expect[off:off + len(blob)] = blob
    return fields, np.frombuffer(bytes(expect), dtype=np.uint8)


@pytest.mark.parametrize("name", ["bf16_five_values.txt", "e5m2_ten_values.txt"])
def test_golden_hand_worked_stream(name):
    fields, expect = _load_golden(name)
    dtype = oracle.BF16 if fields["dtype"][0] == "bf16" else oracle.E5M2
    floats = torch.tensor([float(x) for x in fields["values_float"]], dtype=torch.float32)
    if dtype == oracle.BF16:
        bits = np.array([int(x, 16) for x in fields["values_hex"]], dtype=np.uint16)
        # the bit patterns are what torch's own round-to-nearest-even cast gives
        assert np.array_equal(synth.as_bits_numpy(floats.to(torch.bfloat16)), bits)
    else:
        bits = np.array([int(x, 16) for x in fields["values_hex"]], dtype=np.uint8)
        assert np.array_equal(floats.to(torch.float8_e5m2).view(torch.uint8).numpy(), bits)
    cb = np.array([int(x, 16) for x in fields["codebook"]], dtype=np.uint8)
    got = oracle.encode(bits, dtype, cb)
    assert got.size == expect.size
    assert np.array_equal(got, expect), np.nonzero(got != expect)
    assert np.array_equal(oracle.decode(got, dtype, bits.size), bits)
    assert oracle.check_canonical(got, dtype, bits.size) == 0


def test_bruteforce_all_bf16_patterns():
    """Every BF16 bit pattern once, in natural order: one block of 65,536."""
    data = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    cb = oracle.calibrate(data, oracle.BF16)
    # each of the 256 exponent values occurs 2 * 128 = 256 times, so the
    # count-descending / exponent-ascending order is 0, 1, 2, ...
    assert list(cb) == list(range(16))
    s = oracle.encode(data, oracle.BF16, cb)
    sec = streamfmt.sections(s)
    # 16 exponents are coded, 256 patterns each: 65536 - 16 * 256 escapes
    assert sec["header"]["escapes"] == 61440
    assert list(sec["counts"]) == [61440]
    assert s.size == 282880
    # an escape is every pattern whose exponent field is >= 16, i.e. whose
    # magnitude bits are >= 16 << 7
    expect_pos = [h for h in range(65536) if (h & 0x7FFF) >= (16 << 7)]
    assert np.array_equal(sec["pos"], np.array(expect_pos))
    assert np.array_equal(sec["exp"], np.array([(h & 0x7FFF) >> 7 for h in expect_pos]))
    assert np.array_equal(oracle.decode(s, oracle.BF16, 65536), data)


def test_bruteforce_all_e5m2_patterns():
    data = np.arange(256, dtype=np.uint32).astype(np.uint8)
    cb = oracle.calibrate(data, oracle.E5M2)
    assert list(cb) == list(range(16))  # each exponent 8 times
    s = oracle.encode(data, oracle.E5M2, cb)
    sec = streamfmt.sections(s)
    assert sec["header"]["escapes"] == 128
    assert s.size == 1152
    expect_pos = [b for b in range(256) if (b & 0x7F) >= (16 << 2)]
    assert np.array_equal(sec["pos"], np.array(expect_pos))
    assert np.array_equal(oracle.decode(s, oracle.E5M2, 256), data)


def test_size_closed_forms():
    # single 1024x8x128 tensor at zero escapes: 256 (header + 16 counts,
    # padded) + 524288 nibble bytes + 1048576 sign/mantissa bytes
    assert oracle.encoded_size(oracle.BF16, 1 << 20, 0) == 1573120
    assert abs((2 << 20) / 1573120 - 1.333116) < 1e-6
    # Llama-3-8B-shaped cache, 2^29 BF16 values
    n = 1 << 29
    assert oracle.encoded_size(oracle.BF16, n, 0) == 805339392
    assert abs(2 * n / 805339392 - 1.333279) < 1e-6
    # the same cache in E5M2: 2^29 bytes -> 2^28 nibble bytes + 3 * 2^26
    assert oracle.encoded_size(oracle.E5M2, n, 0) == 469795072
    assert abs(n / 469795072 - 1.142777) < 1e-6
    # empty input: the header alone, padded to 256
    assert oracle.encoded_size(oracle.BF16, 0, 0) == 256
    # payload limits of the page: 16 bits -> 4 + 8 bits is 4/3 (Results,
    # "theoretical limit 1.33x"); 8 bits -> 4 + 3 bits is 8/7 (~1.14x, FP8)
    for n in (1 << 16, 1 << 20, 3 << 20):
        fixed_bf16 = oracle.encoded_size(oracle.BF16, n, 0) - oracle.encoded_size(oracle.BF16, 0, 0)
        fixed_e5 = oracle.encoded_size(oracle.E5M2, n, 0) - oracle.encoded_size(oracle.E5M2, 0, 0)
        meta = 256 * ((64 + 4 * (n // 65536) + 255) // 256) - 256
        assert fixed_bf16 - meta == n + n // 2
        assert fixed_e5 - meta == n // 2 + 3 * n // 8
    # each escape is one 16-bit position plus one 8-bit exponent
    for e in (0, 1, 7, 1000):
        assert oracle.encoded_size(oracle.BF16, 4096, e + 1) - oracle.encoded_size(oracle.BF16, 4096, e) == 3
    assert oracle.encoded_size(7, 10, 0) == 0  # unknown dtype


def _frexp_fields(values_f64):
    """(sign, biased exponent, 7-bit mantissa) of finite normal BF16 values,
    from math.frexp rather than bit operations."""
    m, k = np.frexp(values_f64)
    sign = np.signbit(values_f64).astype(np.int64)
    biased = (k - 1 + 127).astype(np.int64)
    mant7 = np.rint((2 * np.abs(m) - 1) * 128).astype(np.int64)
    return sign, biased, mant7


def test_field_split_against_frexp():
    x = synth.kv_layer(7, tokens=64)                       # 65,536 BF16 values
    f = x.to(torch.float64).numpy()
    assert np.all(np.abs(f) >= 2.0 ** -126)                # all normal numbers
    bits = synth.as_bits_numpy(x)
    cb = oracle.calibrate(bits, oracle.BF16)
    s = oracle.encode(bits, oracle.BF16, cb)
    sec = streamfmt.sections(s)
    sign, biased, mant7 = _frexp_fields(f)
    assert np.array_equal(sec["sm"].astype(np.int64), sign * 128 + mant7)
    escaped = np.zeros(bits.size, dtype=bool)
    escaped[sec["pos"]] = True                              # single block
    assert np.all(sec["codes"][escaped] == 0)
    assert np.array_equal(cb[sec["codes"][~escaped]].astype(np.int64), biased[~escaped])
    assert np.array_equal(sec["exp"], biased[escaped])
    assert not np.isin(sec["exp"], cb).any()


def _exponents_by_frexp(x_bf16):
    f = x_bf16.to(torch.float64).numpy()
    assert np.all(np.isfinite(f)) and np.all((f == 0) | (np.abs(f) >= 2.0 ** -126))
    _, biased, _ = _frexp_fields(np.where(f == 0, 1.0, f))
    return np.where(f == 0, 0, biased)


def test_calibration_matches_lexsort_and_histogram_identity():
    x = synth.kv_layer(1)                                   # 1,048,576 values
    expo = _exponents_by_frexp(x)
    hist = np.bincount(expo, minlength=256)
    order = np.lexsort((np.arange(256), -hist))             # count desc, exp asc
    bits = synth.as_bits_numpy(x)
    cb = oracle.calibrate(bits, oracle.BF16)
    assert np.array_equal(cb, order[:16])
    assert np.array_equal(oracle.histogram(bits, oracle.BF16), hist)
    # the page's observation: top-16 exponents cover > 99% of entries
    assert hist[order[:16]].sum() / hist.sum() > 0.99
    # escapes = N - (elements whose exponent is in the codebook)
    data = synth.as_bits_numpy(synth.kv_layer(0))
    e_expected = data.size - int(np.isin(_exponents_by_frexp(synth.kv_layer(0)), cb).sum())
    s = oracle.encode(data, oracle.BF16, cb)
    assert streamfmt.header(s)["escapes"] == e_expected


def test_escape_positions_are_block_local():
    """Constructed two-block input: every element has exponent 127 except
    four placed by hand; their records carry block-local positions."""
    n = 65536 + 3
    data = np.full(n, 0x3F80, dtype=np.uint16)             # 1.0, exponent 127
    for i in (5, 65535, 65536, 65538):
        data[i] = 0x0001                                     # exponent 0
    cb = np.array([127] + list(range(1, 16)), dtype=np.uint8)
    s = oracle.encode(data, oracle.BF16, cb)
    sec = streamfmt.sections(s)
    assert list(sec["counts"]) == [2, 2]
    assert list(sec["pos"]) == [5, 65535, 0, 2]
    assert list(sec["exp"]) == [0, 0, 0, 0]
    assert sec["codes"][65536 + 1] == 0 and sec["codes"][65536 + 2] == 0
    assert np.array_equal(oracle.decode(s, oracle.BF16, n), data)


def _check_invariants(data, dtype, cb, s):
    sec = streamfmt.sections(s)
    h = sec["header"]
    n = data.size
    assert h["magic"] == 0x50495A53 and h["version"] == 1 and h["log2_block"] == 16
    assert h["n"] == n and h["dtype"] == dtype and h["nb"] == (n + 65535) // 65536
    assert np.array_equal(h["codebook"], cb)
    assert s.size == sec["size"]
    for a, b in streamfmt.padding_ranges(s):
        assert not s[a:b].any(), (a, b)
    assert not sec["tail_code"].any() and not sec["sm_tail"].any()
    if dtype == 0:
        expo = (data >> 7) & 0xFF
    else:
        expo = (data >> 2) & 0x1F
    in_cb = np.isin(expo, cb)
    per_block = [int((~in_cb[b:b + 65536]).sum()) for b in range(0, n, 65536)]
    assert list(sec["counts"]) == per_block
    assert h["escapes"] == int((~in_cb).sum()) == int(sec["counts"].sum())
    idx = np.nonzero(~in_cb)[0]
    assert np.array_equal(sec["pos"], idx % 65536)
    assert np.array_equal(sec["exp"], expo[idx])
    assert np.all(sec["codes"][idx] == 0)
    ok = np.nonzero(in_cb)[0]
    assert np.array_equal(cb[sec["codes"][ok]], expo[ok])


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(n=st.one_of(st.integers(0, 40), st.sampled_from([65535, 65536, 65537, 131071, 131072 + 9])),
       seed=st.integers(0, 2 ** 31 - 1), dtype=st.sampled_from([0, 1]),
       mode=st.sampled_from(["random_cb", "calibrated", "narrow"]))
def test_roundtrip_and_invariants_fuzz(n, seed, dtype, mode):
    rng = np.random.default_rng(seed)
    if dtype == 0:
        data = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
        if mode == "narrow" and n:
            data = ((data & 0x807F) | (rng.integers(120, 136, n).astype(np.uint16) << 7)).astype(np.uint16)
        symbols = 256
    else:
        data = rng.integers(0, 256, n, dtype=np.uint32).astype(np.uint8)
        if mode == "narrow" and n:
            data = ((data & 0x83) | (rng.integers(8, 26, n).astype(np.uint8) << 2)).astype(np.uint8)
        symbols = 32
    if mode == "random_cb":
        cb = rng.permutation(symbols)[:16].astype(np.uint8)
    else:
        cb = oracle.calibrate(data, dtype)
    s = oracle.encode(data, dtype, cb)
    _check_invariants(data, dtype, cb, s)
    assert np.array_equal(oracle.decode(s, dtype, n), data)
    assert oracle.check_canonical(s, dtype, n) == 0


def test_workload_escape_rates_small():
    """Stress workloads at reduced size keep their defining properties."""
    cb = oracle.calibrate(synth.as_bits_numpy(synth.calibration_tensor("kv1m")), oracle.BF16)
    assert 127 in cb
    one = synth.as_bits_numpy(synth.workload("stress_oneexp", size="small")[0])
    assert oracle.count_escapes(one, oracle.BF16, cb) == 0
    rnd = synth.as_bits_numpy(synth.workload("stress_random", size="small")[0])
    p = 1 - 16 / 255
    sigma = math.sqrt(p * (1 - p) / rnd.size)
    rate = oracle.count_escapes(rnd, oracle.BF16, cb) / rnd.size
    assert abs(rate - p) < 5 * sigma


def _valid_stream():
    data = np.full(70000, 0x3F80, dtype=np.uint16)
    data[[3, 9, 66000]] = 0x0001
    cb = np.array([127] + list(range(1, 16)), dtype=np.uint8)
    return data, cb, oracle.encode(data, oracle.BF16, cb)


def test_error_injection():
    data, cb, s = _valid_stream()
    n = data.size
    assert oracle.validate(s, 0, n) == 0
    L = streamfmt.layout(0, n)

    def bad(mutate, expect=oracle.E_FORMAT, dtype=0, nn=n, trunc=None):
        t = s.copy() if trunc is None else s[:trunc].copy()
        mutate(t)
        rc, _ = oracle.decode_rc(t, dtype, nn)
        assert rc == expect

    bad(lambda t: t.__setitem__(0, 0))                          # magic
    bad(lambda t: t.__setitem__(4, 2))                          # version
    bad(lambda t: None, expect=oracle.E_DTYPE, dtype=1)         # dtype
    bad(lambda t: None, nn=n - 1)                               # N mismatch
    bad(lambda t: t.__setitem__(16, 4))                         # sum(counts) != E
    bad(lambda t: t.__setitem__(64, 3))                         # count vs E
    bad(lambda t: None, trunc=s.size - 1)                       # truncated
    first = L["off_esc"]
    bad(lambda t: t.__setitem__(slice(first, first + 2), [9, 0]))      # pos 9 then 9
    bad(lambda t: t.__setitem__(slice(first + 3, first + 5), [2, 0]))  # descending
    last = first + 6                                            # block 1, len 4464
    bad(lambda t: t.__setitem__(slice(last, last + 2), [0xFF, 0xFF]))  # pos >= len
    bad(lambda t: t.__setitem__(32, 40), expect=0)              # cb entry changes nothing structural
    # encoder-side errors
    assert oracle.encode_rc(data, 0, cb, s.size - 1) == oracle.E_CAPACITY
    dup = cb.copy()
    dup[1] = dup[0]
    assert oracle.encode_rc(data, 0, dup, s.size) == oracle.E_ARG
    assert oracle.encode_rc(data, 5, cb, s.size) == oracle.E_DTYPE
    big = cb.copy()
    big[3] = 40
    assert oracle.encode_rc(data.astype(np.uint8), 1, big, 10 ** 6) == oracle.E_ARG
    # a non-canonical but valid stream: escape record whose exponent is coded
    t = s.copy()
    t[first + 2] = 127
    assert oracle.validate(t, 0, n) == 0
    assert oracle.check_canonical(t, 0, n) == 1
