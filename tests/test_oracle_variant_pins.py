"""Pins for the oracle of the two ablation formats (BF16 only): version 2,
Top-8 (3-bit codes, position records) and version 3, Top-15 with code 15 as
escape sentinel (one exponent byte per escape, no positions).  The page
weighs both against its Top-16 design (gist.science summary of "SplitZip:
Ultra Fast Lossless KV Compression for Disaggregated LLM Serving", Method,
decoding "design choice" bullet; Results, ablations).

Checked against facts that do not come from the oracle: hand-worked streams,
closed-form sizes, brute force over every BF16 pattern, numpy's unpackbits /
isin / bincount views of the sections, and error injection.
"""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import synth
from tests.test_oracle_pins import _load_golden

import torch

BLOCK = 65536


def _layout(version, n):
    a = lambda x: (x + 255) // 256 * 256
    nb = (n + BLOCK - 1) // BLOCK
    code_bytes = 3 * ((n + 7) // 8) if version == 2 else (n + 1) // 2
    off_code = a(64 + 4 * nb)
    off_sm = off_code + a(code_bytes)
    return dict(nb=nb, off_code=off_code, code_bytes=code_bytes, off_sm=off_sm, off_esc=off_sm + a(n))


def _codes_of(stream, version, n):
    L = _layout(version, n)
    sec = stream[L["off_code"]:L["off_code"] + L["code_bytes"]]
    if version == 2:
        bits = np.unpackbits(sec, bitorder="little")[:3 * n].reshape(n, 3).astype(np.int64)
        return bits[:, 0] | (bits[:, 1] << 1) | (bits[:, 2] << 2)
    codes = np.empty(2 * sec.size, dtype=np.int64)
    codes[0::2], codes[1::2] = sec & 0xF, sec >> 4
    return codes[:n]


@pytest.mark.parametrize("name", ["bf16_five_values_top8.txt", "bf16_five_values_top15s.txt"])
def test_golden_hand_worked_variant_stream(name):
    fields, expect = _load_golden(name)
    version = int(fields["version"][0])
    floats = torch.tensor([float(x) for x in fields["values_float"]], dtype=torch.float32)
    bits = np.array([int(x, 16) for x in fields["values_hex"]], dtype=np.uint16)
    assert np.array_equal(synth.as_bits_numpy(floats.to(torch.bfloat16)), bits)
    cb = [int(x, 16) for x in fields["codebook"]]
    assert len(cb) == oracle.BOOK_ENTRIES[version]
    got = oracle.encode_variant(bits, version, cb)
    assert got.size == expect.size
    assert np.array_equal(got, expect), np.nonzero(got != expect)
    assert np.array_equal(oracle.decode_variant(got, version, bits.size), bits)


def test_all_bf16_patterns_variants():
    """Every BF16 pattern once, book 0..15 (the calibration of this input):
    an exponent v escapes iff v >= 8 (Top-8) or v >= 15 (Top-15)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    expo = (bits >> 7) & 0xFF
    assert list(oracle.calibrate(bits, oracle.BF16)) == list(range(16))
    # Top-8
    s = oracle.encode_variant(bits, 2, list(range(8)))
    assert s.size == 280832 and int(s[16:24].view(np.uint64)[0]) == 65536 - 8 * 256 == 63488
    L = _layout(2, 65536)
    esc = expo >= 8
    codes = _codes_of(s, 2, 65536)
    assert np.array_equal(codes, np.where(esc, 0, expo))
    rec = s[L["off_esc"]:].reshape(-1, 3).astype(np.int64)
    assert np.array_equal(rec[:, 0] | (rec[:, 1] << 8), np.nonzero(esc)[0])
    assert np.array_equal(rec[:, 2], expo[esc])
    assert np.array_equal(s[L["off_sm"]:L["off_sm"] + 65536], ((bits >> 8) & 0x80) | (bits & 0x7F))
    # Top-15 + sentinel
    s = oracle.encode_variant(bits, 3, list(range(15)))
    assert s.size == 160256 and int(s[16:24].view(np.uint64)[0]) == 65536 - 15 * 256 == 61696
    L = _layout(3, 65536)
    esc = expo >= 15
    assert np.array_equal(_codes_of(s, 3, 65536), np.where(esc, 15, expo))
    assert np.array_equal(s[L["off_esc"]:], expo[esc].astype(np.uint8))
    for v in (2, 3):
        book = list(range(oracle.BOOK_ENTRIES[v]))
        assert np.array_equal(oracle.decode_variant(oracle.encode_variant(bits, v, book), v, 65536), bits)


def test_variant_size_closed_forms():
    n = 1 << 29
    # Top-8: 64 + 4*8192 -> 33,024; 3 * 2^26 code bytes; 2^29 sign/mantissa bytes
    assert oracle.encoded_size_variant(2, n, 0) == 33024 + 201326592 + 536870912 == 738230528
    assert oracle.encoded_size_variant(2, n, 10) == 738230528 + 30
    # Top-15 + sentinel: the Top-16 sections, one byte per escape
    assert oracle.encoded_size_variant(3, n, 0) == 805339392
    assert oracle.encoded_size_variant(3, n, 10) == 805339392 + 10
    assert oracle.encoded_size_variant(1, n, 10) == 805339392 + 30
    # payload ratio at zero escapes: 16 bits -> 3 + 8 bits (Top-8), -> 4 + 8 bits (Top-15)
    assert abs(2 * n / 738230528 - 16 / 11) < 1e-4
    assert oracle.encoded_size_variant(2, 0, 0) == 256 and oracle.encoded_size_variant(3, 0, 0) == 256   # header only


@pytest.mark.parametrize("version", [2, 3])
def test_variant_sections_on_kv_data(version):
    """Sections of a KV-like tensor read back with numpy: codes = book index
    (0 for Top-8 escapes, 15 for sentinels), escapes exactly where isin says,
    per-block counts from bincount of the escape positions, and E from the
    exponent histogram."""
    x, _ = synth.workload("llama3_8b_kv", size="small")
    bits = synth.as_bits_numpy(x)[: 3 * BLOCK + 4321]
    n = bits.size
    book = list(oracle.calibrate(synth.as_bits_numpy(synth.calibration_tensor("llama3_8b_kv")), 0))
    book = book[:oracle.BOOK_ENTRIES[version]]
    s = oracle.encode_variant(bits, version, book)
    L = _layout(version, n)
    expo = ((bits >> 7) & 0xFF).astype(np.int64)
    esc = ~np.isin(expo, book)
    index = {v: c for c, v in enumerate(book)}
    want_codes = np.array([index.get(int(v), 0 if version == 2 else 15) for v in expo])
    assert np.array_equal(_codes_of(s, version, n), want_codes)
    hist = np.bincount(expo, minlength=256)
    E = int(s[16:24].view(np.uint64)[0])
    assert E == n - int(hist[book].sum()) == int(esc.sum())
    counts = s[64:64 + 4 * L["nb"]].view(np.uint32)
    assert np.array_equal(counts, np.bincount(np.nonzero(esc)[0] // BLOCK, minlength=L["nb"]))
    if version == 2:
        rec = s[L["off_esc"]:].reshape(-1, 3).astype(np.int64)
        assert np.array_equal(rec[:, 0] | (rec[:, 1] << 8), np.nonzero(esc)[0] % BLOCK)
        assert np.array_equal(rec[:, 2], expo[esc])
    else:
        assert np.array_equal(s[L["off_esc"]:], expo[esc].astype(np.uint8))
    assert np.array_equal(oracle.decode_variant(s, version, n), bits)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(st.data())
def test_variant_roundtrip_fuzz(data):
    version = data.draw(st.sampled_from([2, 3]))
    n = data.draw(st.one_of(st.integers(0, 40), st.sampled_from([65535, 65536, 65537, 2 * 65536 + 9])))
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    kind = data.draw(st.sampled_from(["random", "narrow"]))
    if kind == "random":
        bits = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
    else:
        e = rng.integers(118, 136, n)
        bits = ((rng.integers(0, 2, n) << 15) | (e << 7) | rng.integers(0, 128, n)).astype(np.uint16)
    k = oracle.BOOK_ENTRIES[version]
    book = list(rng.permutation(256)[:k])
    s = oracle.encode_variant(bits, version, book)
    assert s.size == oracle.encoded_size_variant(version, n, oracle.count_escapes_variant(version, bits, book))
    assert oracle.validate_variant(s, version, n) == 0
    assert np.array_equal(oracle.decode_variant(s, version, n), bits)
    L = _layout(version, n)
    pad = np.concatenate([s[64 + 4 * L["nb"]:L["off_code"]],
                          s[L["off_code"] + L["code_bytes"]:L["off_sm"]], s[L["off_sm"] + n:L["off_esc"]]])
    assert not pad.any()


def test_variant_error_injection():
    x, _ = synth.workload("stress_t3", size="small")
    bits = synth.as_bits_numpy(x)[:2 * BLOCK + 100]
    n = bits.size
    book = list(range(118, 133))
    for version in (2, 3):
        s = oracle.encode_variant(bits, version, book[:oracle.BOOK_ENTRIES[version]])
        L = _layout(version, n)
        assert oracle.validate_variant(s, version, n) == 0

        def bad(mutate, code=-5):
            t = s.copy()
            t = mutate(t)
            assert oracle.validate_variant(t, version, n) == code
            assert oracle.decode_variant_rc(t, version, n)[0] == code

        bad(lambda t: np.concatenate([t[:4], np.array([1, 0], np.uint8), t[6:]]))       # version 1 header
        bad(lambda t: (t.__setitem__(6, 1), t)[1], -2)                                  # dtype E5M2
        bad(lambda t: (t.__setitem__(47, 5), t)[1])                                     # unused book byte
        bad(lambda t: t[:-1])                                                           # truncated
        bad(lambda t: (t.__setitem__(64, t[64] + 1), t)[1])                             # count != E
        if version == 3:
            # an extra sentinel in block 0 without a count to match
            def extra_sentinel(t):
                codes = _codes_of(t, 3, n)
                i = int(np.nonzero(codes != 15)[0][0])
                t[L["off_code"] + i // 2] |= 0xF << (4 * (i % 2))
                return t
            bad(extra_sentinel)
        else:
            def descending(t):
                r = L["off_esc"]
                t[r:r + 6] = np.concatenate([t[r + 3:r + 6], t[r:r + 3]])
                return t
            bad(descending)
        # a repeated book entry is refused by the encoder
        with pytest.raises(ValueError):
            oracle.encode_variant(bits, version, [7] * oracle.BOOK_ENTRIES[version])
