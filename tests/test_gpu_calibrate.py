"""On-device calibration (sz_calibrate_device) and encode with a device
codebook (sz_encode_devcb), against the CPU oracle.

The device histogram must equal the oracle's histogram of the sampled blocks
(64K blocks 0, s, 2s, ...) exactly, the device codebook the oracle's Top-16
of that sample, and a stream encoded with the device codebook must equal the
oracle's stream for that codebook byte for byte.  At full size the histogram
is also checked against torch.bincount of the exponent field, which shares
nothing with either implementation.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

BLOCK = 65536


def _sz():
    import fp8_kv_cache_sz_amd as sz
    return sz


def _dev(bits, dtype):
    t = torch.from_numpy(bits.copy())
    if dtype == 0:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def _sample(bits, every):
    nb = (bits.size + BLOCK - 1) // BLOCK
    parts = [bits[b * BLOCK:(b + 1) * BLOCK] for b in range(0, nb, every)]
    return np.concatenate(parts) if parts else bits[:0]


def _check_calibration(bits, dtype, every):
    sz = _sz()
    print("calibrate_device n=%d dtype=%d every=%d" % (bits.size, dtype, every), flush=True)
    x = _dev(bits, dtype)
    out = torch.full((sz.DEVICE_CODEBOOK_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
    d_cb, d_hist = sz.calibrate_device(x, sample_every=every, out=out, hist=True)
    torch.cuda.synchronize()
    sample = _sample(bits, every)
    want_hist = oracle.histogram(sample, dtype)
    want_cb = oracle.calibrate(sample, dtype)
    assert np.array_equal(d_hist.cpu().numpy().astype(np.uint64), want_hist)
    cb = sz.codebook_from_device(d_cb)
    assert cb.dtype == dtype
    assert list(cb.exps) == list(want_cb)
    assert np.all(d_cb[20:].cpu().numpy() == 0xA5)        # nothing past the sz_codebook written
    return d_cb, want_cb


SIZES = [0, 1, 2, 4095, 4096, 4097, 65535, 65536, 65537, 5 * 65536 + 777, 13 * 65536]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype", [0, 1])
def test_histogram_and_codebook_random_bits(n, dtype):
    bits = synth.as_bits_numpy(synth.random_bits(300 + n % 97, n, dtype))
    _check_calibration(bits, dtype, 1)


@pytest.mark.parametrize("every", [1, 2, 3, 7, 100])
@pytest.mark.parametrize("dtype", [0, 1])
def test_sampled_blocks(every, dtype):
    x, _ = synth.workload("llama3_8b_kv" if dtype == 0 else "llama3_8b_kv_e5m2", size="small")
    bits = synth.as_bits_numpy(x)
    _check_calibration(bits, dtype, every)


def test_all_patterns_tie_break():
    """Every BF16 pattern once: all 256 exponents tie at 256, so the book is
    0..15 by the exponent-ascending tie-break; likewise for E5M2."""
    d_cb, cb = _check_calibration(np.arange(65536, dtype=np.uint32).astype(np.uint16), 0, 1)
    assert list(cb) == list(range(16))
    d_cb, cb = _check_calibration(np.arange(256, dtype=np.uint32).astype(np.uint8), 1, 1)
    assert list(cb) == list(range(16))


@pytest.mark.parametrize("dtype", [0, 1])
def test_encode_with_device_codebook(dtype):
    """calibrate_device -> encode on the same stream, no host round trip: the
    stream equals the oracle's for the oracle's own calibration, and the
    host-codebook encode's."""
    sz = _sz()
    x, _ = synth.workload("stress_t3" if dtype == 0 else "llama3_8b_kv_e5m2", size="small")
    bits = synth.as_bits_numpy(x)
    xd = _dev(bits, dtype)
    d_cb = sz.calibrate_device(xd)
    buf, size, esc = sz.encode(xd, d_cb)
    cb = oracle.calibrate(bits, dtype)
    expect = oracle.encode(bits, dtype, cb)
    assert size == expect.size
    assert np.array_equal(buf[:size].cpu().numpy(), expect)
    buf2, size2, _ = sz.encode(xd, sz.Codebook(dtype, tuple(int(v) for v in cb)))
    assert size2 == size and torch.equal(buf2[:size2], buf[:size])
    y = sz.decode(buf[:size], dtype, bits.size)
    assert np.array_equal(synth.as_bits_numpy(y), bits)


@pytest.mark.parametrize("dtype", [0, 1])
def test_device_codebook_is_checked(dtype):
    """A device codebook with a repeated entry, an entry out of range (E5M2:
    32; a BF16 byte cannot be out of range) or the other dtype's word sets
    the status word and leaves a stream that decode rejects."""
    sz = _sz()
    bits = synth.as_bits_numpy(synth.random_bits(7, 70000, dtype))
    xd = _dev(bits, dtype)
    good = list(range(16))
    cases = [(dtype, good[:15] + [3], -1), (1 - dtype, good, -2)]
    if dtype == 1:
        cases.append((dtype, good[:15] + [32], -1))
    for word, exps, code in cases:
        raw = np.zeros(sz.DEVICE_CODEBOOK_BYTES, dtype=np.uint8)
        raw[:4] = np.array([word], dtype=np.uint32).view(np.uint8)
        raw[4:20] = np.array(exps, dtype=np.uint8)
        d_cb = torch.from_numpy(raw).cuda()
        with pytest.raises(sz.SplitZipError) as e:
            sz.encode(xd, d_cb)
        assert e.value.code == code
        buf, _, _ = sz.encode(xd, d_cb, sync=False)
        torch.cuda.synchronize()
        with pytest.raises(sz.SplitZipError) as e:
            sz.decode(buf, dtype, bits.size)
        assert e.value.code == -5


@pytest.mark.parametrize("name", ["llama3_8b_kv", "llama3_8b_kv_e5m2"])
def test_full_size_calibration(name):
    """The full workload: device histogram = torch.bincount of the exponent
    field; device codebook = the oracle's Top-16 of the whole tensor."""
    sz = _sz()
    torch.cuda.empty_cache()
    x, dtype = synth.workload(name, device="cuda")
    print("full-size calibration", name, flush=True)
    d_cb, d_hist = sz.calibrate_device(x, hist=True)
    if dtype == 0:
        expo = (x.view(torch.int16).to(torch.int32) >> 7) & 0xFF
        want = torch.bincount(expo, minlength=256)
    else:
        expo = (x.view(torch.uint8).to(torch.int32) >> 2) & 0x1F
        want = torch.bincount(expo, minlength=32)
    del expo
    assert torch.equal(d_hist, want)
    bits = synth.as_bits_numpy(x)
    del x
    assert list(sz.codebook_from_device(d_cb).exps) == list(oracle.calibrate(bits, dtype))
    torch.cuda.empty_cache()
