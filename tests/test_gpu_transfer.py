"""Chunked transfer through pinned host memory (sz_transfer), compressed and
raw.  The received tensor must equal the sent one bit for bit; with
compression, the bytes that crossed the link must add up to the oracle's
stream size of every chunk, and the streams still held in the host wire
slots must equal the oracle's encoding of their chunks byte for byte."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _sz():
    import fp8_kv_cache_sz_amd as sz
    return sz


def _slot_bytes(sz, dtype, chunk):
    return (sz.encoded_size(dtype, chunk, chunk) + 255) // 256 * 256


CASES = [
    # (dtype, n, chunk, depth)
    (0, 0, 4096, 2),
    (0, 1000, 4096, 2),
    (0, 5 * 65536 + 123, 65536, 3),
    (0, 3 * 100000, 100000, 2),
    (0, 2_000_000, 131072, 4),
    (1, 777_777, 65536, 3),
    (1, 4096, 4096, 1),
]


@pytest.mark.parametrize("dtype,n,chunk,depth", CASES)
def test_transfer_compressed(dtype, n, chunk, depth):
    sz = _sz()
    print("transfer dtype=%d n=%d chunk=%d depth=%d" % (dtype, n, chunk, depth), flush=True)
    if dtype == 0:
        x = synth.kv_layer(11, tokens=(n + 1023) // 1024 + 1).reshape(-1)[:n].contiguous()
        cal = synth.calibration_tensor("kv1m")
    else:
        x = synth.kv_cache_e5m2(12, 1, (n + 2047) // 2048 + 1, 8, 128).reshape(-1)[:n].contiguous()
        cal = synth.calibration_tensor("llama3_8b_kv_e5m2")
    cb = sz.calibrate(cal)
    xd = x.cuda()
    staging = sz.transfer_buffers(dtype, n, chunk, depth)
    out = torch.full_like(xd, 0) if n else torch.empty_like(xd)
    got, st = sz.transfer(xd, chunk, cb, depth=depth, out=out, staging=staging)
    bits = synth.as_bits_numpy(x)
    assert np.array_equal(synth.as_bits_numpy(got), bits)
    chunks = (n + chunk - 1) // chunk
    assert st["chunks"] == chunks and st["decode_status"] == 0
    assert st["raw_bytes"] == n * (2 if dtype == 0 else 1)
    sizes, escs = [], []
    for i in range(chunks):
        part = bits[i * chunk:(i + 1) * chunk]
        e = oracle.count_escapes(part, dtype, list(cb.exps))
        escs.append(e)
        sizes.append(oracle.encoded_size(dtype, part.size, e))
    assert st["wire_bytes"] == sum(sizes) and st["escapes"] == sum(escs)
    # the last `depth` chunks' streams are still in their wire slots
    h = staging[0].numpy()
    slot = _slot_bytes(sz, dtype, chunk)
    for i in range(max(0, chunks - depth), chunks):
        k = i % depth
        part = bits[i * chunk:(i + 1) * chunk]
        want = oracle.encode(part, dtype, list(cb.exps))
        assert np.array_equal(h[k * slot:k * slot + want.size], want), i


@pytest.mark.parametrize("dtype,n,chunk,depth", CASES[:4] + CASES[5:6])
def test_transfer_raw(dtype, n, chunk, depth):
    sz = _sz()
    if dtype == 0:
        x = synth.random_bits(13, n, 0)
    else:
        x = synth.random_bits(14, n, 1)
    xd = x.cuda()
    got, st = sz.transfer(xd, chunk, None, depth=depth)
    assert torch.equal(got.view(torch.uint8), xd.view(torch.uint8))
    assert st["wire_bytes"] == st["raw_bytes"] == n * (2 if dtype == 0 else 1)


def test_transfer_full_llama3_kv_by_layer():
    """The 1 GiB Llama-3-8B KV cache, one layer (K and V) per chunk."""
    sz = _sz()
    torch.cuda.empty_cache()
    x, dtype = synth.workload("llama3_8b_kv", device="cuda")
    cb = sz.calibrate(synth.calibration_tensor("llama3_8b_kv"))
    layer = 2 * 8192 * 8 * 128
    got, st = sz.transfer(x, layer, cb, depth=3)
    print("full transfer: %.2f ms, wire %d of %d bytes" % (st["total_ms"], st["wire_bytes"], st["raw_bytes"]),
          flush=True)
    assert torch.equal(got.view(torch.int16), x.view(torch.int16))
    assert st["chunks"] == 32 and st["decode_status"] == 0
    assert st["escapes"] == sz.read_escape_count(sz.encode(x, cb)[0])
    del got, x
    torch.cuda.empty_cache()
