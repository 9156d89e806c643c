"""sz_decode_noalloc (decode with its scratch in the library's fixed device
array) against sz_decode (decode with a caller workspace), through the C ABI:
the decoded values and the status word must be identical, on two calls in a
row, the second on a smaller stream, so that what the first call left in the
shared array cannot leak into the second."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

POISON = 0xA5


def _decode_both(sz, nat, buf, size, dtype, n):
    """(values, status) from sz_decode and from sz_decode_noalloc, each into
    its own poison-filled output."""
    elem = 2 if dtype == 0 else 1
    stream = torch.cuda.current_stream().cuda_stream
    out_ws = torch.full((n * elem + 64,), POISON, dtype=torch.uint8, device="cuda")
    ws = torch.full((sz.decode_workspace_size(dtype, n),), POISON, dtype=torch.uint8, device="cuda")
    rc = nat.sz_decode(buf.data_ptr(), size, dtype, out_ws.data_ptr(), n, ws.data_ptr(), ws.numel(), stream)
    assert rc == 0
    out_na = torch.full((n * elem + 64,), POISON, dtype=torch.uint8, device="cuda")
    status = torch.full((4,), -99, dtype=torch.int32, device="cuda")
    rc = nat.sz_decode_noalloc(buf.data_ptr(), size, dtype, out_na.data_ptr(), n, status.data_ptr(), stream)
    assert rc == 0
    torch.cuda.synchronize()
    return (out_ws.cpu().numpy(), int(ws[:4].cpu().view(torch.int32)[0]),
            out_na.cpu().numpy(), int(status[0].cpu()), status[1:].cpu().numpy())


@pytest.mark.parametrize("dtype, sizes", [(0, (9 * 65536 + 4321, 3 * 65536 + 77)),
                                          (0, (1100 * 65536 + 5, 70000)),
                                          (1, (5 * 65536 + 123, 65536 + 9))])
def test_noalloc_matches_workspace_decode(dtype, sizes):
    import fp8_kv_cache_sz_amd as sz
    from fp8_kv_cache_sz_amd import _native as nat
    cal = synth.calibration_tensor("kv1m" if dtype == 0 else "llama3_8b_kv_e5m2")
    cb = sz.calibrate(cal)
    for call, n in enumerate(sizes):
        print("noalloc dtype=%d call=%d n=%d" % (dtype, call, n), flush=True)
        if dtype == 0:
            x = synth.student_t_with_random_exponents(60 + call, n, device="cuda")
        else:
            x = synth.random_bits(60 + call, n, dtype=1, device="cuda")
        buf, size, esc = sz.encode(x, cb)
        vals_ws, st_ws, vals_na, st_na, untouched = _decode_both(sz, nat, buf, size, dtype, n)
        assert st_ws == 0 and st_na == 0
        assert np.array_equal(vals_na, vals_ws)
        assert np.array_equal(vals_na[:n * (2 - dtype)], synth.as_bits_numpy(x).view(np.uint8))
        assert np.all(vals_na[n * (2 - dtype):] == POISON)
        assert np.all(untouched == -99)          # only the first word of d_status is written


def test_noalloc_reports_a_bad_stream_like_sz_decode():
    """A stream whose escape count disagrees with its header: both entry
    points report the same device verdict, also right after a clean call."""
    import fp8_kv_cache_sz_amd as sz
    from fp8_kv_cache_sz_amd import _native as nat
    cb = sz.calibrate(synth.calibration_tensor("kv1m"))
    n = 4 * 65536 + 11
    x = synth.student_t_with_random_exponents(70, n, device="cuda")
    buf, size, _ = sz.encode(x, cb)
    _, st_ws, _, st_na, _ = _decode_both(sz, nat, buf, size, 0, n)
    assert st_ws == 0 and st_na == 0
    bad = buf[:size].clone()
    bad[64] += 1                                   # first block's escape count
    _, st_ws, _, st_na, _ = _decode_both(sz, nat, bad, size, 0, n)
    assert st_ws == st_na == -5
