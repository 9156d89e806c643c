"""CPU checks of the C-ABI library: it loads, exports every call that
include/splitzip.h declares, and its host-side logic (calibration, sizes,
argument checks that fail before any launch) agrees with the oracle and the
format's closed forms.  No GPU work is started here."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _native():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_splitzip_build", os.path.join(ROOT, "fp8_kv_cache_sz_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    if not os.path.exists(build.LIBRARY):
        build.build()
    from fp8_kv_cache_sz_amd import _native
    return _native


def declared_functions():
    text = open(os.path.join(ROOT, "include", "splitzip.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|uint64_t|void)\s*\*?\s*(sz_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    nat = _native()
    names = declared_functions()
    assert {"sz_calibrate", "sz_encoded_size", "sz_workspace_size", "sz_encode", "sz_decode"} <= set(names)
    for name in names:
        assert hasattr(nat.lib, name), name
    assert set(names) == set(nat.EXPORTS)


def test_header_is_plain_c(tmp_path):
    """include/splitzip.h is a C header: a C11 program that takes the address
    of every declared call compiles with -pedantic -Werror and links against
    the library."""
    import shutil
    import subprocess
    nat = _native()
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = tmp_path / "abi.c"
    src.write_text('#include "splitzip.h"\n#include <stddef.h>\n'
                   "typedef void (*any_call)(void);\n"
                   "any_call const calls[] = {\n" + ",\n".join("    (any_call)%s" % n for n in names) + "\n};\n"
                   "int main(void) { size_t k = 0; for (size_t i = 0; i < sizeof calls / sizeof calls[0]; ++i) "
                   "k += calls[i] != NULL; return k == sizeof calls / sizeof calls[0] ? 0 : 1; }\n")
    lib_dir = os.path.dirname(nat.LIBRARY)
    exe = tmp_path / "abi"
    subprocess.check_call([gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                           "-I", os.path.join(ROOT, "include"), str(src), "-L", lib_dir, "-lsplitzip",
                           "-Wl,-rpath," + lib_dir, "-o", str(exe)])
    assert os.path.exists(exe)


def test_encoded_size_matches_oracle():
    nat = _native()
    for dtype in (0, 1):
        for n in (0, 1, 2, 7, 8, 9, 255, 256, 65535, 65536, 65537, 1 << 20, (1 << 29) + 3, 1879048192):
            for e in (0, 1, n // 3, n):
                assert nat.sz_encoded_size(dtype, n, e) == oracle.encoded_size(dtype, n, e), (dtype, n, e)
    assert nat.sz_encoded_size(9, 10, 0) == 0
    assert nat.sz_workspace_size(9, 10) == 0
    up = lambda x: (x + 255) // 256 * 256
    for dtype in (0, 1):
        for n in (0, 1, 1 << 20, (1 << 25) - 1, 1 << 25, (1 << 25) + 1, 1879048192):
            ws = nat.sz_workspace_size(dtype, n)
            nt, nb = (n + 16383) // 16384, (n + 65535) // 65536
            assert ws % 256 == 0
            # status, tile counts, block offsets, the scan workgroups' escape
            # totals and flagged-tile words (one u64 and sixteen u32 per 8,192
            # blocks), then one staging slot per 16K
            # tile: 3 bytes per element up to 2,048 tiles, 12 KB per tile
            # (4,096 records) above
            slot = 3 * 16384 if nt <= 2048 else 3 * 4096
            groups = (nb + 8191) // 8192
            fixed = 256 + up(4 * nt + 16) + up(8 * nb + 16) + up(8 * groups) + up(64 * groups)
            assert ws == fixed + up(slot * nt + 16), (dtype, n)
            dws = nat.sz_decode_workspace_size(dtype, n)
            assert dws == 256 + up(8 * nb + 16) and dws <= ws
            if dtype == 0:
                assert nat.sz_workspace_size_format(1, 0, n) == ws
                assert nat.sz_workspace_size_format(2, 0, n) == fixed + up(3 * 16384 * nt + 16)
                assert nat.sz_workspace_size_format(3, 0, n) == fixed + up(16384 * nt + 16)
            else:
                assert nat.sz_workspace_size_format(2, 1, n) == 0 and nat.sz_workspace_size_format(3, 1, n) == 0
    assert nat.sz_decode_workspace_size(9, 10) == 0 and nat.sz_workspace_size_format(4, 0, 10) == 0


@pytest.mark.parametrize("source", ["kv1m", "bruteforce", "random_cb_data", "empty"])
@pytest.mark.parametrize("dtype", [0, 1])
def test_calibrate_matches_oracle(source, dtype):
    nat = _native()
    if source == "kv1m":
        if dtype == 0:
            data = synth.as_bits_numpy(synth.calibration_tensor("kv1m"))
        else:
            data = synth.as_bits_numpy(synth.calibration_tensor("llama3_8b_kv_e5m2"))
    elif source == "bruteforce":
        data = np.arange(65536 if dtype == 0 else 256, dtype=np.uint32).astype(np.uint16 if dtype == 0 else np.uint8)
    elif source == "random_cb_data":
        rng = np.random.default_rng(3)
        data = rng.integers(0, 1 << (16 if dtype == 0 else 8), 50000).astype(np.uint16 if dtype == 0 else np.uint8)
    else:
        data = np.zeros(0, dtype=np.uint16 if dtype == 0 else np.uint8)
    ptr = data.ctypes.data if data.size else None
    cb = nat.sz_calibrate(dtype, ptr, data.size)
    assert cb.dtype == dtype
    assert list(cb.exp) == list(oracle.calibrate(data, dtype))


def test_host_argument_checks():
    nat = _native()
    cb = nat.sz_codebook()
    cb.dtype = 0
    for c in range(16):
        cb.exp[c] = 120 + c
    dummy = 1 << 20        # never dereferenced: every call below fails a host check first
    assert nat.sz_encode(5, dummy, 16, cb, dummy, 1 << 30, dummy, 1 << 30, None) == -2
    cb.dtype = 1
    assert nat.sz_encode(0, dummy, 16, cb, dummy, 1 << 30, dummy, 1 << 30, None) == -2
    cb.dtype = 0
    cb.exp[3] = cb.exp[2]
    assert nat.sz_encode(0, dummy, 16, cb, dummy, 1 << 30, dummy, 1 << 30, None) == -1
    cb.exp[3] = 123
    assert nat.sz_encode(0, None, 16, cb, dummy, 1 << 30, dummy, 1 << 30, None) == -1
    assert nat.sz_encode(0, dummy + 2, 16, cb, dummy, 1 << 30, dummy, 1 << 30, None) == -4
    cap = nat.sz_encoded_size(0, 16, 16)
    assert nat.sz_encode(0, dummy, 16, cb, dummy, cap - 1, dummy, 1 << 30, None) == -3
    ws = nat.sz_workspace_size(0, 16)
    assert nat.sz_encode(0, dummy, 16, cb, dummy, cap, dummy, ws - 1, None) == -7
    assert nat.sz_encode(0, dummy, (1 << 40) + 1, cb, dummy, 1 << 62, dummy, 1 << 62, None) == -1
    # decode: stream shorter than the fixed sections, bad dtype, alignment
    fixed = nat.sz_encoded_size(0, 1000, 0)
    assert nat.sz_decode(dummy, fixed - 1, 0, dummy, 1000, dummy, 1 << 30, None) == -5
    assert nat.sz_decode(dummy, fixed, 3, dummy, 1000, dummy, 1 << 30, None) == -2
    assert nat.sz_decode(dummy + 8, fixed, 0, dummy, 1000, dummy, 1 << 30, None) == -4
    assert nat.sz_decode(dummy, fixed, 0, dummy, 1000, dummy, 16, None) == -7
    dws = nat.sz_decode_workspace_size(0, 1000)
    assert nat.sz_decode(dummy, fixed, 0, dummy, 1000, dummy, dws - 1, None) == -7


def test_host_argument_checks_device_calibration():
    """sz_calibrate_device and sz_encode_devcb reject bad arguments before any
    launch (the pointers are never dereferenced)."""
    nat = _native()
    dummy = 1 << 20
    cws = nat.sz_calibrate_workspace_size(0)
    assert cws == 256 * 512 * 4 and nat.sz_calibrate_workspace_size(1) == 32 * 512 * 4
    assert nat.sz_calibrate_workspace_size(7) == 0
    assert nat.sz_calibrate_device(7, dummy, 16, 1, dummy, None, dummy, cws, None) == -2
    assert nat.sz_calibrate_device(0, dummy, 16, 0, dummy, None, dummy, cws, None) == -1
    assert nat.sz_calibrate_device(0, dummy, 16, 1, None, None, dummy, cws, None) == -1
    assert nat.sz_calibrate_device(0, None, 16, 1, dummy, None, dummy, cws, None) == -1
    assert nat.sz_calibrate_device(0, dummy, 16, 1, dummy + 4, None, dummy, cws, None) == -4
    assert nat.sz_calibrate_device(0, dummy, 16, 1, dummy, dummy + 8, dummy, cws, None) == -4
    assert nat.sz_calibrate_device(0, dummy, 16, 1, dummy, None, dummy, cws - 1, None) == -7
    assert nat.sz_calibrate_device(0, dummy, (1 << 40) + 1, 1, dummy, None, dummy, cws, None) == -1
    cap = nat.sz_encoded_size(1, 16, 16)
    ws = nat.sz_workspace_size(1, 16)
    assert nat.sz_encode_devcb(4, dummy, 16, dummy, dummy, cap, dummy, ws, None) == -2
    assert nat.sz_encode_devcb(1, dummy, 16, None, dummy, cap, dummy, ws, None) == -1
    assert nat.sz_encode_devcb(1, dummy, 16, dummy + 4, dummy, cap, dummy, ws, None) == -4
    assert nat.sz_encode_devcb(1, dummy, 16, dummy, dummy, cap - 1, dummy, ws, None) == -3
    assert nat.sz_encode_devcb(1, dummy, 16, dummy, dummy, cap, dummy, ws - 1, None) == -7


def test_host_argument_checks_formats():
    """sz_encode_format / sz_decode_format / sz_encoded_size_format reject bad
    arguments before any launch, and the sizes match the oracle's."""
    nat = _native()
    dummy = 1 << 20
    cb = nat.sz_codebook()
    cb.dtype = 0
    for c in range(16):
        cb.exp[c] = 120 + c
    for fmt in (2, 3):
        for n, e in [(0, 0), (1, 1), (65537, 300), (1 << 29, 12345)]:
            assert nat.sz_encoded_size_format(fmt, 0, n, e) == oracle.encoded_size_variant(fmt, n, e)
        assert nat.sz_encoded_size_format(fmt, 1, 100, 0) == 0
        cap = nat.sz_encoded_size_format(fmt, 0, 16, 16)
        ws = nat.sz_workspace_size_format(fmt, 0, 16)
        assert nat.sz_encode_format(fmt, 1, dummy, 16, cb, dummy, cap, dummy, ws, None) == -2
        assert nat.sz_decode_format(fmt, dummy, 1 << 20, 1, dummy, 16, dummy, ws, None) == -2
        assert nat.sz_encode_format(fmt, 0, dummy, 16, cb, dummy, cap - 1, dummy, ws, None) == -3
        assert nat.sz_encode_format(fmt, 0, dummy, 16, cb, dummy, cap, dummy, ws - 1, None) == -7
        fixed = nat.sz_encoded_size_format(fmt, 0, 1000, 0)
        assert nat.sz_decode_format(fmt, dummy, fixed - 1, 0, dummy, 1000, dummy, 1 << 30, None) == -5
        # a repeat among the used entries is refused; one beyond them is ignored
        used = 8 if fmt == 2 else 15
        cb.exp[used - 1] = cb.exp[0]
        assert nat.sz_encode_format(fmt, 0, dummy, 16, cb, dummy, cap, dummy, ws, None) == -1
        cb.exp[used - 1] = 120 + used - 1
    assert nat.sz_encoded_size_format(9, 0, 100, 0) == 0
    assert nat.sz_encode_format(9, 0, dummy, 16, cb, dummy, 1 << 30, dummy, 1 << 30, None) == -1
    assert nat.sz_decode_format(0, dummy, 1 << 30, 0, dummy, 16, dummy, 1 << 30, None) == -1
    assert nat.sz_encoded_size_format(1, 0, 1000, 7) == nat.sz_encoded_size(0, 1000, 7)


def test_host_argument_checks_transfer():
    """sz_transfer rejects bad arguments before touching any buffer."""
    nat = _native()
    dummy = 1 << 20
    cb = nat.sz_codebook()
    cb.dtype = 0
    for c in range(16):
        cb.exp[c] = 120 + c
    ws = nat.sz_transfer_workspace_size(0, 65536, 3)
    hb = nat.sz_transfer_host_bytes(0, 1 << 20, 65536, 3)
    slot = (nat.sz_encoded_size(0, 65536, 65536) + 255) // 256 * 256
    assert ws == 2 * 3 * slot + (nat.sz_workspace_size(0, 65536) + 255) // 256 * 256 + \
        (nat.sz_decode_workspace_size(0, 65536) + 255) // 256 * 256
    assert hb == 3 * slot + 3 * 64 + 256
    assert nat.sz_transfer_workspace_size(0, 65536, 0) == 0 and nat.sz_transfer_workspace_size(0, 65536, 9) == 0
    assert nat.sz_transfer_host_bytes(5, 100, 16, 1) == 0
    args = lambda **kw: dict(dict(dtype=0, d_src=dummy, n=1 << 20, chunk=65536, cb=cb, compress=1, depth=3,
                                  h_staging=dummy, h_bytes=hb, d_dst=dummy, d_ws=dummy, ws_bytes=ws,
                                  stream=None), **kw)
    call = lambda **kw: nat.sz_transfer(**args(**kw))[0]
    assert call(dtype=4) == -2
    assert call(depth=0) == -1 and call(depth=9) == -1
    assert call(chunk=0) == -1 and call(chunk=65537) == -1
    assert call(cb=None) == -1 and call(h_staging=None) == -1 and call(d_ws=None) == -1
    assert call(d_src=dummy + 4) == -4 and call(h_staging=dummy + 8) == -4
    assert call(h_bytes=hb - 1) == -7 and call(ws_bytes=ws - 1) == -7


def test_host_argument_checks_reference_copy():
    """sz_reference_copy checks size, pointers, alignment and overlap on the
    host, before any launch."""
    nat = _native()
    a, b = 1 << 20, 1 << 30
    assert nat.sz_reference_copy(None, None, 0, None) == 0           # nothing to copy
    assert nat.sz_reference_copy(a, b, 24, None) == -1                 # not a multiple of 16
    assert nat.sz_reference_copy(None, b, 32, None) == -1
    assert nat.sz_reference_copy(a, None, 32, None) == -1
    assert nat.sz_reference_copy(a + 8, b, 32, None) == -4
    assert nat.sz_reference_copy(a, b + 4, 32, None) == -4
    assert nat.sz_reference_copy(a, a + 16, 32, None) == -1            # overlapping ranges
    assert nat.sz_reference_copy(a + 16, a, 32, None) == -1


def test_host_argument_checks_reference_split():
    """sz_reference_split checks dtype, size, pointers and alignment on the
    host, before any launch."""
    nat = _native()
    a, b, c = 1 << 20, 1 << 30, 1 << 31
    assert nat.sz_reference_split(0, None, 0, None, None, None) == 0    # nothing to do
    assert nat.sz_reference_split(2, a, 16384, b, c, None) == -2
    assert nat.sz_reference_split(0, a, 16384 + 8, b, c, None) == -1     # not whole tiles
    assert nat.sz_reference_split(1, None, 16384, b, c, None) == -1
    assert nat.sz_reference_split(1, a, 16384, None, c, None) == -1
    assert nat.sz_reference_split(1, a, 16384, b, None, None) == -1
    assert nat.sz_reference_split(0, a + 8, 16384, b, c, None) == -4
    assert nat.sz_reference_split(0, a, 16384, b + 4, c, None) == -4
    assert nat.sz_reference_split(0, a, 16384, b, c + 2, None) == -4


def test_host_argument_checks_reference_join():
    """sz_reference_join checks dtype, size, pointers and alignment on the
    host, before any launch."""
    nat = _native()
    a, b, c = 1 << 20, 1 << 30, 1 << 31
    assert nat.sz_reference_join(0, None, None, 0, None, None) == 0     # nothing to do
    assert nat.sz_reference_join(2, a, b, 16384, c, None) == -2
    assert nat.sz_reference_join(1, a, b, 16384 + 32, c, None) == -1     # not whole tiles
    assert nat.sz_reference_join(0, None, b, 16384, c, None) == -1
    assert nat.sz_reference_join(0, a, None, 16384, c, None) == -1
    assert nat.sz_reference_join(0, a, b, 16384, None, None) == -1
    assert nat.sz_reference_join(1, a + 8, b, 16384, c, None) == -4
    assert nat.sz_reference_join(1, a, b + 4, 16384, c, None) == -4
    assert nat.sz_reference_join(1, a, b, 16384, c + 2, None) == -4


def test_host_argument_checks_decode_noalloc():
    """sz_decode_noalloc rejects bad arguments, and requests beyond its fixed
    scratch, on the host before any launch."""
    nat = _native()
    dummy = 1 << 20
    cap = nat.sz_decode_noalloc_max_elems()
    assert cap == ((1 << 20) - 256 - 16) // 8 * 65536
    big = nat.sz_encoded_size(0, cap + 1, 0)
    assert nat.sz_decode_noalloc(dummy, big, 0, dummy, cap + 1, dummy, None) == -8
    assert nat.sz_decode_noalloc(dummy, big, 0, dummy, (1 << 40) + 1, dummy, None) == -1
    fixed = nat.sz_encoded_size(0, 1000, 0)
    assert nat.sz_decode_noalloc(dummy, fixed, 0, dummy, 1000, None, None) == -1
    assert nat.sz_decode_noalloc(dummy, fixed, 0, dummy, 1000, dummy + 2, None) == -4
    assert nat.sz_decode_noalloc(dummy, fixed - 1, 0, dummy, 1000, dummy, None) == -5
    assert nat.sz_decode_noalloc(dummy, fixed, 3, dummy, 1000, dummy, None) == -2
    assert nat.sz_decode_noalloc(dummy + 8, fixed, 0, dummy, 1000, dummy, None) == -4

