"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host only): a child process loads an instrumented build of
``oracle/splitzip_oracle.c`` and runs encode/decode round trips of both
dtypes and both ablation formats, then validate/decode/check_canonical on
corrupted and truncated copies of those streams.  Any out-of-bounds access or
undefined behaviour aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import numpy as np
import oracle
rng = np.random.default_rng(7)
cases = 0
for dtype in (0, 1):
    for n in (0, 1, 7, 33, 4097, 65536, 65537, 3 * 65536 + 11):
        if dtype == 0:
            e = np.clip(np.rint(rng.normal(126, 6, n)), 0, 255).astype(np.uint16)
            bits = ((rng.integers(0, 2, n) << 15) | (e << 7) | rng.integers(0, 128, n)).astype(np.uint16)
        else:
            e = np.clip(np.rint(rng.normal(14, 4, n)), 0, 31).astype(np.uint8)
            bits = ((rng.integers(0, 2, n) << 7) | (e << 2) | rng.integers(0, 4, n)).astype(np.uint8)
        cb = oracle.calibrate(bits, dtype)
        good = [(oracle.encode(bits, dtype, cb), None)]
        if dtype == 0 and n:
            good += [(oracle.encode_variant(bits, 2, cb[:8]), 2), (oracle.encode_variant(bits, 3, cb[:15]), 3)]
        for s, v in good:
            back = oracle.decode(s, dtype, n) if v is None else oracle.decode_variant(s, v, n)
            assert np.array_equal(back, bits), (dtype, n, v)
            for trial in range(60):
                t = s.copy()
                kind = trial % 4
                if kind == 0:                                   # bytes anywhere
                    idx = rng.integers(0, t.size, int(rng.integers(1, 6)))
                    t[idx] = rng.integers(0, 256, idx.size)
                elif kind == 1:                                 # header and block counts
                    idx = rng.integers(0, min(t.size, 72 + 4 * ((n + 65535) // 65536)), 3)
                    t[idx] = rng.integers(0, 256, idx.size)
                elif kind == 2:                                 # truncated
                    t = t[: int(rng.integers(0, t.size))]
                else:                                           # the last records
                    idx = t.size - 1 - rng.integers(0, min(t.size, 48), 3)
                    t[idx] = rng.integers(0, 256, 3)
                if v is None:
                    ok = oracle.validate(t, dtype, n) == 0
                    assert ok == (oracle.decode_rc(t, dtype, n)[0] == 0)
                    oracle.check_canonical(t, dtype, n)
                else:
                    ok = oracle.validate_variant(t, v, n) == 0
                    assert ok == (oracle.decode_variant_rc(t, v, n)[0] == 0)
                cases += 1
print("sanitized oracle cases", cases)
"""


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc has no ASan/UBSan runtime here")
    so = str(tmp_path / "liboracle_sanitized.so")
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared", "-fPIC",
                           "-o", so, os.path.join(ROOT, "oracle", "splitzip_oracle.c")])
    env = dict(os.environ, SPLITZIP_ORACLE_LIB=so, LD_PRELOAD=asan + " " + ubsan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONPATH=ROOT)
    p = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-4000:]
    assert "sanitized oracle cases" in p.stdout
