"""CPU checks of bench.py's host logic: profiler kernel names map to the launch
names the library's instrumentation records (the key that joins rocprofv3
counters and durations to HIP-event timings)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

NS = "void sz::(anonymous namespace)::"


@pytest.mark.parametrize("demangled, launch", [
    (NS + "sz_enc_dense_bf16<1, 8>(unsigned short const*, unsigned long)", "sz_enc_dense_bf16"),
    (NS + "sz_enc_dense_bf16<1, 2>(unsigned short const*, unsigned long)", "sz_enc_dense_bf16"),
    (NS + "sz_enc_dense_bf16<2, 8>(unsigned short const*, unsigned long)", "sz_enc_dense_top8"),
    (NS + "sz_enc_dense_bf16<3, 8>(unsigned short const*, unsigned long)", "sz_enc_dense_top15s"),
    (NS + "sz_enc_compact<1>(unsigned char*, unsigned long)", "sz_enc_compact"),
    (NS + "sz_cal_hist<0>(unsigned short const*)", "sz_cal_hist_bf16"),
    (NS + "sz_cal_hist<1>(unsigned char const*)", "sz_cal_hist_e5m2"),
    (NS + "sz_dec_bf16_span<256, 4>(unsigned char const*, sz::DecodeArgs)", "sz_dec_bf16_span"),
    (NS + "sz_dec_top8_span<256, 2>(unsigned char const*, sz::DecodeArgs)", "sz_dec_top8_span"),
    (NS + "sz_dec_top15s(unsigned char const*, sz::DecodeArgs)", "sz_dec_top15s"),
    ("sz_ref_copy(uint4 const*, uint4*, unsigned long)", "sz_ref_copy"),
])
def test_short_kernel_name(demangled, launch):
    assert bench.short_kernel_name(demangled) == launch


def test_every_mapped_name_is_a_launch_name():
    """Each name the map produces is one the library's instrumentation records."""
    src = ""
    csrc = os.path.join(ROOT, "fp8_kv_cache_sz_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        src += open(os.path.join(csrc, f)).read()
    for name in set(bench.LAUNCH_NAMES.values()):
        assert 'LaunchScope scope("%s"' % name in src, name
