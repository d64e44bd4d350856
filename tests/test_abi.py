"""CPU-side checks of the C ABI: the library loads, exports every function the public header
declares, sizes its workspace, and rejects bad arguments on the host before touching a GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_cycle.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from draft_sampling_lossless_spec_amd import binding
    if not os.path.exists(binding.lib_path()):
        from draft_sampling_lossless_spec_amd import build
        build.build()
    return binding._load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"spec_cycle", "spec_workspace_bytes", "spec_error_string", "spec_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_sizing(lib):
    from draft_sampling_lossless_spec_amd import spec_workspace_bytes, BF16, FP32, FLAT, CHUNKED
    n = spec_workspace_bytes(256, 16, 151936, 256, BF16, CHUNKED)
    assert n > 0 and n % 256 == 0
    assert spec_workspace_bytes(512, 16, 151936, 256, BF16, CHUNKED) > n
    assert spec_workspace_bytes(2, 4, 1024, 32, FP32, FLAT) > 0
    for bad in [(0, 4, 100, 16), (2, 0, 100, 16), (2, 33, 100, 16), (2, 4, 1, 16), (2, 4, 100, 0),
                (2, 4, 100, 300), (1025, 4, 100, 16)]:
        assert spec_workspace_bytes(*bad, BF16, CHUNKED) == 0, bad
    assert spec_workspace_bytes(2, 4, 100, 24, BF16, CHUNKED) == 0      # bf16 needs R % 16 == 0
    assert spec_workspace_bytes(2, 4, 100, 24, FP32, CHUNKED) > 0
    assert spec_workspace_bytes(2, 4, 100, 16, 7, CHUNKED) == 0
    assert spec_workspace_bytes(2, 4, 100, 16, BF16, 5) == 0


def test_host_checks_reject_before_any_gpu_call(lib):
    from draft_sampling_lossless_spec_amd.binding import _Dims
    d = _Dims(2, 4, 100, 16, 1, 1)
    args = [None] * 7 + [C.c_float(0.5), C.c_uint64(1), C.c_int64(0), None, None, None, None, C.c_size_t(0), None]
    assert lib.spec_cycle(C.byref(d), *args) == -1                      # NULL inputs
    bad = _Dims(2, 4, 100, 24, 1, 1)
    assert lib.spec_cycle(C.byref(bad), *args) == -2                    # bf16 with R % 16 != 0
    assert lib.spec_cycle(None, *args) == -1
    fake = C.c_void_p(4096)                                             # never dereferenced
    full = [fake, fake, fake, fake, None, fake, fake, C.c_float(0.5), C.c_uint64(1), C.c_int64(0), fake, fake,
            None, None, C.c_size_t(0), None]
    assert lib.spec_cycle(C.byref(d), *full) == -3                      # no workspace
    mis = [fake, fake, C.c_void_p(4100), fake] + full[4:]
    assert lib.spec_cycle(C.byref(d), *mis) == -1                       # misaligned A


def test_error_strings(lib):
    from draft_sampling_lossless_spec_amd import spec_error_string, spec_version
    for code in (0, -1, -2, -3, -4, -5, 42):
        assert isinstance(spec_error_string(code), str) and spec_error_string(code)
    assert spec_version() >= 100


def test_stats_host_checks_reject_before_any_gpu_call(lib):
    from draft_sampling_lossless_spec_amd.binding import _Dims
    from draft_sampling_lossless_spec_amd import spec_stats_workspace_bytes, BF16, FP32
    assert spec_stats_workspace_bytes(256, 16, 151936, 256, BF16) % 256 == 0
    assert spec_stats_workspace_bytes(256, 16, 151936, 256, BF16) > spec_stats_workspace_bytes(64, 5, 151936, 256,
                                                                                                BF16)
    assert spec_stats_workspace_bytes(2, 4, 100, 24, BF16) == 0 and spec_stats_workspace_bytes(2, 4, 100, 24, FP32) > 0
    d = _Dims(2, 4, 100, 16, 1, 1)
    fake = C.c_void_p(4096)                                             # never dereferenced
    nulls = [None] * 10 + [None, C.c_size_t(0), None]
    assert lib.spec_accept_stats(C.byref(d), *nulls) == -1              # NULL inputs
    assert lib.spec_accept_stats(None, *nulls) == -1
    full = [fake] * 4 + [None, fake, fake, fake, None, None, None, C.c_size_t(0), None]
    assert lib.spec_accept_stats(C.byref(d), *full) == -3               # no workspace
    bad = _Dims(2, 4, 100, 24, 1, 1)
    assert lib.spec_accept_stats(C.byref(bad), *full) == -2             # bf16 with R % 16 != 0
    mis = [fake, fake, C.c_void_p(4100)] + full[3:]
    assert lib.spec_accept_stats(C.byref(d), *mis) == -1                # misaligned A
    e = [fake, fake, fake]
    assert lib.spec_calibration_error(*e, 0, 4, 10, fake, fake, None) == -1          # B < 1
    assert lib.spec_calibration_error(*e, 2, 4, 0, fake, fake, None) == -1           # no bin
    assert lib.spec_calibration_error(*e, 2, 4, 5000, fake, fake, None) == -1        # too many bins
    assert lib.spec_calibration_error(None, fake, fake, 2, 4, 10, fake, fake, None) == -1


def test_schedule_host_checks_reject_before_any_gpu_call(lib):
    fake = C.c_void_p(4096)                                             # never dereferenced
    assert lib.spec_schedule(None, 2, 4, fake, 64, fake, fake, None) == -1
    assert lib.spec_schedule(fake, 0, 4, fake, 64, fake, fake, None) == -1          # B < 1
    assert lib.spec_schedule(fake, 2, 33, fake, 64, fake, fake, None) == -1         # K > 32
    assert lib.spec_schedule(fake, 2, 4, fake, 0, fake, fake, None) == -1           # no bin
    assert lib.spec_schedule(fake, 2, 4, fake, 4097, fake, fake, None) == -1        # too many bins
    assert lib.spec_schedule(fake, 2, 4, None, 64, fake, fake, None) == -1


def test_cycle_lengths_host_checks(lib):
    from draft_sampling_lossless_spec_amd.binding import _Dims
    d = _Dims(2, 4, 100, 16, 1, 1)
    fake = C.c_void_p(4096)                                             # never dereferenced
    args = [fake] * 5 + [None, fake, C.c_uint64(1), C.c_int64(0), fake, fake, None, None, C.c_size_t(0), None]
    assert lib.spec_cycle_lengths(C.byref(d), *args) == -1              # no verify_len
    args[5] = fake
    assert lib.spec_cycle_lengths(C.byref(d), *args) == -3              # no workspace


def test_temperature_scaling_host_checks(lib):
    fake = C.c_void_p(4096)                                             # never dereferenced
    assert lib.spec_temperature_scaling_workspace_bytes(1000, 61) > 0
    assert lib.spec_temperature_scaling_workspace_bytes(0, 61) == 0
    assert lib.spec_temperature_scaling_workspace_bytes(1000, 2000) == 0
    good = [fake, fake, fake, 1000, 4, fake, 61, 10, fake, None, None]
    assert lib.spec_temperature_scaling(*good, None, C.c_size_t(0), None) == -3      # no workspace
    assert lib.spec_temperature_scaling(None, *good[1:], fake, C.c_size_t(1 << 20), None) == -1
    bad = list(good)
    bad[7] = 65                                                         # too many bins
    assert lib.spec_temperature_scaling(*bad, fake, C.c_size_t(1 << 20), None) == -1
    bad = list(good)
    bad[4] = 300                                                        # K > 256
    assert lib.spec_temperature_scaling(*bad, fake, C.c_size_t(1 << 20), None) == -1


def test_advance_host_checks(lib):
    fake = C.c_void_p(4096)                                             # never dereferenced
    assert lib.spec_advance(None, fake, 2, 4, fake, None, None) == -1
    assert lib.spec_advance(fake, fake, 0, 4, fake, None, None) == -1
    assert lib.spec_advance(fake, fake, 2, 33, fake, None, None) == -1
    assert lib.spec_advance(fake, fake, 2, 4, None, None, None) == -1


def test_noalloc_host_checks(lib):
    """spec_cycle_noalloc: dims that need more than the static scratch array are rejected with
    SPEC_E_SCRATCH on the host, before the device is touched."""
    from draft_sampling_lossless_spec_amd import SPEC_SCRATCH_BYTES, spec_workspace_bytes
    from draft_sampling_lossless_spec_amd.binding import _Dims
    assert SPEC_SCRATCH_BYTES == 64 << 20
    hdr = open(HEADER).read()
    assert "#define SPEC_SCRATCH_BYTES ((size_t)64 << 20)" in hdr
    fake = C.c_void_p(4096)                                             # never dereferenced
    args = [fake] * 4 + [None, fake, fake, C.c_float(0.5), C.c_uint64(1), C.c_int64(0), fake, fake, None, None]
    over = [dims for dims in [(1024, 32, 151936, 256), (1024, 32, 1 << 22, 256)]
            if spec_workspace_bytes(*dims, 1, 1) > SPEC_SCRATCH_BYTES]
    assert over, "no test shape exceeds the static scratch array"
    big = _Dims(*over[0], 1, 1)
    assert lib.spec_cycle_noalloc(C.byref(big), *args) == -6
    assert lib.spec_cycle_noalloc(None, *args) == -1
    bad = _Dims(2, 4, 100, 24, 1, 1)
    assert lib.spec_cycle_noalloc(C.byref(bad), *args) == -2            # bf16 with R % 16 != 0
    from draft_sampling_lossless_spec_amd import spec_error_string
    assert "scratch" in spec_error_string(-6)
