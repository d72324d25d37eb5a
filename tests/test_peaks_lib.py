"""The attained-peak microbenchmark library (libmoda_peaks.so) on the host: it
loads, exports what include/moda_peaks.h declares, and rejects bad arguments
before any launch (no GPU needed: no call here reaches a launch)."""
import ctypes
import os
import re

from joint_sequence_depth_amd import build

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moda_peaks.h")


def _lib():
    L = ctypes.CDLL(build.PEAKS_PATH)
    L.moda_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p]
    L.moda_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    L.moda_peak_mfma_flops_per_launch.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.moda_peak_mfma_flops_per_launch.restype = ctypes.c_double
    return L


def test_exports_every_declared_symbol():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = set(re.findall(r"\b(moda_[a-z_0-9]+)\s*\(", text))
    L = _lib()
    assert names == {"moda_peak_stream_read", "moda_peak_mfma_bf16", "moda_peak_mfma_flops_per_launch"}
    for n in names:
        assert hasattr(L, n)


def test_invalid_arguments_launch_nothing():
    L = _lib()
    P = 0x10000
    assert L.moda_peak_stream_read(None, 1 << 20, P, 64, None) == 1
    assert L.moda_peak_stream_read(P, 1000, P, 64, None) == 1  # not a multiple of 16
    assert L.moda_peak_stream_read(P + 8, 1 << 20, P, 64, None) == 1  # misaligned
    assert L.moda_peak_stream_read(P, 1 << 20, P, 0, None) == 1
    assert L.moda_peak_mfma_bf16(0, P, 64, None) == 1
    assert L.moda_peak_mfma_bf16(16, None, 64, None) == 1


def test_flop_count():
    L = _lib()
    # 4 waves x 4 products of 32 x 32 x 16 multiply-adds per iteration
    assert L.moda_peak_mfma_flops_per_launch(10, 3) == 3 * 4 * 10 * 4 * 2 * 32 * 32 * 16
