"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The units whose host code does the argument checks, the size arithmetic and the
dispatch (moda_attn.hip, moda_decode_noalloc.hip) are rebuilt with both
sanitizers on the host side only (device code is compiled as usual), linked with
the library's other objects, and driven through the whole ABI validation suite
(tests/test_abi.py) in a child process with the sanitizer runtime preloaded: an
out-of-bounds access, a signed overflow or any other undefined behaviour on
those paths ends the run with a report. CPU only; no call reaches a launch.
"""
import glob
import os
import subprocess
import sys

import pytest

from joint_sequence_depth_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_UNITS = ("moda_attn.hip", "moda_decode_noalloc.hip")
# host-side only: each sanitizer flag goes to the host compilation
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def host_clang():
    path = "/opt/rocm/lib/llvm/bin/clang++"
    return path if os.path.exists(path) else None


@pytest.fixture(autouse=True)
def _no_gpu_here():
    try:
        import torch

        if torch.cuda.is_available():
            pytest.skip("host-only validation tests run where no GPU can be reached")
    except ImportError:
        pass


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm installation")
    objdir = os.path.join(B.PKG, "_build")
    others = [os.path.join(objdir, stem + ".o") for src, stem, _ in B.UNITS if src not in HOST_UNITS]
    if not all(os.path.exists(o) for o in others):
        B.build()
    out = tmp_path_factory.mktemp("hostsan")
    objs = []
    for src in HOST_UNITS:
        obj = str(out / (src[:-4] + ".o"))
        r = subprocess.run([B.hipcc(), *B.compile_flags(src), *SAN, "-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    lib = str(out / "libmoda_attn_hostsan.so")
    r = subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address,undefined", "-shared-libsan", *objs, *others, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib, rt


def run_sanitized(args, rt, timeout=600):
    env = dict(os.environ, LD_PRELOAD=rt, **ENV)
    return subprocess.run(args, env=env, cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def test_sanitizers_report_a_planted_overflow(tmp_path):
    # the flags and the runtime work: a host program with a signed overflow
    # (planted here, in a throwaway C++ file) is stopped with a report
    cc, rt = host_clang(), asan_runtime()
    if cc is None or rt is None:
        pytest.skip("no clang++ / sanitizer runtime in this ROCm installation")
    src = tmp_path / "planted.cpp"
    src.write_text("#include <climits>\nint main(int argc, char**) { volatile long big = LONG_MAX; "
                   "long x = big + argc; return x > 0 ? 0 : 1; }\n")
    exe = tmp_path / "planted"
    subprocess.run([cc, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], env=dict(os.environ, **ENV), capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and "runtime error" in r.stderr


def test_abi_checks_under_host_sanitizers(sanitized_lib):
    lib, rt = sanitized_lib
    code = (
        "import sys, pytest\n"
        "import joint_sequence_depth_amd._lib as L\n"
        f"L.LIB_PATH = {lib!r}\n"
        f"rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi.py')!r}])\n"
        "print('SANITIZED LIBRARY LOADED:', L.LIB_PATH in open('/proc/self/maps').read())\n"
        "sys.exit(int(rc))\n"
    )
    r = run_sanitized([sys.executable, "-c", code], rt)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-6000:]
    assert "SANITIZED LIBRARY LOADED: True" in log, log[-3000:]
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-6000:]
    assert " passed" in log and " failed" not in log, log[-3000:]
