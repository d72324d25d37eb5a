"""Builds libmoda_attn.so (the C ABI + HIP kernels) in-tree for gfx950 with hipcc.

    python -m joint_sequence_depth_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoda_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
PEAKS_PATH = os.path.join(PKG, "libmoda_peaks.so")  # measurement only (include/moda_peaks.h)
# Debug build: the same sources with -DMODA_POISON_LDS=1 (csrc/moda_debug.h), every
# kernel's LDS filled with NaNs at its start; loaded only by its GPU test.
POISON_LIB_PATH = os.path.join(PKG, "libmoda_attn_poison.so")
SOURCES = ["moda_attn.hip", "moda_fwd_bf16.hip", "moda_fwd_f32.hip", "moda_depth_select.hip", "moda_decode.hip",
           "moda_decode_noalloc.hip", "moda_bwd.hip", "moda_depth_kv.hip", "moda_depth_kv_project.hip"]
# Compilation units: (source, object stem, extra flags). The bf16 forward's
# template instances are split by head dim and query heads per workgroup, one
# unit each, so that they compile side by side.
UNITS = [(src, src[:-4], []) for src in SOURCES if src != "moda_fwd_bf16.hip"] + [
    ("moda_fwd_bf16.hip", f"moda_fwd_bf16_d{d}_g{g}", [f"-DMODA_FWD_D={d}", f"-DMODA_FWD_GB={g}"])
    for d in (64, 128) for g in (1, 2, 4)
]
# Sources whose kernels keep matrix-core accumulators in AGPRs (the backward
# holds two 128 x 32 fp32 accumulators per wave, more than the VGPRs alone)
AGPR_ACCUMULATORS = {"moda_bwd.hip"}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags(source: str = ""):
    flags = [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # packed fp32 VALU ops stay off: plain float code only
        "-Xclang",
        "-target-feature",
        "-Xclang",
        "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-function",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]
    if source not in AGPR_ACCUMULATORS:
        # MFMA accumulators in VGPRs: where LDS caps a kernel at one wave per SIMD
        # the compiler would otherwise place MFMA results in AGPRs and copy every
        # score back to VGPRs for the softmax
        flags += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return flags


def build(verbose: bool = False, poison: bool = True) -> str:
    """Compile every source and link the shared library (and, with `poison`, the
    poisoned-LDS debug build beside it); returns the library's path."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, stem + ".o") for _, stem, _ in UNITS]
    cmds = [[cc, *compile_flags(src), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            for (src, _, extra), obj in zip(UNITS, objs)]
    # one hipcc per unit, side by side (each is a separate process); the
    # attained-peak microbenchmarks go into a library of their own
    peaks_obj = os.path.join(objdir, "moda_peaks.o")
    cmds.append([cc, *compile_flags("moda_peaks.hip"), "-c", os.path.join(CSRC, "moda_peaks.hip"), "-o", peaks_obj])
    links = [(LIB_PATH, objs), (PEAKS_PATH, [peaks_obj])]
    if poison:
        pdir = os.path.join(PKG, "_build_poison")
        os.makedirs(pdir, exist_ok=True)
        pobjs = [os.path.join(pdir, stem + ".o") for _, stem, _ in UNITS]
        cmds += [[cc, *compile_flags(src), *extra, "-DMODA_POISON_LDS=1", "-c", os.path.join(CSRC, src), "-o", obj]
                 for (src, _, extra), obj in zip(UNITS, pobjs)]
        links.append((POISON_LIB_PATH, pobjs))
    # the slowest units (the bf16 forward's) first
    cmds.sort(key=lambda c: "moda_fwd_bf16" not in c[-1])
    workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in cmds]:
            f.result()
    for path, ob in links:
        tmp = path + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ob, "-o", tmp], verbose)
        os.replace(tmp, path)
    return LIB_PATH


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        line for line in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in line
    )
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
