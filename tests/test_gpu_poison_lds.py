"""No kernel reads LDS bytes that its own workgroup did not write first.

The library's poisoned-LDS debug build (the same sources compiled with
-DMODA_POISON_LDS=1: every kernel fills its LDS with NaNs before anything else)
must give results bit-identical to the normal build, and finite, on cases that
reach each kernel that uses LDS: the bf16 forward in its tile schedules (shared
tiles of 2 and 4 waves, split tiles, one, two and four heads per workgroup, both
head dims, ragged segments), its parts and its bounded depth reads, the fp32
slot selection, both decode kernels, the backward's three kernels and the two
projection kernels. Every kernel is deterministic (no atomics), so any
difference comes from a read of LDS that nothing wrote in that workgroup.
"""
import os
import sys

import pytest

from parity_util import SCHEDULE_CASES, run_hip, schedule_workload, with_, workload
from workloads import configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(fn):
    """fn() with the normal library, then with the poisoned-LDS build."""
    from joint_sequence_depth_amd import _lib, build

    assert os.path.exists(build.POISON_LIB_PATH), "the poisoned-LDS build is missing: run the package build"
    a = fn()
    torch.cuda.synchronize()
    with _lib.library(build.POISON_LIB_PATH):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        if x is None:
            assert y is None
            continue
        assert bool(torch.isfinite(y.float()).all()), f"{what}: output {i} of the poisoned build is not finite"
        assert torch.equal(x, y), f"{what}: output {i} differs, max |diff| {float((x.float() - y.float()).abs().max())}"


FWD_CASES = ["split_d64_g2", "split_d128", "shared2_d64", "shared2_d128_g4", "whole_shared4_d64_g4",
             "whole_shared4_d128_g1", "whole_shared4_d128_g4_pairs", "shared4_d128_g2"]


@pytest.mark.parametrize("case", FWD_CASES)
def test_forward_schedules(case):
    w = schedule_workload(case)
    _say(f"poison forward {case} {SCHEDULE_CASES[case]['kernel']}")
    x = configs.make_device(w, "cuda")
    for kw in (dict(), dict(out_f32=True), dict(phase=1), dict(phase=2), dict(depth_topk=2, depth_recent=1)):
        a, b = _both(lambda: run_hip(w, inputs=x, **kw)[1:])
        _same(a, b, f"{case} {kw}")


def test_forward_ragged_segments():
    for d, hq, hkv in ((64, 8, 2), (128, 8, 8), (128, 16, 4)):
        w = workload(head_dim=d, seqlens=(1, 37, 128, 300, 65, 1000), n_heads_q=hq, n_heads_kv=hkv, n_depth=6,
                     seed=7)
        _say(f"poison forward ragged d={d} Hq={hq} Hkv={hkv}")
        x = configs.make_device(w, "cuda")
        a, b = _both(lambda: run_hip(w, inputs=x)[1:])
        _same(a, b, f"ragged d={d} Hq={hq} Hkv={hkv}")


def test_fp32_slot_selection():
    w = workload(dtype="f32", head_dim=64, seqlen=96, n_heads_q=4, n_heads_kv=2, n_depth=9, seed=8)
    _say("poison fp32 top-S selection")
    x = configs.make_device(w, "cuda")
    a, b = _both(lambda: run_hip(w, inputs=x, depth_topk=3, depth_recent=2)[1:])
    _same(a, b, "fp32 selection")


@pytest.mark.parametrize("d,hq,hkv", [(64, 4, 4), (128, 32, 8), (128, 16, 2)])
def test_decode(d, hq, hkv):
    from joint_sequence_depth_amd import attn_decode

    w = configs.DecodeWorkload("case", "", "bf16", (5, 700, 64, 1500), 1500, hq, hkv, d, 5, 11)
    _say(f"poison decode d={d} Hq={hq} Hkv={hkv}")
    x = configs.make_decode_device(w, "cuda")
    a, b = _both(lambda: attn_decode(x["q"], x["k"], x["v"], x["seqlens"], x["kd"], x["vd"], n_depth=w.n_depth,
                                     scale=w.scale))
    _same(a, b, f"decode d={d} Hq={hq} Hkv={hkv}")


@pytest.mark.parametrize("d,hq,hkv", [(64, 4, 4), (128, 8, 2), (128, 12, 2)])
def test_backward(d, hq, hkv):
    from joint_sequence_depth_amd import attn_bwd, attn_fwd

    w = workload(head_dim=d, seqlens=(200, 57, 300), n_heads_q=hq, n_heads_kv=hkv, n_depth=5, seed=12)
    _say(f"poison backward d={d} Hq={hq} Hkv={hkv}")
    x = configs.make_device(w, "cuda")
    cu = torch.from_numpy(w.cu_seqlens()).cuda()
    ml = max(w.lengths)
    out, lse = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, causal=w.causal,
                        scale=w.scale, cu_seqlens=cu, max_seqlen=ml)
    dout = configs.make_dout_device(w, "cuda", torch.bfloat16)
    a, b = _both(lambda: attn_bwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], out, dout, lse, n_depth=w.n_depth,
                                  causal=w.causal, scale=w.scale, cu_seqlens=cu, max_seqlen=ml))
    _same(a, b, f"backward d={d} Hq={hq} Hkv={hkv}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_projection(dtype):
    from joint_sequence_depth_amd import depth_kv_project

    _say(f"poison projection {dtype}")
    g = torch.Generator(device="cuda").manual_seed(5)
    n, dm, hkv, d, s_cap = 300, 256, 2, 64, 3
    xin = torch.randn(n, dm, device="cuda", generator=g).to(dtype)
    wkv = (torch.randn(2 * hkv * d, dm, device="cuda", generator=g) / 16).to(dtype)

    def run():
        kd = torch.zeros(n, s_cap, hkv, d, device="cuda", dtype=dtype)
        vd = torch.zeros_like(kd)
        depth_kv_project(xin, wkv, kd, vd, slot=1)
        return kd, vd

    a, b = _both(run)
    _same(a, b, f"projection {dtype}")
