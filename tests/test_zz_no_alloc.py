"""moda_attn_decode_noalloc (the decode step through the library's own per-GPU
scratch array, for callers that cannot allocate) against moda_attn_decode with a
caller workspace, through the C ABI on an MI355X: two calls in a row, the second
smaller, each bit-identical to the workspace call (same kernels, same chunking)
and within the parity bound of the fp64 oracle. (The rejection of steps whose
scratch need exceeds the array is checked on the host, in test_abi.py.)"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import check_lse, check_out, to_np
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


CASES = [  # the second call is smaller than the first
    configs.DecodeWorkload("noalloc_big", "", "bf16", (700, 1, 333, 512, 64, 699), 700, 8, 2, 128, 5, seed=71),
    configs.DecodeWorkload("noalloc_small", "", "bf16", (100, 37), 100, 4, 4, 64, 3, seed=72),
]


def _one(w, out_f32):
    from joint_sequence_depth_amd import attn_decode, attn_decode_noalloc, decode_workspace_size

    _say(f"no-alloc decode {w.name}: B={w.batch} Hq={w.n_heads_q} Hkv={w.n_heads_kv} d={w.head_dim} "
         f"S={w.n_depth} out_f32={out_f32} scratch need "
         f"{decode_workspace_size(w.batch, w.n_heads_q, w.n_heads_kv, w.head_dim, w.max_cache_len)} B")
    x = configs.make_decode_device(w, "cuda")
    odt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.empty(w.shape_q(), dtype=odt, device="cuda")
    lse = torch.empty((w.batch, w.n_heads_q), dtype=torch.float32, device="cuda")
    attn_decode_noalloc(x["q"], x["k"], x["v"], x["seqlens"], out, x["kd"], x["vd"], n_depth=w.n_depth,
                        scale=w.scale, lse=lse)
    ref_out, ref_lse = attn_decode(x["q"], x["k"], x["v"], x["seqlens"], x["kd"], x["vd"], n_depth=w.n_depth,
                                   scale=w.scale, out_dtype=odt)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    h = configs.make_decode_host(w)
    ro, rl = oracle.decode(h["q"], h["k"], h["v"], h["seqlens"], h["kd"], h["vd"], w.n_depth, w.scale)
    err, ratio = check_out(w, to_np(out), ro, f"{w.name} no-alloc decode out_f32={out_f32}",
                           out_bf16=not out_f32)
    check_lse(w, to_np(lse), rl, w.name)
    _say(f"  max err {err:.3e}, error/bound {ratio:.3f}")


@pytest.mark.parametrize("out_f32", [False, True])
def test_noalloc_matches_workspace_call_twice(out_f32):
    for w in CASES:
        _one(w, out_f32)
