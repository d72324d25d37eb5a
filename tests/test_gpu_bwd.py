"""Backward on the HIP path vs the fp64 oracle's backward, through the C ABI.

The forward that produces out and lse is the library's own (the backward's
inputs); the oracle recomputes everything from q, k, v, the depth slots and the
upstream gradient, all regenerated on the host. Small and ragged shapes compare
every gradient element; the benchmarked workloads compare every gradient of one
(segment, KV head) unit, recomputed by the oracle on that unit alone (the unit's
gradients depend on nothing outside it).
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import bwd_rounding_magnitudes, check_grad, check_grad_bf16, unit_operands, workload
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


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run(w, grad_f32=False, grads=None):
    from joint_sequence_depth_amd import attn_bwd, attn_fwd

    x = configs.make_device(w, "cuda")
    gdt = torch.float32 if (grad_f32 or not w.bf16) else torch.bfloat16
    cu = torch.from_numpy(w.cu_seqlens()).cuda() if w.varlen else None
    ml = max(w.lengths) if w.varlen else None
    out, lse = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, causal=w.causal, scale=w.scale,
                        cu_seqlens=cu, max_seqlen=ml, out_dtype=gdt)
    dout = configs.make_dout_device(w, "cuda", gdt)
    g = attn_bwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], out, dout, lse, n_depth=w.n_depth, causal=w.causal,
                 scale=w.scale, cu_seqlens=cu, max_seqlen=ml, grads=grads)
    torch.cuda.synchronize()
    return g, gdt == torch.bfloat16


NAMES = ("dq", "dk", "dv", "dk_depth", "dv_depth")


def _compare(w, got, ref, grad_bf16, mags=None, tag=""):
    """fp32 inputs: the forward's 1e-5 absolute bound. bf16 inputs: 2e-2 RMS(ref)
    plus each element's first-order rounding magnitude (``mags``)."""
    S = w.n_depth
    worst = 0.0
    for i, (name, gt, rf) in enumerate(zip(NAMES, got, ref)):
        mg = None if mags is None else mags[i]
        if name in ("dk_depth", "dv_depth"):
            if S == 0 or gt is None:
                continue
            gt, rf = gt[..., :S, :, :], rf[..., :S, :, :]
            mg = None if mg is None else mg[..., :S, :, :]
        if w.bf16:
            _, ratio = check_grad_bf16(w, gt, rf, mg, f"{tag}{name}", grad_bf16)
        else:
            _, ratio = check_grad(w, gt, rf, f"{tag}{name}", grad_bf16)
        worst = max(worst, ratio)
    return worst


def _full_compare(w, grad_f32=False):
    _say(f"bwd case {w} grad_f32={grad_f32}")
    g, grad_bf16 = _run(w, grad_f32)
    h = configs.make_host(w)
    dout = configs.make_dout_host(w, grad_bf16)
    cu = w.cu_seqlens() if w.varlen else None
    ref = oracle.joint_attention_backward(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, dout, w.causal, w.scale,
                                          cu_seqlens=cu)
    mags = None
    if w.bf16:
        mags = bwd_rounding_magnitudes(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, dout, w.causal, w.scale,
                                       cu_seqlens=cu)
    got = [None if t is None else _np(t) for t in g]
    worst = _compare(w, got, ref, grad_bf16, mags)
    _say(f"  worst error/bound {worst:.3f}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 63, 65, 129, 300])
def test_bwd_ragged_lengths(dtype, d, T):
    _full_compare(workload(dtype=dtype, head_dim=d, seqlen=T, batch=2, n_heads_q=2, n_heads_kv=2, n_depth=3,
                           seed=T + d + 1000))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,S_cap", [(0, 0), (0, 3), (1, 1), (3, 5), (24, 24)])
def test_bwd_depth_counts(dtype, S, S_cap):
    _full_compare(workload(dtype=dtype, head_dim=128, seqlen=200, batch=1, n_heads_q=2, n_heads_kv=2, n_depth=S,
                           depth_capacity=S_cap, seed=1100 + S))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,S_cap,Hq,Hkv,d", [(65, 70, 8, 2, 128), (130, 131, 4, 4, 64)])
def test_bwd_many_depth_slots(dtype, S, S_cap, Hq, Hkv, d):
    # the prep kernel's ring of slot loads wraps many times and ends ragged
    _full_compare(workload(dtype=dtype, head_dim=d, seqlen=90, batch=1, n_heads_q=Hq, n_heads_kv=Hkv, n_depth=S,
                           depth_capacity=S_cap, seed=1150 + S))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 1), (8, 2), (6, 2), (16, 1), (12, 4)])
def test_bwd_grouped_heads(dtype, Hq, Hkv):
    _full_compare(workload(dtype=dtype, head_dim=64, seqlen=150, batch=1, n_heads_q=Hq, n_heads_kv=Hkv, n_depth=4,
                           seed=1200 + Hq * 10 + Hkv))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_not_causal(dtype):
    _full_compare(workload(dtype=dtype, head_dim=128, seqlen=170, batch=2, n_heads_q=4, n_heads_kv=2, n_depth=5,
                           causal=False, seed=1300))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lens,causal", [((5, 130, 64, 1, 200), True), ((5, 1, 130, 64, 0, 257), True),
                                         ((70, 0, 33), False)])
def test_bwd_varlen(dtype, lens, causal):
    # includes empty sequences (equal offsets) and a non-causal packed case
    _full_compare(workload(dtype=dtype, head_dim=64, seqlens=lens, n_heads_q=4, n_heads_kv=1, n_depth=3,
                           causal=causal, seed=1400 + len(lens)))


def test_bwd_fp32_gradients_of_bf16_inputs():
    _full_compare(workload(dtype="bf16", head_dim=128, seqlen=257, batch=2, n_heads_q=8, n_heads_kv=2, n_depth=6,
                           seed=1500), grad_f32=True)


def test_bwd_large_key_scale():
    # keys scaled by 4: peaked softmax rows, where the probabilities are far from uniform
    _full_compare(workload(dtype="bf16", head_dim=64, seqlen=190, batch=1, n_heads_q=2, n_heads_kv=1, n_depth=4,
                           key_mult=4.0, seed=1600))


def test_bwd_unread_slots_untouched():
    w = workload(dtype="bf16", head_dim=64, seqlen=70, batch=1, n_heads_q=2, n_heads_kv=1, n_depth=2,
                 depth_capacity=5, seed=1700)
    x = configs.make_device(w, "cuda")
    nan = float("nan")
    grads = (torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"]),
             torch.full_like(x["kd"], nan), torch.full_like(x["vd"], nan))
    g, _ = _run(w, grads=grads)
    for t in g[3:]:
        assert torch.isnan(t[:, :, 2:]).all() and torch.isfinite(t[:, :, :2]).all()


# ------------------------------------------------------------------ benchmarked workloads, one unit each
@pytest.mark.parametrize("name", ["small_bf16", "mha_bf16", "gqa_bf16", "packed_bf16", "tiny_f32"])
def test_bwd_workload_unit(name):
    w = configs.WORKLOADS[name]
    _say(f"bwd workload {name}")
    g, grad_bf16 = _run(w)
    rng = np.random.default_rng(7)
    s = int(rng.integers(0, len(w.lengths)))
    hk = int(rng.integers(0, w.n_heads_kv))
    q, k, v, kd, vd, do = unit_operands(w, s, hk, grad_bf16)
    ref = oracle.joint_attention_backward(q, k, v, kd, vd, w.n_depth, do, w.causal, w.scale)
    mags = bwd_rounding_magnitudes(q, k, v, kd, vd, w.n_depth, do, w.causal, w.scale) if w.bf16 else None
    G, L = w.group, w.lengths[s]
    if w.varlen:
        t0 = int(w.cu_seqlens()[s])
        sl = (slice(t0, t0 + L),)
    else:
        sl = (s, slice(0, L))
    hq = slice(hk * G, (hk + 1) * G)
    got = [_np(g[0][sl + (hq,)]), _np(g[1][sl + (slice(hk, hk + 1),)]), _np(g[2][sl + (slice(hk, hk + 1),)])]
    if w.s_cap > 0:
        got += [_np(g[3][sl + (slice(None), slice(hk, hk + 1))]), _np(g[4][sl + (slice(None), slice(hk, hk + 1))])]
    else:
        got += [None, None]
    ref = [r[0] if r is not None else None for r in ref]  # drop the unit's batch axis
    if mags is not None:
        mags = [m[0] if m is not None else None for m in mags]
    worst = _compare(w, got, ref, grad_bf16, mags, tag=f"{name} seg {s} kv head {hk} ")
    _say(f"  unit (segment {s}, KV head {hk}): worst error/bound {worst:.3f}")
