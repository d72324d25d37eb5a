"""HIP path vs the fp64 oracle, through the C ABI, on an MI355X.

Small and ragged shapes are compared element by element over the whole output;
the five full-size workloads are launched exactly as the benchmark launches them
and checked on sampled rows (t = 0, tile boundaries, each sequence's last token,
random rows), each recomputed by the oracle from operands regenerated on the host.
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import (SCHEDULE_CASES, check_lse, check_out, gpu_row, oracle_full, oracle_row, run_hip,
                         sample_rows, schedule_workload, stored_rms, to_np, with_, workload)
from workloads import configs, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _full_compare(w, both_outputs=True):
    """Whole-output comparison; bf16 inputs are run with a bf16 and an fp32 output."""
    _say(f"case {w}")
    ref_o, ref_l = oracle_full(w)
    res = None
    for out_f32 in ([False, True] if (w.bf16 and both_outputs) else [False]):
        _, out, lse = run_hip(w, out_f32=out_f32)
        r = check_out(w, to_np(out), ref_o, f"{w.name} whole out_f32={out_f32}", out_bf16=w.bf16 and not out_f32)
        check_lse(w, to_np(lse), ref_l, w.name)
        _say(f"  out_f32={out_f32}: max err {r[0]:.3e}, error/bound {r[1]:.3f}")
        res = res or r
    return res


# ------------------------------------------------------------------ generator parity on the device
def test_device_generator_matches_host():
    w = configs.WORKLOADS["small_bf16"]
    x = configs.make_device(w, "cuda")
    rng = np.random.default_rng(1)
    for name in ("q", "k", "kd", "vd"):
        t = x[name]
        idx = rng.integers(0, t.numel(), size=4096)
        dev = t.view(-1)[torch.from_numpy(idx).cuda()].float().cpu().numpy()
        mult = w.key_mult if name in ("k", "kd") else 1.0
        host = gen.values_np(w.seed, configs.tids()[name], idx, mult, True)
        assert np.array_equal(dev.view(np.uint32), host.view(np.uint32)), name


# ------------------------------------------------------------------ whole-output cases
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 63, 65, 129, 300])
def test_ragged_lengths(dtype, d, T):
    _full_compare(workload(dtype=dtype, head_dim=d, seqlen=T, batch=2, n_heads_q=2, n_heads_kv=2, n_depth=3,
                           seed=T + d))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,S_cap", [(0, 0), (1, 1), (3, 5), (8, 8), (13, 13)])
def test_depth_counts(dtype, S, S_cap):
    _full_compare(workload(dtype=dtype, head_dim=128, seqlen=200, batch=1, n_heads_q=2, n_heads_kv=2, n_depth=S,
                           depth_capacity=S_cap, seed=7 + S))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,S_cap,Hq,Hkv,d", [(65, 70, 2, 2, 128), (130, 130, 8, 2, 128), (97, 100, 8, 4, 64),
                                              (200, 201, 4, 1, 64)])
def test_many_depth_slots(dtype, S, S_cap, Hq, Hkv, d):
    # more slots than any load batch, round or selection width covers (64):
    # the depth pass's batches over slots wrap many times and end ragged
    _full_compare(workload(dtype=dtype, head_dim=d, seqlen=100, batch=1, n_heads_q=Hq, n_heads_kv=Hkv, n_depth=S,
                           depth_capacity=S_cap, seed=S + Hq))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 1), (8, 2), (16, 2), (6, 2), (3, 1), (12, 4)])
def test_grouped_heads(dtype, Hq, Hkv):
    _full_compare(workload(dtype=dtype, head_dim=64, seqlen=150, batch=2, n_heads_q=Hq, n_heads_kv=Hkv, n_depth=4,
                           seed=Hq * 10 + Hkv))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_not_causal(dtype, d):
    _full_compare(workload(dtype=dtype, head_dim=d, seqlen=190, batch=2, n_heads_q=4, n_heads_kv=2, n_depth=5,
                           causal=False, seed=31))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lens", [(5, 1, 130, 64, 0, 257), (1,), (128, 128), (127, 129, 2)])
def test_packed_sequences(dtype, lens):
    _full_compare(workload(dtype=dtype, head_dim=128, seqlens=tuple(lens), n_heads_q=4, n_heads_kv=4, n_depth=6,
                           seed=len(lens)))


def test_packed_grouped_d64():
    _full_compare(workload(dtype="bf16", head_dim=64, seqlens=(300, 17, 99), n_heads_q=8, n_heads_kv=2, n_depth=7,
                           seed=5))


def test_large_logits_stay_finite():
    w = workload(dtype="bf16", head_dim=128, seqlen=256, n_heads_q=4, n_heads_kv=4, n_depth=4, seed=9,
                 key_mult=16.0)
    _full_compare(w)


def test_lse_optional_and_stream():
    w = workload(dtype="bf16", head_dim=64, seqlen=130, n_heads_q=4, n_heads_kv=2, n_depth=3, seed=3)
    x = configs.make_device(w, "cuda")
    from joint_sequence_depth_amd import attn_fwd

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, _ = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], scale=w.scale)
    s.synchronize()
    out2 = torch.empty_like(x["q"])
    _, none = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], scale=w.scale, out=out2, return_lse=False)
    torch.cuda.synchronize()
    assert none is None
    ref_o, _ = oracle_full(w)
    check_out(w, to_np(out), ref_o)
    assert torch.equal(out, out2)


def test_deterministic():
    w = workload(dtype="bf16", head_dim=128, seqlen=333, n_heads_q=8, n_heads_kv=2, n_depth=5, seed=11)
    x, o1, l1 = run_hip(w)
    _, o2, l2 = run_hip(w, inputs=x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_joint_not_separate():
    """The kernel computes one softmax over both key sets, not softmax + softmax."""
    w = workload(dtype="bf16", head_dim=64, seqlen=128, n_heads_q=2, n_heads_kv=2, n_depth=4, seed=13)
    _, out, _ = run_hip(w)
    h = configs.make_host(w)
    sep = oracle.separate_then_add(h["q"], h["k"], h["v"], h["kd"], h["vd"], 4, True, w.scale)
    ref, _ = oracle_full(w)
    o = to_np(out)
    assert np.max(np.abs(o - ref)) < 0.25 * np.max(np.abs(o - sep))


def test_empty_inputs_are_noops():
    from joint_sequence_depth_amd import lib

    L = lib()
    assert L.moda_attn_fwd(None, None, None, None, None, None, None, 1, 1, 0, 128, 2, 2, 64, 0, 0, 1, 0.125, None) == 0
    assert L.moda_attn_fwd(None, None, None, None, None, None, None, 1, 1, 2, 0, 2, 2, 64, 0, 0, 1, 0.125, None) == 0
    assert L.moda_attn_fwd_varlen(None, None, None, None, None, None, None, 1, 1, None, 0, 0, 0, 2, 2, 64, 0, 0, 1,
                                  0.125, None) == 0


# ------------------------------------------------------------------ the five workloads
@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16"])
def test_workload_full_output(name):
    w = configs.WORKLOADS[name]
    err, ratio = _full_compare(w)
    _say(f"{name}: max err {err:.3e} (error/bound {ratio:.3f})")


@pytest.mark.parametrize("name", configs.ORDER)
def test_workload_sampled_rows(name):
    """Full-size workload, launched as the benchmark launches it (bf16 output)."""
    _sampled_compare(configs.WORKLOADS[name])


@pytest.mark.parametrize("case", list(SCHEDULE_CASES))
def test_tile_schedules(case):
    """Every tile schedule, checked on the kernel instance it must reach: the whole
    output where the oracle computes it in seconds, else sampled rows against the
    RMS of the whole output."""
    import bench

    w = schedule_workload(case)
    kern = bench.kernel_name(w)
    _say(f"{case}: {kern}")
    assert kern.endswith(SCHEDULE_CASES[case]["kernel"]), kern
    if SCHEDULE_CASES[case].get("whole"):
        _full_compare(w)
    else:
        _sampled_compare(w)


def _sampled_compare(w):
    """Sampled rows (t = 0, tile boundaries, each sequence's last token, random
    rows) checked element by element. The bf16 bound uses the RMS of the WHOLE
    reference output (stored by tests/golden/make_output_rms.py), not of the
    sampled rows: those favour early tokens, whose outputs are larger."""
    name = w.name
    rms = stored_rms(name) if w.bf16 else None
    _say(f"workload {name}: generating inputs on the device (whole-output rms {rms})")
    x, out, lse = run_hip(w)
    _, out32, _ = run_hip(w, inputs=x, out_f32=True) if w.bf16 else (None, None, None)
    rows = sample_rows(w, n_random=24, seed=3)
    got, got32, refs, lerr = [], [], [], 0.0
    for s, t, h in rows:
        ro, rl = oracle_row(w, s, t, h)
        go, gl = gpu_row(w, out, lse, s, t, h)
        got.append(go)
        refs.append(ro)
        if out32 is not None:
            got32.append(gpu_row(w, out32, lse, s, t, h)[0])
        lerr = max(lerr, abs(gl - rl))
    ref = np.stack(refs)
    err, ratio = check_out(w, np.stack(got), ref, name + " sampled", rms=rms)
    _say(f"{name}: {len(rows)} rows, max err {err:.3e} error/bound {ratio:.3f}, lse err {lerr:.2e}")
    if got32:
        err32, ratio32 = check_out(w, np.stack(got32), ref, name + " sampled fp32 out", out_bf16=False, rms=rms)
        _say(f"{name} fp32 out: max err {err32:.3e} error/bound {ratio32:.3f}")
    assert lerr <= (1e-3 if w.bf16 else 1e-5)
    del x, out, lse, out32
    torch.cuda.empty_cache()
