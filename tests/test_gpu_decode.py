"""Decode step (one new token per sequence) on the HIP path vs the fp64 oracle.

Small cases compare the whole output; the two decode workloads the benchmark
times are checked on sampled (sequence, head) rows recomputed from operands
regenerated on the host. Tolerances are those of the forward parity tests.
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import TOL_BF16_REL_RMS, check_lse, half_ulp_bf16, to_np
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


def dw(lengths, T_max=None, Hq=2, Hkv=2, d=64, S=3, S_cap=None, dtype="bf16", seed=300, key_mult=1.0):
    lengths = tuple(int(x) for x in lengths)
    return configs.DecodeWorkload("case", "", dtype, lengths, T_max or max(lengths), Hq, Hkv, d, S, seed,
                                  key_mult=key_mult, depth_capacity=S_cap)


def _tol(w, ref, out_bf16):
    if not w.bf16:
        return np.full(ref.shape, 1e-5)
    rms = float(np.sqrt(np.mean(ref**2))) if ref.size else 1.0
    e = TOL_BF16_REL_RMS * rms
    tol = np.full(ref.shape, e)
    return tol + half_ulp_bf16(np.abs(ref) + e) if out_bf16 else tol


def _check(w, out, ref, what, out_bf16):
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    diff = np.abs(out - ref)
    ratio = float(np.max(diff / _tol(w, ref, out_bf16)))
    assert ratio <= 1.0, f"{what}: max|out-ref| = {float(diff.max()):.3e}, worst error/bound = {ratio:.3f}"
    return float(diff.max()), ratio


def _run(w, x, out_f32=False, **kw):
    from joint_sequence_depth_amd import attn_decode

    if out_f32:
        kw["out_dtype"] = torch.float32
    out, lse = attn_decode(x["q"], x["k"], x["v"], x["seqlens"], x["kd"], x["vd"], n_depth=w.n_depth,
                           scale=w.scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def _oracle(w, lengths=None):
    h = configs.make_decode_host(w)
    lens = h["seqlens"] if lengths is None else lengths
    return oracle.decode(h["q"], h["k"], h["v"], lens, h["kd"], h["vd"], w.n_depth, w.scale)


def _full_compare(w, both_outputs=True):
    _say(f"decode case B={w.batch} lens={w.cache_lengths[:8]} T_max={w.max_cache_len} Hq={w.n_heads_q} "
         f"Hkv={w.n_heads_kv} d={w.head_dim} S={w.n_depth}/{w.s_cap} {w.dtype}")
    ref_o, ref_l = _oracle(w)
    x = configs.make_decode_device(w, "cuda")
    for out_f32 in ([False, True] if (w.bf16 and both_outputs) else [False]):
        out, lse = _run(w, x, out_f32=out_f32)
        err, ratio = _check(w, to_np(out), ref_o, f"out_f32={out_f32}", out_bf16=w.bf16 and not out_f32)
        check_lse(w, to_np(lse), ref_l, "decode")
        _say(f"  out_f32={out_f32}: max err {err:.3e}, error/bound {ratio:.3f}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lengths", [(1,), (1, 2, 63, 64, 65), (129, 1, 300, 257), (1000, 17)])
def test_decode_ragged_lengths(dtype, d, lengths):
    _full_compare(dw(lengths, d=d, dtype=dtype, seed=len(lengths) + d))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,S_cap", [(0, 0), (0, 4), (1, 1), (3, 5), (8, 8), (46, 46), (70, 80)])
def test_decode_depth_counts(dtype, S, S_cap):
    _full_compare(dw((200, 37, 1), d=128, S=S, S_cap=S_cap, dtype=dtype, seed=11 + S))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 1), (8, 2), (16, 2), (32, 2), (6, 2), (3, 1), (12, 4), (24, 8)])
def test_decode_grouped_heads(dtype, Hq, Hkv):
    _full_compare(dw((150, 1, 77), Hq=Hq, Hkv=Hkv, d=128, S=5, dtype=dtype, seed=Hq * 10 + Hkv))


@pytest.mark.parametrize("d", [64, 128])
def test_decode_many_chunks(d):
    # one (sequence, KV head) pair: the key range splits into many chunks, with a
    # ragged last chunk and a sequence whose prefix ends inside the first chunk
    _full_compare(dw((5000, 3), T_max=5003, Hq=1, Hkv=1, d=d, S=6, seed=d + 1))


def test_decode_depth_dominates():
    # depth keys scaled up so the depth slots hold most of the probability mass
    w = dw((40, 90), Hq=4, Hkv=2, d=128, S=12, seed=5, key_mult=2.0)
    _full_compare(w)


def test_decode_lengths_are_clamped():
    # stored lengths of 0 and above T_max read as 1 and T_max
    w = dw((5, 70), T_max=70, Hq=2, Hkv=1, d=64, S=2, seed=9)
    x = configs.make_decode_device(w, "cuda")
    x["seqlens"] = torch.tensor([0, 99], dtype=torch.int32, device="cuda")
    out, lse = _run(w, x)
    ref_o, ref_l = _oracle(w, lengths=np.array([1, 70]))
    _check(w, to_np(out), ref_o, "clamped", out_bf16=True)
    check_lse(w, to_np(lse), ref_l, "clamped")


def test_decode_without_lse_and_workspace_reuse():
    from joint_sequence_depth_amd import decode_workspace_size

    big = dw((300, 1, 64, 257), Hq=8, Hkv=2, d=128, S=4, seed=21)
    small = dw((3, 90), Hq=8, Hkv=2, d=128, S=4, seed=22)
    n = decode_workspace_size(big.batch, 8, 2, 128, big.max_cache_len)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-filled floats on entry
    for w in (big, small, big):
        x = configs.make_decode_device(w, "cuda")
        out, lse = _run(w, x, workspace=ws, return_lse=False)
        assert lse is None
        ref_o, _ = _oracle(w)
        _check(w, to_np(out), ref_o, "workspace reuse", out_bf16=True)


def test_decode_preallocated_outputs():
    w = dw((120, 33), Hq=4, Hkv=4, d=64, S=3, seed=31)
    x = configs.make_decode_device(w, "cuda")
    out = torch.full(w.shape_q(), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.batch, w.n_heads_q), float("nan"), dtype=torch.float32, device="cuda")
    o2, l2 = _run(w, x, out=out, lse=lse)
    assert o2.data_ptr() == out.data_ptr() and l2.data_ptr() == lse.data_ptr()
    ref_o, ref_l = _oracle(w)
    _check(w, to_np(out), ref_o, "prealloc", out_bf16=False)
    check_lse(w, to_np(lse), ref_l, "prealloc")


def test_decode_empty_batch():
    from joint_sequence_depth_amd import attn_decode

    q = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((0, 8, 2, 64), dtype=torch.bfloat16, device="cuda")
    L = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out, lse = attn_decode(q, kc, kc, L)
    assert out.shape == (0, 4, 64) and lse.shape == (0, 4)


# ------------------------------------------------------------------ the benchmarked workloads, sampled rows
def _sample(w, n_random=20, seed=0):
    rng = np.random.default_rng(seed)
    rows = {(b, int(rng.integers(0, w.n_heads_q))) for b in range(min(w.batch, 4))}
    rows |= {(int(rng.integers(0, w.batch)), int(rng.integers(0, w.n_heads_q))) for _ in range(n_random)}
    rows.add((w.batch - 1, w.n_heads_q - 1))
    return sorted(rows)


def _oracle_row(w, b, h):
    d = w.head_dim
    hk = h // w.group
    c = np.arange(d)
    L = w.cache_lengths[b]
    q = configs.decode_host_slice(w, "q", (np.full(d, b), np.full(d, h), c))[None, None]
    J = np.arange(L)
    kidx = (np.full((L, d), b), J[:, None], np.full((L, d), hk), c[None, :])
    k = configs.decode_host_slice(w, "k", kidx)[None, :, None]
    v = configs.decode_host_slice(w, "v", kidx)[None, :, None]
    S = w.n_depth
    if S > 0:
        i = np.arange(S)
        didx = (np.full((S, d), b), i[:, None], np.full((S, d), hk), c[None, :])
        kd = configs.decode_host_slice(w, "kd", didx)[None, :, None]
        vd = configs.decode_host_slice(w, "vd", didx)[None, :, None]
    else:
        kd = vd = None
    o, l = oracle.decode(q, k, v, np.array([L]), kd, vd, S, w.scale)
    return o[0, 0], float(l[0, 0])


@pytest.mark.parametrize("name", list(configs.DECODE_WORKLOADS))
def test_decode_workload_sampled(name):
    w = configs.DECODE_WORKLOADS[name]
    _say(f"decode workload {name}")
    x = configs.make_decode_device(w, "cuda")
    out, lse = _run(w, x)
    out, lse = to_np(out), to_np(lse)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    rows = _sample(w)
    refs = [_oracle_row(w, b, h) for b, h in rows]
    ref_o = np.stack([r[0] for r in refs])
    got_o = np.stack([out[b, h] for b, h in rows])
    _check(w, got_o, ref_o, name, out_bf16=True)
    check_lse(w, np.array([lse[b, h] for b, h in rows]), np.array([r[1] for r in refs]), name)
