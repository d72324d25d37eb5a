"""The parity bound itself (CPU): half-ulp arithmetic and the bound's independence
from the output under test."""
import numpy as np

from parity_util import check_out, half_ulp_bf16, tolerance, workload
from workloads import gen


def test_half_ulp_matches_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-10, 10, 200000))).astype(np.float32)
    r = gen.round_bf16_np(x).astype(np.float64)
    assert np.all(np.abs(r - x.astype(np.float64)) <= half_ulp_bf16(x.astype(np.float64)))
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0**-8
    assert half_ulp_bf16(np.array([0.75]))[0] == 2.0**-9


def test_bound_rejects_large_errors():
    w = workload(dtype="bf16")
    ref = np.random.default_rng(1).standard_normal((50, 8)) * 0.1
    t = tolerance(w, ref)
    assert np.all(t < 0.01)
    bad = ref.copy()
    bad[3, 2] = 1e6
    try:
        check_out(w, bad, ref, record=False)
    except AssertionError:
        pass
    else:
        raise AssertionError("bound accepted a wild output")
    # the correctly rounded reference always passes
    check_out(w, gen.round_bf16_np(ref.astype(np.float32)).astype(np.float64), ref, record=False)


# ------------------------------------------------------------------ backward bound (bf16 inputs)
import os  # noqa: E402
import types  # noqa: E402

import oracle  # noqa: E402
from parity_util import bwd_rounding_magnitudes, check_grad_bf16  # noqa: E402
from workloads import configs  # noqa: E402


def _rb(x):
    return gen.round_bf16_np(np.asarray(x, dtype=np.float32)).astype(np.float64)


def _rounded_backward(h, w, dout):
    """dq, dk, dv of the sequence keys with the bf16 path's rounding points applied
    in float64 (MHA, batch layout, depth included in the softmax): out stored in
    bf16, P rounded in dv = P^T dout, dS rounded in dq and dk."""
    out, lse = oracle.joint_attention(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, w.causal, w.scale)
    B, T, H, d = h["q"].shape
    dq, dk, dv = np.zeros((B, T, H, d)), np.zeros((B, T, H, d)), np.zeros((B, T, H, d))
    S = w.n_depth
    for b in range(B):
        for hh in range(H):
            q, k, v = (h[n][b, :, hh].astype(np.float64) for n in ("q", "k", "v"))
            dO = dout[b, :, hh].astype(np.float64)
            delta = np.sum(dO * _rb(out[b, :, hh]), axis=1)
            s = np.where(np.tril(np.ones((T, T))) > 0, w.scale * q @ k.T, -np.inf)
            P = np.exp(s - lse[b, hh][:, None])
            dS = _rb(P * (dO @ v.T - delta[:, None]))
            dq[b, :, hh] = w.scale * dS @ k
            dk[b, :, hh] = w.scale * dS.T @ q
            dv[b, :, hh] = _rb(P).T @ dO
            if S:
                kd, vd = h["kd"][b, :, :S, hh], h["vd"][b, :, :S, hh]
                pb = np.exp(w.scale * np.einsum("tc,tsc->ts", q, kd) - lse[b, hh][:, None])
                dq[b, :, hh] += w.scale * np.einsum("ts,tsc->tc", pb * (np.einsum("tc,tsc->ts", dO, vd) - delta[:, None]),
                                                     kd)
    return dq, dk, dv


BWD_CASES = [
    dict(head_dim=128, seqlen=300, batch=2, n_heads_q=2, n_heads_kv=2, n_depth=3, seed=1428),
    dict(head_dim=64, seqlen=190, batch=1, n_heads_q=2, n_heads_kv=2, n_depth=4, key_mult=4.0, seed=1600),
]


def _bwd_case(kw):
    w = workload(dtype="bf16", **kw)
    h = configs.make_host(w)
    dout = configs.make_dout_host(w, True)
    ref = oracle.joint_attention_backward(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, dout, True, w.scale)
    mags = bwd_rounding_magnitudes(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, dout, True, w.scale)
    return w, h, dout, ref, mags


def test_bwd_bound_admits_the_bf16_roundings():
    """The bf16 path's own rounding points, applied exactly in float64, stay inside
    the bound (with room: the worst ratio is well below one)."""
    for kw in BWD_CASES:
        w, h, dout, ref, mags = _bwd_case(kw)
        got = _rounded_backward(h, w, dout)
        for i in range(3):
            _, ratio = check_grad_bf16(w, got[i], ref[i], mags[i], f"grad {i}", grad_bf16=False)
            assert ratio < 0.5, ratio


SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moda_oracle.py")
PLANTED = {
    "diagonal key dropped": ("rows[:, None] >= np.arange(kend)", "rows[:, None] > np.arange(kend)"),
    "depth share of dq dropped": ("dq[st + r0 : st + r1, h] += scale * np.sum(dSb", "dq[st + r0 : st + r1, h] += 0.0 * np.sum(dSb"),
    "depth left out of delta": ("rowdot = rowdot + np.sum(Pb * dPb, axis=1)", "rowdot = rowdot + 0.0"),
    "first key dropped": ("a = np.where(rows[:, None] >= np.arange(kend)[None, :], a, -np.inf)",
                          "a = np.where((rows[:, None] >= np.arange(kend)[None, :]) & (np.arange(kend)[None, :] > 0), a, -np.inf)"),
}


def test_bwd_bound_rejects_planted_mistakes():
    """Plausible kernel mistakes, planted in a copy of the oracle, exceed the bound."""
    for kw in BWD_CASES:
        w, h, dout, ref, mags = _bwd_case(kw)
        for name, (old, new) in PLANTED.items():
            src = open(SRC).read()
            assert src.count(old) == 1, name
            mod = types.ModuleType("planted")
            exec(compile(src.replace(old, new), "planted", "exec"), mod.__dict__)
            bad = mod.joint_attention_backward(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, dout, True, w.scale)
            caught = False
            for i in range(5):
                g, r, m = bad[i], ref[i], mags[i]
                if i >= 3:
                    g, r, m = g[:, :, : w.n_depth], r[:, :, : w.n_depth], m[:, :, : w.n_depth]
                try:
                    check_grad_bf16(w, g, r, m, name, grad_bf16=True)
                except AssertionError:
                    caught = True
            assert caught, f"bound accepts: {name}"
