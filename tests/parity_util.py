"""Shared helpers for the parity tests: run the HIP path, regenerate operands on
the host, evaluate the oracle, and apply the tolerances.

Tolerances. fp32 inputs: max |out - ref| <= 1e-5. bf16 inputs (fp32 accumulation):
max |out - ref| <= 2e-2 * RMS(ref), RMS over the whole compared output. That bound
applies as written to an fp32 output. A bf16 output is that result rounded once to
nearest-even, which by itself moves an element by up to half a bf16 ulp of its
value (2^-9 relative); rows that average few values can exceed ten times the RMS,
where that rounding alone is larger than 2e-2 * RMS. So a bf16 output gets, per
element, e + half a bf16 ulp at |ref| + e, with e = 2e-2 * RMS(ref): the value
before the final rounding is within e of ref, and rounding moves it by at most half
an ulp at its own magnitude. The bound never depends on the kernel's output.
lse (natural log of the joint denominator, fp32 in both paths): <= 1e-5 absolute
for fp32 inputs and <= 1e-3 for bf16 inputs.
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np

import oracle
from workloads import configs

TOL_F32 = 1e-5
TOL_BF16_REL_RMS = 2e-2
TOL_LSE_F32 = 1e-5
TOL_LSE_BF16 = 1e-3

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# (check, max error, worst error/bound) of every comparison made in this process,
# printed at the end of the pytest run (tests/conftest.py)
RESULTS: list = []


def stored_rms(name: str) -> float:
    """RMS of the whole reference output of a sampled workload, written by
    tests/golden/make_output_rms.py from the oracle alone."""
    with open(os.path.join(GOLDEN, "output_rms.json")) as f:
        return float(json.load(f)[name]["rms"])


def workload(**kw) -> configs.Workload:
    base = dict(name="case", desc="", dtype="bf16", batch=1, seqlen=64, n_heads_q=2, n_heads_kv=2,
                head_dim=64, n_depth=3, seed=100)
    base.update(kw)
    if base.get("seqlens") is not None:
        base["seqlen"] = int(sum(base["seqlens"]))
        base["batch"] = 1
    return configs.Workload(**base)


def run_hip(w: configs.Workload, dev="cuda", batch_index=0, inputs=None, out_f32=False, **call_kw):
    import torch

    from joint_sequence_depth_amd import attn_fwd

    x = inputs if inputs is not None else configs.make_device(w, dev, batch_index)
    cu = None
    if w.varlen:
        cu = torch.from_numpy(w.cu_seqlens()).to(dev)
        call_kw.setdefault("max_seqlen", max(w.lengths))
    if out_f32:
        call_kw["out_dtype"] = torch.float32
    out, lse = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, causal=w.causal,
                        scale=w.scale, cu_seqlens=cu, **call_kw)
    torch.cuda.synchronize()
    return x, out, lse


def oracle_full(w: configs.Workload, batch_index=0):
    h = configs.make_host(w, batch_index)
    cu = w.cu_seqlens() if w.varlen else None
    return oracle.joint_attention(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, w.causal, w.scale,
                                  cu_seqlens=cu)


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def half_ulp_bf16(x):
    """Half a bfloat16 ulp at |x| (8 significant bits): 2^(e-9) for |x| = m 2^e, m in [0.5, 1)."""
    _, e = np.frexp(np.abs(x))
    return np.where(x != 0, np.ldexp(1.0, e - 9), 0.0)


def tolerance(w, ref, out_bf16=True, rms=None):
    """Per-element bound (array) for an output compared with the fp64 reference.
    ``rms``: the RMS of the whole reference output when ``ref`` holds only some of
    its rows (default: the RMS of ``ref`` itself)."""
    if not w.bf16:
        return np.full(ref.shape, TOL_F32)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref**2))) if ref.size else 1.0
    e = TOL_BF16_REL_RMS * rms
    tol = np.full(ref.shape, e)
    if out_bf16:
        tol = tol + half_ulp_bf16(np.abs(ref) + e)
    return tol


def check_out(w, out, ref, what="", out_bf16=None, rms=None, record=True):
    """Assert the bound elementwise; returns (max error, max error / bound).
    ``record``: list the ratio in the session's parity summary (off for checks of
    the checker itself, such as a planted failure)."""
    if out_bf16 is None:
        out_bf16 = w.bf16
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    if not out.size:
        return 0.0, 0.0
    diff = np.abs(out - ref)
    tol = tolerance(w, ref, out_bf16, rms)
    ratio = float(np.max(diff / tol))
    err = float(np.max(diff))
    if record:
        RESULTS.append((what or w.name, err, ratio))
    assert ratio <= 1.0, f"{what}: max|out-ref| = {err:.3e}, worst error/bound = {ratio:.3f}"
    return err, ratio


def check_lse(w, lse, ref, what=""):
    tol = TOL_LSE_BF16 if w.bf16 else TOL_LSE_F32
    err = float(np.max(np.abs(lse - ref))) if lse.size else 0.0
    assert np.all(np.isfinite(lse)), f"{what}: non-finite lse"
    assert err <= tol, f"{what}: max|lse-ref| = {err:.3e} > tol {tol:.3e}"
    return err


# --------------------------------------------------------------------------- sampled rows


def sample_rows(w: configs.Workload, n_random=24, seed=0, tile=128):
    """(segment, t, head) triples: t = 0, tile boundaries, the last token, plus random rows."""
    rng = np.random.default_rng(seed)
    rows = []
    lengths = w.lengths
    for s, L in enumerate(lengths):
        ts = {0, L - 1, min(L - 1, tile - 1), min(L - 1, tile), L // 2}
        ts |= {int(x) for x in rng.integers(0, L, size=2)}
        for t in sorted(ts):
            rows.append((s, t, int(rng.integers(0, w.n_heads_q))))
    for _ in range(n_random):
        s = int(rng.integers(0, len(lengths)))
        rows.append((s, int(rng.integers(0, lengths[s])), int(rng.integers(0, w.n_heads_q))))
    return rows


def _lead(w, s, t):
    """Leading index tuple of token t of segment s."""
    if w.varlen:
        return (int(w.cu_seqlens()[s]) + t,)
    return (s, t)


def oracle_row(w: configs.Workload, s: int, t: int, h: int, batch_index=0):
    """Oracle output row from operands regenerated on the host (numpy generator)."""
    d = w.head_dim
    hk = h // w.group
    c = np.arange(d)
    L = w.lengths[s]
    lead = _lead(w, s, t)
    q = configs.host_slice(w, "q", tuple(np.full(d, x) for x in lead) + (np.full(d, h), c), batch_index)
    J = np.arange(t + 1 if w.causal else L)
    if w.varlen:
        tok = int(w.cu_seqlens()[s]) + J
        kidx = (tok[:, None], np.full((len(J), d), hk), c[None, :])
    else:
        kidx = (np.full((len(J), d), s), J[:, None], np.full((len(J), d), hk), c[None, :])
    k = configs.host_slice(w, "k", kidx, batch_index)
    v = configs.host_slice(w, "v", kidx, batch_index)
    S = w.n_depth
    if S > 0:
        i = np.arange(S)
        didx = tuple(np.full((S, d), x) for x in lead) + (i[:, None], np.full((S, d), hk), c[None, :])
        kd = configs.host_slice(w, "kd", didx, batch_index)
        vd = configs.host_slice(w, "vd", didx, batch_index)
    else:
        kd = vd = None
    return oracle.joint_rows(q, k, v, kd, vd, w.scale)


def gpu_row(w, out, lse, s, t, h):
    lead = _lead(w, s, t)
    o = out[lead + (h,)]
    if w.varlen:
        l = lse[h, lead[0]]
    else:
        l = lse[s, h, t]
    return to_np(o), float(l)


def with_(w, **kw):
    return dataclasses.replace(w, **kw)


# --------------------------------------------------------------------------- tile schedules

# Mid-size shapes that reach every tile schedule of the bf16 kernel (the host picks
# it from the tile count): shared tiles of 4 and 2 waves, one, two or four query
# heads per workgroup, both head dims, and split tiles (waves dividing one tile's
# key blocks). Each names the kernel instance it must reach. "whole" cases are
# small enough for the oracle to compute their whole output in seconds; the
# others are checked on sampled rows against the RMS of their whole output.
SCHEDULE_CASES = {
    "shared4_d64": dict(head_dim=64, batch=4, seqlen=2048, n_heads_q=16, n_heads_kv=16, n_depth=8,
                        kernel="<64, 1, 4, 1, false, false>"),
    "shared2_d64": dict(head_dim=64, batch=1, seqlen=2048, n_heads_q=16, n_heads_kv=16, n_depth=8,
                        kernel="<64, 1, 2, 1, false, false>"),
    "split_d64_g2": dict(head_dim=64, batch=1, seqlen=1024, n_heads_q=8, n_heads_kv=4, n_depth=11,
                         kernel="<64, 2, 2, 1, false, true>"),
    "shared2_d128_g4": dict(head_dim=128, batch=1, seqlen=2048, n_heads_q=16, n_heads_kv=4, n_depth=9,
                            kernel="<128, 4, 2, 1, false, false>"),
    "shared4_d128_g2": dict(head_dim=128, batch=2, seqlen=2048, n_heads_q=16, n_heads_kv=8, n_depth=6,
                            kernel="<128, 2, 4, 1, false, false>"),
    "split_d128": dict(head_dim=128, batch=1, seqlen=1500, n_heads_q=4, n_heads_kv=4, n_depth=13,
                       kernel="<128, 1, 2, 1, false, true>"),
    # one 65536-token sequence: 512 query blocks, up to 1024 key blocks per tile
    # (the headline instance, with the plain tile order: two pairs)
    "long_d128": dict(head_dim=128, batch=1, seqlen=65536, n_heads_q=2, n_heads_kv=2, n_depth=4,
                      kernel="<128, 1, 4, 1, false, false>"),
    # whole-output cases
    "whole_shared2_d64_g4": dict(head_dim=64, batch=1, seqlen=1024, n_heads_q=32, n_heads_kv=8, n_depth=5,
                                 kernel="<64, 4, 2, 1, false, false>", whole=True),
    "whole_shared4_d64_g4": dict(head_dim=64, batch=2, seqlen=2048, n_heads_q=32, n_heads_kv=8, n_depth=5,
                                 kernel="<64, 4, 4, 1, false, false>", whole=True),
    "whole_shared4_d64_g2": dict(head_dim=64, batch=2, seqlen=2048, n_heads_q=16, n_heads_kv=8, n_depth=7,
                                 kernel="<64, 2, 4, 1, false, false>", whole=True),
    "whole_shared2_d128_g4": dict(head_dim=128, batch=1, seqlen=2048, n_heads_q=16, n_heads_kv=4, n_depth=9,
                                  kernel="<128, 4, 2, 1, false, false>", whole=True),
    "whole_shared4_d128_g1": dict(head_dim=128, batch=4, seqlen=2048, n_heads_q=8, n_heads_kv=8, n_depth=9,
                                  kernel="<128, 1, 4, 1, false, false>", whole=True),
    # the pair-major tile order (8 (sequence, KV head) pairs, H_kv not a multiple of
    # 8 or two head groups per KV head); the cases above with H_kv = 8 or 16 and
    # one head group take the KV-head-fastest order
    "whole_shared4_d128_g4_pairs": dict(head_dim=128, batch=2, seqlen=2048, n_heads_q=16, n_heads_kv=4, n_depth=7,
                                        kernel="<128, 4, 4, 1, false, false>", whole=True),
    "whole_shared4_d128_g8_pairs": dict(head_dim=128, batch=2, seqlen=1024, n_heads_q=32, n_heads_kv=4, n_depth=5,
                                        kernel="<128, 4, 4, 1, false, false>", whole=True),
}


def schedule_workload(case: str) -> configs.Workload:
    kw = {k: v for k, v in SCHEDULE_CASES[case].items() if k not in ("kernel", "whole")}
    return workload(name=case, dtype="bf16", seed=40 + list(SCHEDULE_CASES).index(case), **kw)


# --------------------------------------------------------------------------- backward


def bwd_tolerance(w, ref, grad_bf16):
    """Per-element bound for a gradient compared with the fp64 reference: the
    forward's rule (1e-5 absolute for fp32 inputs; 2e-2 RMS(ref) for bf16 inputs,
    plus half a bf16 ulp for bf16 gradients), RMS over the whole compared tensor."""
    return tolerance(w, ref, out_bf16=grad_bf16)


def check_grad(w, got, ref, what, grad_bf16):
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    if not got.size:
        return 0.0, 0.0
    diff = np.abs(got - ref)
    ratio = float(np.max(diff / bwd_tolerance(w, ref, grad_bf16)))
    err = float(np.max(diff))
    assert ratio <= 1.0, f"{what}: max|got-ref| = {err:.3e}, worst error/bound = {ratio:.3f}"
    return err, ratio


def unit_operands(w, s, hk, grad_bf16, batch_index=0):
    """Operands of one (segment, KV head) unit regenerated on the host: the G query
    heads of hk over the segment's tokens, as a batch-layout problem with B = 1:
    q, dout [1, L, G, d]; k, v [1, L, 1, d]; depth [1, L, S_cap, 1, d] (or None)."""
    d, G = w.head_dim, w.group
    L = w.lengths[s]
    if w.varlen:
        lead = (np.arange(int(w.cu_seqlens()[s]), int(w.cu_seqlens()[s]) + L),)
    else:
        lead = (np.array([s]), np.arange(L))

    def ix(*rest):
        if len(lead) == 2:
            idx = np.ix_(lead[0], lead[1], *rest)
            return tuple(a[0] for a in idx)
        return np.ix_(lead[0], *rest)

    hq = np.arange(hk * G, (hk + 1) * G)
    c = np.arange(d)
    q = configs.host_slice(w, "q", ix(hq, c), batch_index)[None]
    do = configs.host_slice(w, "do", ix(hq, c), batch_index, bf16=grad_bf16)[None]
    k = configs.host_slice(w, "k", ix(np.array([hk]), c), batch_index)[None]
    v = configs.host_slice(w, "v", ix(np.array([hk]), c), batch_index)[None]
    if w.s_cap > 0:
        i = np.arange(w.s_cap)
        kd = configs.host_slice(w, "kd", ix(i, np.array([hk]), c), batch_index)[None]
        vd = configs.host_slice(w, "vd", ix(i, np.array([hk]), c), batch_index)[None]
    else:
        kd = vd = None
    return q, k, v, kd, vd, do


BF16_U = 2.0**-8  # unit roundoff of bfloat16 (8 significant bits, nearest-even)


def bwd_rounding_magnitudes(q, k, v, kd, vd, n_depth, dout, causal, scale, cu_seqlens=None, row_block=256):
    """First-order rounding-error magnitudes of every gradient element of the bf16
    backward path, in float64, from the inputs alone (no kernel output).

    The bf16 path rounds to bf16 (unit roundoff u) where the exact derivative has
    none: the probabilities P in dv = P^T dout, the softmax gradient dS in
    dq = scale dS K and dk = scale dS^T Q, and dout where it enters the matrix
    products. Through the forward it also consumes out, itself computed with P in
    bf16 and stored in bf16: |delta error| <= 2 u D_t, D_t = sum_c |dout_tc| (P |V|)_tc.
    A sum sum_x a_x b_x whose a_x carry relative error u is off by at most
    u sum_x |a_x| |b_x|; so, with E_tx = u <|dout_t|, |value_x|> the error of dP:
        dq_tc  <- scale sum_x (u |dS_x| + P_x (2 u D_t + E_tx)) |key_xc|
        dk_jc  <- scale sum_t (u |dS_tj| + P_tj (2 u D_t + E_tj)) |q_tc|
        dv_jc  <- 2 u sum_t P_tj |dout_tc|
        dk_depth_{t,i,c} <- scale P_ti (2 u D_t + E_ti) |q_tc|,  dv_depth: 0
    Returns arrays shaped like (dq, dk, dv, dk_depth, dv_depth)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    kd = None if kd is None else np.asarray(kd, dtype=np.float64)
    vd = None if vd is None else np.asarray(vd, dtype=np.float64)
    u = BF16_U
    batch = cu_seqlens is None
    if batch:
        B, T = q.shape[:2]
        flat = lambda x: None if x is None else x.reshape((B * T,) + x.shape[2:])  # noqa: E731
        q, k, v, do, kd, vd = map(flat, (q, k, v, do, kd, vd))
        cu = np.arange(B + 1) * T
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    mkd = None if kd is None else np.zeros_like(kd)
    S = n_depth
    for s in range(len(cu) - 1):
        st, en = int(cu[s]), int(cu[s + 1])
        L = en - st
        for h in range(Hq):
            hk = h // G
            Q, dO, K, V = q[st:en, h], do[st:en, h], k[st:en, hk], v[st:en, hk]
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                rows = np.arange(r0, r1)
                kend = r1 if causal else L
                a = scale * (Q[r0:r1] @ K[:kend].T)
                if causal:
                    a = np.where(rows[:, None] >= np.arange(kend)[None, :], a, -np.inf)
                lg = [a]
                if S > 0:
                    KD, VD = kd[st + r0 : st + r1, :S, hk], vd[st + r0 : st + r1, :S, hk]
                    lg.append(scale * np.sum(Q[r0:r1][:, None, :] * KD, axis=2))
                M = np.max(np.concatenate(lg, axis=1), axis=1)
                Z = sum(np.exp(x - M[:, None]).sum(axis=1) for x in lg)
                Pa = np.exp(a - M[:, None]) / Z[:, None]
                dPa = dO[r0:r1] @ V[:kend].T
                Ea = u * (np.abs(dO[r0:r1]) @ np.abs(V[:kend]).T)
                PV = Pa @ np.abs(V[:kend])
                rowdot = np.sum(Pa * dPa, axis=1)
                if S > 0:
                    Pb = np.exp(lg[1] - M[:, None]) / Z[:, None]
                    dPb = np.sum(dO[r0:r1][:, None, :] * VD, axis=2)
                    Eb = u * np.sum(np.abs(dO[r0:r1])[:, None, :] * np.abs(VD), axis=2)
                    PV = PV + np.sum(Pb[:, :, None] * np.abs(VD), axis=1)
                    rowdot = rowdot + np.sum(Pb * dPb, axis=1)
                Dt = np.sum(np.abs(dO[r0:r1]) * PV, axis=1)
                wa = u * np.abs(Pa * (dPa - rowdot[:, None])) + Pa * (2 * u * Dt[:, None] + Ea)
                mq[st + r0 : st + r1, h] += scale * (wa @ np.abs(K[:kend]))
                mk[st : st + kend, hk] += scale * (wa.T @ np.abs(Q[r0:r1]))
                mv[st : st + kend, hk] += 2 * u * (Pa.T @ np.abs(dO[r0:r1]))
                if S > 0:
                    wb = u * np.abs(Pb * (dPb - rowdot[:, None])) + Pb * (2 * u * Dt[:, None] + Eb)
                    mq[st + r0 : st + r1, h] += scale * np.sum(wb[:, :, None] * np.abs(KD), axis=1)
                    mkd[st + r0 : st + r1, :S, hk] += scale * (Pb * (2 * u * Dt[:, None] + Eb))[:, :, None] * np.abs(
                        Q[r0:r1])[:, None, :]
    mvd = None if vd is None else np.zeros_like(vd)
    if batch:
        unflat = lambda x: None if x is None else x.reshape((B, T) + x.shape[1:])  # noqa: E731
        mq, mk, mv, mkd, mvd = map(unflat, (mq, mk, mv, mkd, mvd))
    return mq, mk, mv, mkd, mvd


def check_grad_bf16(w, got, ref, mag, what, grad_bf16):
    """bf16-input gradients: per element |got - ref| <= 2e-2 RMS(ref) + mag (the
    first-order rounding magnitude), plus half a bf16 ulp for bf16 storage."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    if not got.size:
        return 0.0, 0.0
    rms = float(np.sqrt(np.mean(ref**2)))
    e = TOL_BF16_REL_RMS * rms + mag
    tol = e + (half_ulp_bf16(np.abs(ref) + e) if grad_bf16 else 0.0)
    diff = np.abs(got - ref)
    ratio = float(np.max(diff / tol))
    assert ratio <= 1.0, f"{what}: max|got-ref| = {float(diff.max()):.3e}, worst error/bound = {ratio:.3f}"
    return float(diff.max()), ratio
