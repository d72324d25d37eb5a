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

import numpy as np

import oracle
from workloads import configs

TOL_F32 = 1e-5
TOL_BF16_REL_RMS = 2e-2
TOL_LSE_F32 = 1e-5
TOL_LSE_BF16 = 1e-3


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


def tolerance(w, ref, out_bf16=True):
    """Per-element bound (array) for an output compared with the fp64 reference."""
    if not w.bf16:
        return np.full(ref.shape, TOL_F32)
    rms = float(np.sqrt(np.mean(ref**2))) if ref.size else 1.0
    e = TOL_BF16_REL_RMS * rms
    tol = np.full(ref.shape, e)
    if out_bf16:
        tol = tol + half_ulp_bf16(np.abs(ref) + e)
    return tol


def check_out(w, out, ref, what="", out_bf16=None):
    """Assert the bound elementwise; returns (max error, max error / bound)."""
    if out_bf16 is None:
        out_bf16 = w.bf16
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    if not out.size:
        return 0.0, 0.0
    diff = np.abs(out - ref)
    tol = tolerance(w, ref, out_bf16)
    ratio = float(np.max(diff / tol))
    err = float(np.max(diff))
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
