"""Bounded depth reads (top-S, sliding window, hybrid: moda_attn_fwd_topk /
moda_attn_fwd_varlen_topk) on the HIP path vs the fp64 oracle, on an MI355X.

Reading (MoDA deck, slide "The main open cost is retaining and reading depth
history"): of a row's slots, the last ``recent`` always enter its softmax and of
the others the ``topk`` with the largest depth logits, ties to the lower slot.

The selection is an integer decision taken from floating-point logits: the
kernel ranks fp32 logits, the oracle fp64 ones. Where the oracle's k-th and
(k+1)-th largest logits of a row lie within 1e-4 of each other, both choices are
correct readings of the row at fp32 precision, so such rows are checked against
the oracle under either choice; every other row is compared element by element
with the usual bound.
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import check_lse, check_out, to_np, workload
from workloads import configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NEAR_TIE = 1e-4  # logit gap below which either side of the selection boundary is accepted


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _packed(w, h):
    """Host operands in packed layout [N, ...] and cu_seqlens."""
    if w.varlen:
        return h["q"], h["k"], h["v"], h["kd"], h["vd"], w.cu_seqlens()
    B, T = w.batch, w.seqlen
    f = lambda x: x.reshape((B * T,) + x.shape[2:])  # noqa: E731
    return f(h["q"]), f(h["k"]), f(h["v"]), f(h["kd"]), f(h["vd"]), np.arange(B + 1) * T


def _boundary_rows(w, h, topk, recent):
    """Rows (token n, head hq) whose selection boundary is a near-tie, with the
    slot sets of both readings."""
    q, _, _, kd, _, _ = _packed(w, h)
    S, G = w.n_depth, w.group
    old = S - min(recent, S)
    k = min(topk, old)
    if k <= 0 or k >= old:
        return {}
    kdh = np.repeat(kd[:, :S].astype(np.float64), G, axis=2)  # [N, S, Hq, d]
    b = w.scale * np.einsum("nhc,nshc->nhs", q.astype(np.float64), kdh)  # [N, Hq, S]
    order = np.argsort(-b[:, :, :old], axis=2, kind="stable")
    srt = np.take_along_axis(b[:, :, :old], order, axis=2)
    gap = srt[:, :, k - 1] - srt[:, :, k]
    out = {}
    for n, hq in zip(*np.nonzero(gap < NEAR_TIE)):
        first = list(order[n, hq, :k])
        alt = first[:-1] + [order[n, hq, k]]
        # every slot whose logit ties with the boundary could take its place; the two
        # nearest orders are what fp32 rounding can produce
        out[(int(n), int(hq))] = [sorted(first) + list(range(old, S)), sorted(alt) + list(range(old, S))]
    return out


def _lse_rows(w, lse):
    """lse [B,Hq,T] or [Hq,N] -> [N, Hq] (token-major, like out)."""
    if w.varlen:
        return lse.T
    return lse.transpose(0, 2, 1).reshape(-1, w.n_heads_q)


def _row_ref(w, h, n, hq, slots):
    q, k, v, kd, vd, cu = _packed(w, h)
    s = int(np.searchsorted(cu, n, side="right") - 1)
    start, end = int(cu[s]), int(cu[s + 1])
    hk = hq // w.group
    J = np.arange(start, n + 1 if w.causal else end)
    sl = np.array(slots, dtype=np.int64)
    return oracle.joint_rows(q[n, hq], k[J, hk], v[J, hk], kd[n, sl, hk] if len(sl) else None,
                             vd[n, sl, hk] if len(sl) else None, w.scale)


# every schedule of the bf16 kernel the workloads use (split tiles, shared tiles of
# one, two or four heads per workgroup at both head dims), packed sequences with an
# empty one, the fp32 path and the largest slot count a mask holds
CASES = {
    "split_d64": dict(dtype="bf16", head_dim=64, seqlen=300, batch=1, n_heads_q=2, n_heads_kv=2, n_depth=9),
    "shared_d128_g1": dict(dtype="bf16", head_dim=128, seqlen=1024, batch=1, n_heads_q=64, n_heads_kv=64,
                           n_depth=12),
    "shared_d64_g4": dict(dtype="bf16", head_dim=64, seqlen=1024, batch=1, n_heads_q=32, n_heads_kv=8, n_depth=10),
    "shared_d128_g4": dict(dtype="bf16", head_dim=128, seqlen=2048, batch=1, n_heads_q=32, n_heads_kv=8, n_depth=6),
    "split_d128_g2": dict(dtype="bf16", head_dim=128, seqlen=257, batch=2, n_heads_q=4, n_heads_kv=2, n_depth=20,
                          depth_capacity=24),
    "packed_d128": dict(dtype="bf16", head_dim=128, seqlens=(5, 1, 130, 64, 0, 257), n_heads_q=4, n_heads_kv=4,
                        n_depth=8),
    "fp32_d64": dict(dtype="f32", head_dim=64, seqlen=129, batch=2, n_heads_q=4, n_heads_kv=2, n_depth=7),
    "slots_64": dict(dtype="bf16", head_dim=128, seqlen=200, batch=1, n_heads_q=4, n_heads_kv=2, n_depth=64),
    # split tiles of four heads: one token group per wave, so the first value step
    # is issued after the ranking; at d = 64 half of its lane groups lie past the
    # wave's tokens
    "split_d64_g4": dict(dtype="bf16", head_dim=64, seqlen=200, batch=1, n_heads_q=8, n_heads_kv=2, n_depth=11),
    "split_d128_g4": dict(dtype="bf16", head_dim=128, seqlen=150, batch=1, n_heads_q=8, n_heads_kv=2, n_depth=9),
}
SELECTIONS = [(1, 0), (4, 0), (3, 2), (0, 3)]


@pytest.mark.parametrize("name", list(CASES))
def test_topk_matches_oracle(name):
    from joint_sequence_depth_amd import attn_fwd

    w = workload(name=name, seed=80 + list(CASES).index(name), **CASES[name])
    x = configs.make_device(w, "cuda")
    h = configs.make_host(w)
    cu_h = w.cu_seqlens() if w.varlen else None
    cu = torch.from_numpy(cu_h).cuda() if w.varlen else None
    for topk, recent in SELECTIONS:
        ref, ref_l = oracle.joint_attention(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, w.causal,
                                            w.scale, cu_seqlens=cu_h, depth_topk=topk, depth_recent=recent)
        ties = _boundary_rows(w, h, topk, recent)
        for out_f32 in ([False, True] if w.bf16 else [False]):
            tag = f"{name} topk={topk} recent={recent} out_f32={out_f32}"
            _say(tag)
            out, lse = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, causal=w.causal,
                                scale=w.scale, cu_seqlens=cu, max_seqlen=max(w.lengths) if w.varlen else None,
                                out_dtype=torch.float32 if out_f32 else None, depth_topk=topk, depth_recent=recent)
            torch.cuda.synchronize()
            o, lo = to_np(out), to_np(lse)
            flat_o = o.reshape(-1, w.n_heads_q, w.head_dim)
            flat_r = ref.reshape(-1, w.n_heads_q, w.head_dim).copy()
            rms = float(np.sqrt(np.mean(ref**2)))
            for (n, hq), choices in ties.items():  # near-tie rows: either choice is a correct reading
                refs = [_row_ref(w, h, n, hq, c)[0] for c in choices]
                best = min(refs, key=lambda r: float(np.max(np.abs(flat_o[n, hq] - r))))
                flat_r[n, hq] = best
            r = check_out(w, flat_o, flat_r, tag, out_bf16=w.bf16 and not out_f32, rms=rms)
            keep = np.ones((flat_o.shape[0], w.n_heads_q), dtype=bool)  # lse of the rows without a near-tie
            for n, hq in ties:
                keep[n, hq] = False
            check_lse(w, _lse_rows(w, lo)[keep], _lse_rows(w, ref_l)[keep], tag)
            _say(f"  max err {r[0]:.3e}, error/bound {r[1]:.3f}, near-tie rows {len(ties)}")


def test_topk_covering_every_slot_is_the_operator():
    from joint_sequence_depth_amd import attn_fwd

    w = workload(dtype="bf16", head_dim=128, seqlen=333, n_heads_q=8, n_heads_kv=2, n_depth=6, seed=90)
    x = configs.make_device(w, "cuda")
    o1, l1 = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], scale=w.scale)
    o2, l2 = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], scale=w.scale, depth_topk=6)
    o3, l3 = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], scale=w.scale, depth_topk=2, depth_recent=4)
    o4, l4 = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=0, scale=w.scale)
    o5, l5 = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], scale=w.scale, depth_topk=0, depth_recent=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert torch.equal(o4, o5) and torch.equal(l4, l5)
