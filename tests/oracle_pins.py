"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` takes the oracle module and raises AssertionError on a violation,
so the same checks run against the real oracle (test_oracle_pins.py) and against
deliberately broken copies of it (test_oracle_mutants.py).

Sources: MoDA deck (arXiv 2603.15619), slides "One denominator allocates probability
across both memories" (the joint equation), "Shared online-softmax states preserve
the joint operator" (running-state merge), "Local packing avoids scanning irrelevant
depth entries" (Fig. 4 utilizations) and "Backup: grouped indexing preserves the
correct token map" (expanded-row map and its G = 4 example).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_case(seed, B=2, T=9, Hq=2, Hkv=1, d=8, S=3, Scap=None):
    rng = np.random.default_rng(seed)
    Scap = S if Scap is None else Scap
    q = rng.standard_normal((B, T, Hq, d))
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    kd = rng.standard_normal((B, T, Scap, Hkv, d))
    vd = rng.standard_normal((B, T, Scap, Hkv, d))
    return q, k, v, kd, vd


def _sdpa(q, k, v, causal, scale, attn_mask=None):
    """torch's scaled_dot_product_attention in float64 on [B,T,H,d] tensors."""
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    kt = torch.from_numpy(np.ascontiguousarray(np.repeat(k, G, axis=2).transpose(0, 2, 1, 3)))
    vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v, G, axis=2).transpose(0, 2, 1, 3)))
    m = None if attn_mask is None else torch.from_numpy(attn_mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal and m is None, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


# p1 -----------------------------------------------------------------------------
def pin_empty_depth_is_sdpa(orc):
    """An empty depth set leaves ordinary (causal) softmax attention: compare with
    torch's SDPA, an independent library routine, MHA and grouped heads."""
    for seed, (Hq, Hkv), causal in [(1, (2, 2), True), (2, (4, 2), True), (3, (4, 1), False), (4, (3, 3), False)]:
        q, k, v, kd, vd = rand_case(seed, B=2, T=11, Hq=Hq, Hkv=Hkv, d=8, S=2)
        scale = 0.37
        o, _ = orc.joint_attention(q, k, v, kd, vd, 0, causal, scale)
        ref = _sdpa(q, k, v, causal, scale)
        assert np.max(np.abs(o - ref)) < 1e-12, np.max(np.abs(o - ref))


# p2 -----------------------------------------------------------------------------
def pin_equal_logits_plain_mean(orc):
    """q = 0 makes every logit 0: the output is the plain mean of the visible values
    (t+1 sequence values and S depth values) and lse = ln(t+1+S)."""
    B, T, H, d, S = 2, 7, 2, 5, 3
    q, k, v, kd, vd = rand_case(5, B, T, H, H, d, S, Scap=S + 2)
    q[:] = 0
    for causal in (True, False):
        o, lse = orc.joint_attention(q, k, v, kd, vd, S, causal, 0.5)
        for b in range(B):
            for h in range(H):
                for t in range(T):
                    J = t + 1 if causal else T
                    mean = (v[b, :J, h].sum(0) + vd[b, t, :S, h].sum(0)) / (J + S)
                    assert np.max(np.abs(o[b, t, h] - mean)) < 1e-13
                    assert abs(lse[b, h, t] - math.log(J + S)) < 1e-13


# p3 -----------------------------------------------------------------------------
def pin_convex_and_affine(orc):
    """Weights are non-negative and sum to one: each output coordinate lies in the
    range of the visible values, o(v + c) = o + c and o(alpha v) = alpha o."""
    q, k, v, kd, vd = rand_case(6, B=1, T=10, Hq=2, Hkv=2, d=6, S=4)
    o, _ = orc.joint_attention(q, k, v, kd, vd, 4, True, 1.3)
    for t in range(10):
        for h in range(2):
            vals = np.concatenate([v[0, : t + 1, h], vd[0, t, :4, h]], axis=0)
            assert np.all(o[0, t, h] >= vals.min(0) - 1e-12) and np.all(o[0, t, h] <= vals.max(0) + 1e-12)
    c = np.linspace(-2, 3, 6)
    o2, _ = orc.joint_attention(q, k, v + c, kd, vd + c, 4, True, 1.3)
    assert np.max(np.abs(o2 - (o + c))) < 1e-12
    o3, _ = orc.joint_attention(q, k, 2.5 * v, kd, 2.5 * vd, 4, True, 1.3)
    assert np.max(np.abs(o3 - 2.5 * o)) < 1e-12


# p4 -----------------------------------------------------------------------------
def pin_lse_merge(orc):
    """Merging the sequence-only and depth-only running states (m, acc, o) the way
    the shared online-softmax update does gives the joint result:
    o = sigma(lse_s - lse_d) o_s + sigma(lse_d - lse_s) o_d, lse = logaddexp."""
    for seed, Hq, Hkv in [(7, 2, 2), (8, 4, 2)]:
        q, k, v, kd, vd = rand_case(seed, B=2, T=9, Hq=Hq, Hkv=Hkv, d=8, S=3)
        o, lse = orc.joint_attention(q, k, v, kd, vd, 3, True, 0.4)
        os_, ls = orc.sequence_only(q, k, v, True, 0.4)
        od, ld = orc.depth_only(q, k, v, kd, vd, 3, 0.4)
        lm = np.logaddexp(ls, ld)
        ws = np.exp(ls - lm).transpose(0, 2, 1)[..., None]
        wd = np.exp(ld - lm).transpose(0, 2, 1)[..., None]
        assert np.max(np.abs(lse - lm)) < 1e-12
        assert np.max(np.abs(o - (ws * os_ + wd * od))) < 1e-12


# p5 -----------------------------------------------------------------------------
def pin_separate_softmax_differs(orc):
    """Separate softmaxes followed by addition is a different operator."""
    q, k, v, kd, vd = rand_case(9, B=1, T=16, Hq=2, Hkv=2, d=8, S=4)
    o, _ = orc.joint_attention(q, k, v, kd, vd, 4, True)
    sep = orc.separate_then_add(q, k, v, kd, vd, 4, True)
    assert np.max(np.abs(o - sep)) > 1e-2


# p6 -----------------------------------------------------------------------------
def pin_locality_and_causality(orc):
    """Row t sees keys j <= t and only its own depth slots: changing later keys or
    other tokens' depth slots leaves row t bit-identical."""
    q, k, v, kd, vd = rand_case(10, B=1, T=8, Hq=2, Hkv=2, d=4, S=2)
    o, lse = orc.joint_attention(q, k, v, kd, vd, 2, True, 0.7)
    t = 4
    k2, v2, kd2, vd2 = k.copy(), v.copy(), kd.copy(), vd.copy()
    k2[:, t + 1 :] += 5.0
    v2[:, t + 1 :] -= 3.0
    kd2[:, np.arange(8) != t] *= -2.0
    vd2[:, np.arange(8) != t] += 1.0
    o2, lse2 = orc.joint_attention(q, k2, v2, kd2, vd2, 2, True, 0.7)
    assert np.array_equal(o[:, t], o2[:, t]) and np.array_equal(lse[:, :, t], lse2[:, :, t])
    assert not np.allclose(o[:, t + 1], o2[:, t + 1])
    # and slots beyond n_depth are never read
    kd3, vd3 = kd.copy(), vd.copy()
    q2, k3, v3, kd4, vd4 = rand_case(10, B=1, T=8, Hq=2, Hkv=2, d=4, S=2, Scap=4)
    o4, _ = orc.joint_attention(q2, k3, v3, kd4, vd4, 2, True, 0.7)
    kd4[:, :, 2:] = 1e3
    vd4[:, :, 2:] = -1e3
    o5, _ = orc.joint_attention(q2, k3, v3, kd4, vd4, 2, True, 0.7)
    assert np.array_equal(o4, o5)
    del kd3, vd3


# p7 -----------------------------------------------------------------------------
def pin_slot_permutation(orc):
    """The depth slots form a set: a joint permutation of the slot axis of
    (k_depth, v_depth) leaves the output unchanged."""
    q, k, v, kd, vd = rand_case(11, B=1, T=6, Hq=2, Hkv=1, d=5, S=5)
    o, lse = orc.joint_attention(q, k, v, kd, vd, 5, True)
    p = np.array([3, 0, 4, 1, 2])
    o2, lse2 = orc.joint_attention(q, k, v, kd[:, :, p], vd[:, :, p], 5, True)
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12


# p8 -----------------------------------------------------------------------------
def pin_gqa_is_repeated_mha(orc):
    """Query head h reads KV head h // G: identical to MHA with every sequence and
    depth KV head repeated G times in place."""
    q, k, v, kd, vd = rand_case(12, B=2, T=7, Hq=6, Hkv=2, d=4, S=3)
    o, lse = orc.joint_attention(q, k, v, kd, vd, 3, True)
    G = 3
    o2, lse2 = orc.joint_attention(
        q, np.repeat(k, G, 2), np.repeat(v, G, 2), np.repeat(kd, G, 3), np.repeat(vd, G, 3), 3, True
    )
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


# p9 -----------------------------------------------------------------------------
def pin_varlen_is_independent(orc):
    """Packed sequences (cu_seqlens) behave as independent runs."""
    rng = np.random.default_rng(13)
    lens = [5, 1, 9, 3]
    N, Hq, Hkv, d, S = sum(lens), 4, 2, 6, 3
    q = rng.standard_normal((N, Hq, d))
    k = rng.standard_normal((N, Hkv, d))
    v = rng.standard_normal((N, Hkv, d))
    kd = rng.standard_normal((N, S, Hkv, d))
    vd = rng.standard_normal((N, S, Hkv, d))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, lse = orc.joint_attention(q, k, v, kd, vd, S, True, cu_seqlens=cu)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        o1, l1 = orc.joint_attention(q[None, a:b], k[None, a:b], v[None, a:b], kd[None, a:b], vd[None, a:b], S, True)
        assert np.max(np.abs(o[a:b] - o1[0])) < 1e-13
        assert np.max(np.abs(lse[:, a:b] - l1[0])) < 1e-13


# p10 ----------------------------------------------------------------------------
def pin_depth_copies_of_current_kv(orc):
    """If every depth slot of token t holds (k_t, v_t), the joint softmax equals
    causal attention with ln(1 + S) added to the diagonal logit: checked against
    SDPA with that additive mask."""
    q, k, v, _, _ = rand_case(14, B=1, T=9, Hq=2, Hkv=2, d=6, S=1)
    S = 3
    kd = np.repeat(k[:, :, None], S, axis=2)
    vd = np.repeat(v[:, :, None], S, axis=2)
    o, _ = orc.joint_attention(q, k, v, kd, vd, S, True, 0.6)
    T = 9
    mask = np.full((T, T), -np.inf)
    mask[np.tril_indices(T)] = 0.0
    mask[np.diag_indices(T)] = math.log(1 + S)
    ref = _sdpa(q, k, v, False, 0.6, attn_mask=mask)
    assert np.max(np.abs(o - ref)) < 1e-12


# p11 ----------------------------------------------------------------------------
def pin_hand_example(orc):
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    one = lambda x: np.array(x, dtype=np.float64).reshape(1, 1, 1, 1)  # noqa: E731
    kd = np.array(math.log(3.0)).reshape(1, 1, 1, 1, 1)
    vd = np.array(g["v_depth"]).reshape(1, 1, 1, 1, 1)
    o, lse = orc.joint_attention(one(g["q"]), one(g["k"]), one(g["v"]), kd, vd, 1, True, g["scale"])
    assert abs(o.item() - g["out"]) < 1e-15
    assert abs(lse.item() - math.log(4.0)) < 1e-15


# p12 ----------------------------------------------------------------------------
def pin_brute_force(orc):
    """Pure-Python fsum brute force agrees with the vectorised oracle."""
    rng = np.random.default_rng(15)
    for it in range(6):
        T = int(rng.integers(1, 8))
        G = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 3))
        d = int(rng.integers(1, 7))
        S = int(rng.integers(0, 4))
        causal = bool(it % 2 == 0)
        q, k, v, kd, vd = rand_case(100 + it, B=1, T=T, Hq=G * Hkv, Hkv=Hkv, d=d, S=S, Scap=S + 1)
        o, lse = orc.joint_attention(q, k, v, kd, vd, S, causal, 0.8)
        o2, lse2 = orc.scalar_ref(q, k, v, kd, vd, S, causal, 0.8)
        assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12


# p13 ----------------------------------------------------------------------------
def pin_large_logits(orc):
    """Huge logit spread stays finite and tends to the value of the arg-max key."""
    q, k, v, kd, vd = rand_case(16, B=1, T=6, Hq=1, Hkv=1, d=4, S=2)
    o, lse = orc.joint_attention(1e4 * q, k, v, kd, vd, 2, True, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for t in range(6):
        logits = np.concatenate([k[0, : t + 1, 0] @ q[0, t, 0], kd[0, t, :2, 0] @ q[0, t, 0]])
        vals = np.concatenate([v[0, : t + 1, 0], vd[0, t, :2, 0]])
        srt = np.sort(logits)
        if len(srt) > 1 and srt[-1] - srt[-2] < 1e-3:
            continue
        assert np.max(np.abs(o[0, t, 0] - vals[np.argmax(logits)])) < 1e-9


# p14 ----------------------------------------------------------------------------
def pin_index_map_example(orc):
    """G = 4: expanded rows 8-15 see depth entries of positions 2 and 3 only, and the
    sequence keys up to their own position."""
    with open(os.path.join(GOLDEN, "index_map_g4.json")) as f:
        g = json.load(f)
    G, L, T = g["G"], 3, 6
    seen = set()
    for i_q in g["rows"]:
        pos = {j_d // L for j_d in range(T * L) if orc.depth_visible(i_q, j_d, G, L)}
        assert len(pos) == 1
        seen |= pos
        (p,) = pos
        assert [i_k for i_k in range(T) if orc.sequence_visible(i_q, i_k, G)] == list(range(p + 1))
    assert sorted(seen) == g["positions"]


def pin_expanded_rows_equal(orc):
    """The expanded-row formulation with the two visibility predicates computes the
    same operator as the per-head form."""
    for seed, Hq, Hkv, S in [(17, 4, 1, 2), (18, 4, 2, 3), (19, 2, 2, 1)]:
        q, k, v, kd, vd = rand_case(seed, B=1, T=5, Hq=Hq, Hkv=Hkv, d=4, S=S)
        o, _ = orc.joint_attention(q, k, v, kd, vd, S, True, 0.9)
        o2 = orc.expanded_rows_attention(q, k, v, kd, vd, S, 0.9)
        assert np.max(np.abs(o - o2)) < 1e-12


# p15 ----------------------------------------------------------------------------
def pin_utilization(orc):
    """Brute-force counts of usable depth entries reproduce the printed sweep values
    (3.12% at G = 2, 50% at G = 32, C = L = 64) and the 1/T, 1/C, G/C forms."""
    with open(os.path.join(GOLDEN, "depth_utilization.json")) as f:
        g = json.load(f)
    C, L = g["C"], 8  # utilization does not depend on L; a small L keeps the count fast
    for G, pct in g["printed_percent"].items():
        u = orc.depth_utilization("group", T=0, C=C, G=int(G), L=L)
        assert math.floor(100 * u * 100) / 100 == pct or round(100 * u, g["printed_decimals"]) == pct, (G, u)
    assert abs(orc.depth_utilization("chunk", T=0, C=16, G=1, L=3) - 1 / 16) < 1e-15
    assert abs(orc.depth_utilization("contiguous", T=12, C=4, G=1, L=2) - 1 / 12) < 1e-15
    assert abs(orc.depth_utilization("group", T=0, C=16, G=4, L=2) - 4 / 16) < 1e-15


# ---------------------------------------------------------------- decode (one new token per sequence)


def _decode_case(seed, B=3, T=11, Hq=4, Hkv=2, d=8, S=3):
    q, k, v, kd, vd = rand_case(seed, B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, S=S)
    ts = np.array([T - 1, 0, T // 2])[:B]  # the decoded token of each sequence
    b = np.arange(B)
    return q, k, v, kd, vd, ts, q[b, ts], kd[b, ts], vd[b, ts]


def pin_decode_is_last_row(orc):
    """A decode step at position t equals row t of the full causal forward (the
    cache prefix 0..t holds the token's own key)."""
    q, k, v, kd, vd, ts, qt, kdt, vdt = _decode_case(21)
    o_full, l_full = orc.joint_attention(q, k, v, kd, vd, 3, causal=True)
    o, l = orc.decode(qt, k, v, ts + 1, kdt, vdt, 3)
    for b, t in enumerate(ts):
        assert np.abs(o[b] - o_full[b, t]).max() < 1e-12
        assert np.abs(l[b] - l_full[b, :, t]).max() < 1e-12


def pin_decode_empty_depth_is_sdpa(orc):
    """No depth slots: ordinary attention of one query row over the cache prefix
    (torch's scaled_dot_product_attention, float64)."""
    q, k, v, kd, vd, ts, qt, kdt, vdt = _decode_case(22)
    o, _ = orc.decode(qt, k, v, ts + 1, kdt, vdt, 0)
    G = qt.shape[1] // k.shape[2]
    for b, t in enumerate(ts):
        L = int(t) + 1
        qq = torch.from_numpy(qt[b][:, None, :].copy())                       # [Hq, 1, d]
        kk = torch.from_numpy(np.repeat(k[b, :L].transpose(1, 0, 2), G, axis=0).copy())  # [Hq, L, d]
        vv = torch.from_numpy(np.repeat(v[b, :L].transpose(1, 0, 2), G, axis=0).copy())
        ref = F.scaled_dot_product_attention(qq, kk, vv).numpy()[:, 0]
        assert np.abs(o[b] - ref).max() < 1e-12


def pin_decode_single_key(orc):
    """One cached key and no slots: the output is that key's value and lse its
    logit (closed form)."""
    q, k, v, kd, vd, ts, qt, kdt, vdt = _decode_case(23, Hq=2, Hkv=1, d=5)
    o, l = orc.decode(qt, k, v, np.ones(3, dtype=np.int32), kdt, vdt, 0)
    scale = 1.0 / math.sqrt(5)
    for b in range(3):
        for h in range(2):
            assert np.abs(o[b, h] - v[b, 0, 0]).max() < 1e-14
            assert abs(l[b, h] - scale * float(q[b, ts[b], h] @ k[b, 0, 0])) < 1e-12


# backward ----------------------------------------------------------------------
# The pages give the forward only; the backward is its exact derivative. These pins
# tie the oracle's gradients to the forward (finite differences), to identities
# that any derivative of a softmax-weighted average obeys, and to torch's autograd
# of its SDPA routine where the depth set is empty.


def _bwd_cases():
    # (seed, B, T, Hq, Hkv, d, S, Scap, causal, cu_seqlens or None)
    return [
        (11, 2, 5, 4, 2, 4, 2, 3, True, None),
        (12, 1, 6, 2, 2, 4, 3, 3, False, None),
        (13, 1, 7, 2, 1, 4, 1, 2, True, np.array([0, 3, 7])),
        (14, 2, 4, 3, 3, 4, 0, 2, True, None),
    ]


def _bwd_inputs(seed, B, T, Hq, Hkv, d, S, Scap, cu):
    q, k, v, kd, vd = rand_case(seed, B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, S=S, Scap=Scap)
    w = np.random.default_rng(seed + 100).standard_normal(q.shape)
    if cu is not None:  # packed layout: drop the batch axis
        q, k, v, w = (x.reshape((-1,) + x.shape[2:]) for x in (q, k, v, w))
        kd, vd = (x.reshape((-1,) + x.shape[2:]) for x in (kd, vd))
    return [q, k, v, kd, vd], w


def pin_backward_finite_differences(orc):
    """Every gradient element equals the central difference of sum(out * W) under
    the forward oracle (itself pinned above), including zeros for unread slots."""
    for seed, B, T, Hq, Hkv, d, S, Scap, causal, cu in _bwd_cases():
        xs, w = _bwd_inputs(seed, B, T, Hq, Hkv, d, S, Scap, cu)
        scale = 0.61
        grads = orc.joint_attention_backward(*xs[:5], S, w, causal, scale, cu_seqlens=cu)

        def loss(ys):
            o, _ = orc.joint_attention(*ys, S, causal, scale, cu_seqlens=cu)
            return float(np.sum(o * w))

        eps = 1e-6
        for which in range(5):
            g = grads[which]
            for idx in np.ndindex(xs[which].shape):
                up = [x.copy() for x in xs]
                dn = [x.copy() for x in xs]
                up[which][idx] += eps
                dn[which][idx] -= eps
                fd = (loss(up) - loss(dn)) / (2 * eps)
                assert abs(g[idx] - fd) < 1e-6 * (1 + abs(fd)), (seed, which, idx, g[idx], fd)


def pin_backward_sums(orc):
    """Per segment and KV head: the value gradients sum to the summed upstream
    gradient of the head group (each row's weights sum to one), and the key
    gradients sum to zero (a common shift of all keys moves every logit of a row
    by the same amount, which leaves the softmax unchanged)."""
    q, k, v, kd, vd = rand_case(21, B=2, T=13, Hq=4, Hkv=2, d=8, S=4, Scap=5)
    w = np.random.default_rng(22).standard_normal(q.shape)
    for causal in (True, False):
        dq, dk, dv, dkd, dvd = orc.joint_attention_backward(q, k, v, kd, vd, 4, w, causal, 0.4)
        G = 2
        for b in range(2):
            for hk in range(2):
                vsum = dv[b, :, hk].sum(axis=0) + dvd[b, :, :, hk].sum(axis=(0, 1))
                osum = w[b, :, hk * G : (hk + 1) * G].sum(axis=(0, 1))
                assert np.max(np.abs(vsum - osum)) < 1e-10
                ksum = dk[b, :, hk].sum(axis=0) + dkd[b, :, :, hk].sum(axis=(0, 1))
                assert np.max(np.abs(ksum)) < 1e-10
        assert np.all(dkd[:, :, 4:] == 0) and np.all(dvd[:, :, 4:] == 0)


def pin_backward_empty_depth_is_sdpa_autograd(orc):
    """With no depth slots the gradients are those of ordinary softmax attention:
    torch's autograd through its SDPA routine in float64 (grouped heads by repeating
    KV heads, whose gradients then sum over the group)."""
    for seed, (Hq, Hkv), causal in [(31, (2, 2), True), (32, (4, 2), True), (33, (3, 1), False)]:
        q, k, v, kd, vd = rand_case(seed, B=2, T=9, Hq=Hq, Hkv=Hkv, d=8, S=2)
        w = np.random.default_rng(seed).standard_normal(q.shape)
        scale = 0.29
        dq, dk, dv, _, _ = orc.joint_attention_backward(q, k, v, kd, vd, 0, w, causal, scale)
        G = Hq // Hkv
        qt = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)
        kt = torch.tensor(k.transpose(0, 2, 1, 3), requires_grad=True)
        vt = torch.tensor(v.transpose(0, 2, 1, 3), requires_grad=True)
        o = F.scaled_dot_product_attention(qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1),
                                           is_causal=causal, scale=scale)
        (o * torch.from_numpy(np.ascontiguousarray(w.transpose(0, 2, 1, 3)))).sum().backward()
        for mine, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
            ref = ref.numpy().transpose(0, 2, 1, 3)
            assert np.max(np.abs(mine - ref)) < 1e-12, np.max(np.abs(mine - ref))


# p23 ----------------------------------------------------------------------------
def _gather_row(q, k, v, kd, vd, S, cu, s, t, h, G, causal):
    """Operands of row (segment s, token t, head h) of a packed problem, gathered
    the way the sampled GPU checks gather them."""
    a, b = int(cu[s]), int(cu[s + 1])
    hk = h // G
    J = np.arange(a, a + t + 1) if causal else np.arange(a, b)
    n = a + t
    kd_row = kd[n, :S, hk] if S > 0 else None
    vd_row = vd[n, :S, hk] if S > 0 else None
    return q[n, h], k[J, hk], v[J, hk], kd_row, vd_row


def pin_joint_rows(orc):
    """The one-row form used by the full-size sampled checks: (1) equals the
    whole-tensor oracle row by row (causal and not, with and without depth slots,
    grouped heads, packed segments of unequal length); (2) reproduces the hand
    example on its own; (3) stays finite when a depth logit dominates by 10^4
    (the max must run over the depth logits too) and returns that slot's value."""
    rng = np.random.default_rng(23)
    for causal, S, (Hq, Hkv), lens in [(True, 3, (4, 2), (5, 1, 9)), (False, 2, (2, 2), (7, 4)),
                                       (True, 0, (3, 1), (6, 2)), (False, 0, (4, 4), (3,)),
                                       (True, 4, (6, 3), (8,))]:
        N, d, G = sum(lens), 6, Hq // Hkv
        q = rng.standard_normal((N, Hq, d))
        k = rng.standard_normal((N, Hkv, d))
        v = rng.standard_normal((N, Hkv, d))
        kd = rng.standard_normal((N, S + 1, Hkv, d))
        vd = rng.standard_normal((N, S + 1, Hkv, d))
        cu = np.concatenate([[0], np.cumsum(lens)])
        o, lse = orc.joint_attention(q, k, v, kd, vd, S, causal, 0.45, cu_seqlens=cu)
        for s, L in enumerate(lens):
            for t in range(L):
                for h in range(Hq):
                    ro, rl = orc.joint_rows(*_gather_row(q, k, v, kd, vd, S, cu, s, t, h, G, causal), 0.45)
                    n = int(cu[s]) + t
                    assert np.max(np.abs(ro - o[n, h])) < 1e-13, (causal, S, s, t, h)
                    assert abs(rl - lse[h, n]) < 1e-13
    # (2) hand example: weights 1 and 3
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    o, lse = orc.joint_rows(np.array([g["q"]]), np.array([[g["k"]]]), np.array([[g["v"]]]),
                            np.array([[math.log(3.0)]]), np.array([[g["v_depth"]]]), g["scale"])
    assert abs(o.item() - g["out"]) < 1e-15 and abs(lse - math.log(4.0)) < 1e-15
    # (3) a dominant depth logit (1e4 above every sequence logit)
    q_row = np.array([1.0, 0.0])
    ks = np.array([[0.0, 1.0], [0.5, 2.0]])
    vs = np.array([[1.0, 2.0], [3.0, 4.0]])
    kdr = np.array([[1e4, 0.0], [-1.0, 0.0]])
    vdr = np.array([[-7.0, 5.0], [9.0, 9.0]])
    o, lse = orc.joint_rows(q_row, ks, vs, kdr, vdr, 1.0)
    assert np.all(np.isfinite(o)) and np.isfinite(lse)
    assert np.max(np.abs(o - vdr[0])) < 1e-12 and abs(lse - 1e4) < 1e-9


# p24 ----------------------------------------------------------------------------
def _ln(x):
    return math.log(float(x.split()[1])) if isinstance(x, str) else float(x)


def pin_topk_hand_examples(orc):
    """Bounded slot reads (top-S, sliding window, hybrid) worked by hand, including
    the tie rule (tests/golden/topk_example.json)."""
    with open(os.path.join(GOLDEN, "topk_example.json")) as f:
        g = json.load(f)
    one = lambda x: np.array(x, dtype=np.float64).reshape(1, 1, 1, 1)  # noqa: E731
    for c in g["cases"]:
        kd = np.array([_ln(x) for x in c["k_depth"]]).reshape(1, 1, 3, 1, 1)
        vd = np.array(c["v_depth"]).reshape(1, 1, 3, 1, 1)
        o, lse = orc.joint_attention(one(g["q"]), one(g["k"]), one(g["v"]), kd, vd, 3, True, g["scale"],
                                     depth_topk=c["topk"], depth_recent=c["recent"])
        assert abs(o.item() - c["out"]) < 1e-12, c
        assert abs(lse.item() - _ln(c["lse"])) < 1e-12, c
        keep = orc.select_slots(np.array([[_ln(x) for x in c["k_depth"]]]), c["topk"], c["recent"])
        assert list(np.flatnonzero(keep[0])) == c["chosen"], c


# p25 ----------------------------------------------------------------------------
def pin_topk_limits(orc):
    """topk covering every slot is the joint operator (bitwise); no slot at all is
    ordinary causal attention (SDPA); topk = 0 with recent = w equals the operator
    over the window of the last w slots."""
    q, k, v, kd, vd = rand_case(24, B=2, T=9, Hq=4, Hkv=2, d=6, S=5)
    o, lse = orc.joint_attention(q, k, v, kd, vd, 5, True, 0.5)
    for topk, recent in [(5, 0), (9, 0), (0, 5), (3, 2), (2, 7)]:
        o2, lse2 = orc.joint_attention(q, k, v, kd, vd, 5, True, 0.5, depth_topk=topk, depth_recent=recent)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2), (topk, recent)
    o0, _ = orc.joint_attention(q, k, v, kd, vd, 5, True, 0.5, depth_topk=0)
    assert np.max(np.abs(o0 - _sdpa(q, k, v, True, 0.5))) < 1e-12
    ow, lw = orc.joint_attention(q, k, v, kd, vd, 5, True, 0.5, depth_topk=0, depth_recent=2)
    ow2, lw2 = orc.joint_attention(q, k, v, kd[:, :, 3:5], vd[:, :, 3:5], 2, True, 0.5)
    assert np.max(np.abs(ow - ow2)) < 1e-13 and np.max(np.abs(lw - lw2)) < 1e-13


# p26 ----------------------------------------------------------------------------
def pin_topk_brute_force(orc):
    """Pure-Python selection (sort by logit, then index) and fsum agree with the
    vectorised oracle on random tiny shapes, grouped heads, causal or not."""
    rng = np.random.default_rng(26)
    for it in range(8):
        T = int(rng.integers(1, 7))
        G = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 3))
        d = int(rng.integers(1, 6))
        S = int(rng.integers(3, 7))
        recent = int(rng.integers(0, S - 1))  # at least two older slots
        topk = int(rng.integers(1, S - recent))  # a proper subset of them
        causal = bool(it % 2 == 0)
        q, k, v, kd, vd = rand_case(200 + it, B=1, T=T, Hq=G * Hkv, Hkv=Hkv, d=d, S=S, Scap=S + 1)
        o, lse = orc.joint_attention(q, k, v, kd, vd, S, causal, 0.7, depth_topk=topk, depth_recent=recent)
        o2, lse2 = orc.scalar_ref(q, k, v, kd, vd, S, causal, 0.7, depth_topk=topk, depth_recent=recent)
        assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12, (it, topk, recent)


# p27 ----------------------------------------------------------------------------
def pin_projection_hand_example(orc):
    """FFN-input KV projection into one slot, worked by hand
    (tests/golden/projection_example.json)."""
    with open(os.path.join(GOLDEN, "projection_example.json")) as f:
        g = json.load(f)
    x = np.array(g["x"], dtype=np.float64)
    w = np.array(g["w_kv"], dtype=np.float64)
    kd = np.full((1, g["S_cap"], 1, 2), -1.0)
    vd = np.full((1, g["S_cap"], 1, 2), -2.0)
    kd2, vd2 = orc.depth_kv_projection(x, w, kd, vd, g["slot"], 1, 2)
    assert np.array_equal(kd2[0, g["slot"], 0], g["k"]) and np.array_equal(vd2[0, g["slot"], 0], g["v"])
    others = [i for i in range(g["S_cap"]) if i != g["slot"]]
    assert np.all(kd2[0, others] == -1.0) and np.all(vd2[0, others] == -2.0)


# p28 ----------------------------------------------------------------------------
def pin_projection_is_linear_then_slot(orc):
    """Equals torch's linear layer (fp64) followed by placing the rows in the slot;
    other slots are bit-identical; linear in the input."""
    rng = np.random.default_rng(28)
    N, D, Hkv, d, S = 7, 12, 2, 4, 3
    x = rng.standard_normal((N, D))
    w = rng.standard_normal((2 * Hkv * d, D))
    kd = rng.standard_normal((N, S, Hkv, d))
    vd = rng.standard_normal((N, S, Hkv, d))
    kd2, vd2 = orc.depth_kv_projection(x, w, kd, vd, 1, Hkv, d)
    ref = F.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    assert np.max(np.abs(kd2[:, 1].reshape(N, -1) - ref[:, : Hkv * d])) < 1e-12
    assert np.max(np.abs(vd2[:, 1].reshape(N, -1) - ref[:, Hkv * d :])) < 1e-12
    assert np.array_equal(kd2[:, [0, 2]], kd[:, [0, 2]]) and np.array_equal(vd2[:, [0, 2]], vd[:, [0, 2]])
    x2 = rng.standard_normal((N, D))
    ka, va = orc.depth_kv_projection(x, w, kd, vd, 2, Hkv, d)
    kb, vb = orc.depth_kv_projection(x2, w, kd, vd, 2, Hkv, d)
    kc, vc = orc.depth_kv_projection(2.0 * x - 3.0 * x2, w, kd, vd, 2, Hkv, d)
    assert np.max(np.abs(kc[:, 2] - (2.0 * ka[:, 2] - 3.0 * kb[:, 2]))) < 1e-11
    assert np.max(np.abs(vc[:, 2] - (2.0 * va[:, 2] - 3.0 * vb[:, 2]))) < 1e-11


ALL_PINS = [
    pin_empty_depth_is_sdpa,
    pin_equal_logits_plain_mean,
    pin_convex_and_affine,
    pin_lse_merge,
    pin_separate_softmax_differs,
    pin_locality_and_causality,
    pin_slot_permutation,
    pin_gqa_is_repeated_mha,
    pin_varlen_is_independent,
    pin_depth_copies_of_current_kv,
    pin_hand_example,
    pin_brute_force,
    pin_large_logits,
    pin_index_map_example,
    pin_expanded_rows_equal,
    pin_utilization,
    pin_decode_is_last_row,
    pin_decode_empty_depth_is_sdpa,
    pin_decode_single_key,
    pin_backward_finite_differences,
    pin_backward_sums,
    pin_backward_empty_depth_is_sdpa_autograd,
    pin_joint_rows,
    pin_topk_hand_examples,
    pin_topk_limits,
    pin_topk_brute_force,
    pin_projection_hand_example,
    pin_projection_is_linear_then_slot,
]
