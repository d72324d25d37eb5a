"""fp64 CPU oracle of MoDA joint sequence/depth attention (forward).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library and imports nothing from it.

Source: "Mixture-of-Depths Attention" (arXiv 2603.15619), as presented in the MoDA
reading-group deck, slide "One denominator allocates probability across both
memories" (the teaching expansion of Sec. 2.2 / Algorithm 1). For one query head
at layer l and token t, with head dimension d:

    a_j = q_t . k_j / sqrt(d)            causal sequence keys j <= t
    b_i = q_t . k^depth_{i,t} / sqrt(d)  depth slots i of the same token t
    o_t = (sum_j e^{a_j} v_j + sum_i e^{b_i} v^depth_{i,t})
          / (sum_j e^{a_j} + sum_i e^{b_i})

ONE numerator and ONE denominator span both key sets. Separate softmaxes followed
by addition form a different operator (same slide); ``separate_then_add`` exists
only so tests can show that difference.

The slide "Shared online-softmax states preserve the joint operator" computes the
same value block by block with a running max; that is an exact reordering, so this
oracle writes out the closed form instead: per row, the maximum over ALL visible
logits, natural exponentials, one sum, one division. Rows are computed in batches
of whole rows purely to bound memory; each row's max, sum and weighted sum still
run over its complete visible set in one numpy reduction.

Readings where the pages leave a step open (each is listed with its reason in
the design notes):
  * layouts: q/out [B,T,H_q,d]; k,v [B,T,H_kv,d]; depth [B,T,S_cap,H_kv,d];
    packed (varlen) tensors drop B and add cu_seqlens; only slots [0, n_depth)
    are read.
  * grouped heads: query head h reads KV head h // G, G = H_q / H_kv, for both the
    sequence and the depth keys (Table 1 groups the depth cache with G as well).
  * the current token's own key is a sequence key (j = t is visible); the depth
    slots are those already written by earlier layers.
  * scale multiplies both kinds of logit; the workloads use 1/sqrt(d).
  * causal=False makes every key of the segment visible; depth is unchanged.
  * lse = M + ln Z, the natural log of the joint denominator.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _as_packed(q, k, v, kd, vd, cu_seqlens):
    """Return packed [N, ...] views plus cu_seqlens (batch layout -> B equal segments)."""
    if cu_seqlens is None:
        B, T = q.shape[0], q.shape[1]
        q = q.reshape((B * T,) + q.shape[2:])
        k = k.reshape((B * T,) + k.shape[2:])
        v = v.reshape((B * T,) + v.shape[2:])
        if kd is not None:
            kd = kd.reshape((B * T,) + kd.shape[2:])
            vd = vd.reshape((B * T,) + vd.shape[2:])
        cu = np.arange(B + 1, dtype=np.int64) * T
        return q, k, v, kd, vd, cu, (B, T)
    return q, k, v, kd, vd, np.asarray(cu_seqlens, dtype=np.int64), None


def joint_attention(
    q,
    k,
    v,
    k_depth=None,
    v_depth=None,
    n_depth: int = 0,
    causal: bool = True,
    scale: Optional[float] = None,
    cu_seqlens=None,
    row_block: int = 256,
    mode: str = "joint",
    depth_topk: Optional[int] = None,
    depth_recent: int = 0,
):
    """MoDA forward in float64. Returns (out, lse).

    Batch layout: q [B,T,Hq,d], k/v [B,T,Hkv,d], depth [B,T,S_cap,Hkv,d];
    out [B,T,Hq,d], lse [B,Hq,T].
    Packed layout (cu_seqlens given): q [N,Hq,d], k/v [N,Hkv,d], depth
    [N,S_cap,Hkv,d]; out [N,Hq,d], lse [Hq,N].

    ``mode`` selects which keys enter the single softmax: "joint" (the operator),
    "sequence" (depth slots dropped) or "depth" (sequence keys dropped). The last
    two are the partial softmaxes used by the merge identity in the tests.

    ``depth_topk`` (None = every slot): a bounded read of the depth history, the
    top-S / sliding-window / hybrid buffer that the MoDA deck lists as future work
    (slide "The main open cost is retaining and reading depth history", paper Sec.
    6.1-6.2), which the pages name but do not define. Reading taken: of a row's
    slots [0, n_depth), the last ``depth_recent`` always enter; of the others, the
    ``depth_topk`` with the largest depth logits b_i enter, ties going to the lower
    slot index; the remaining slots leave the softmax (as if absent). topk = 0 with
    recent = w is a sliding window of the w most recent slots; recent = 0 is pure
    top-S; both > 0 is the hybrid.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    kd, vd = _f64(k_depth), _f64(v_depth)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    use_seq = mode in ("joint", "sequence")
    use_depth = mode in ("joint", "depth") and n_depth > 0
    if mode == "depth" and n_depth <= 0:
        raise ValueError("depth-only softmax needs n_depth > 0")
    qp, kp, vp, kdp, vdp, cu, batch_shape = _as_packed(q, k, v, kd, vd, cu_seqlens)
    N, Hq, _ = qp.shape
    Hkv = kp.shape[1]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    out = np.zeros_like(qp)
    lse = np.zeros((Hq, N), dtype=np.float64)
    for s in range(len(cu) - 1):
        st, en = int(cu[s]), int(cu[s + 1])
        L = en - st
        if L == 0:
            continue
        for h in range(Hq):
            hk = h // G  # grouped heads: contiguous groups of G query heads
            Q = qp[st:en, h]
            K = kp[st:en, hk]
            V = vp[st:en, hk]
            if use_depth:
                Kd = kdp[st:en, :n_depth, hk]  # [L, S, d]: slots of each token
                Vd = vdp[st:en, :n_depth, hk]
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                rows = np.arange(r0, r1)
                parts_logit, parts_val = [], []
                if use_seq:
                    kend = r1 if causal else L
                    a = scale * (Q[r0:r1] @ K[:kend].T)  # [R, kend]
                    if causal:
                        a = np.where(np.arange(kend)[None, :] <= rows[:, None], a, -np.inf)
                    parts_logit.append(a)
                    parts_val.append(("seq", kend))
                if use_depth:
                    b = scale * np.einsum("rc,rsc->rs", Q[r0:r1], Kd[r0:r1])  # [R, S]
                    if depth_topk is not None:
                        b = np.where(select_slots(b, depth_topk, depth_recent), b, -np.inf)
                    parts_logit.append(b)
                    parts_val.append(("depth", None))
                M = np.max(np.concatenate(parts_logit, axis=1), axis=1)  # finite when j = t is visible
                num = np.zeros((r1 - r0, d))
                Z = np.zeros(r1 - r0)
                for lg, (kind, kend) in zip(parts_logit, parts_val):
                    w = np.exp(lg - M[:, None])
                    Z += w.sum(axis=1)
                    if kind == "seq":
                        num += w @ V[:kend]
                    else:
                        num += np.einsum("rs,rsc->rc", w, Vd[r0:r1])
                out[st + r0 : st + r1, h] = num / Z[:, None]
                lse[h, st + r0 : st + r1] = M + np.log(Z)
    if batch_shape is not None:
        B, T = batch_shape
        out = out.reshape(B, T, Hq, d)
        lse = lse.reshape(Hq, B, T).transpose(1, 0, 2).copy()
    return out, lse


def select_slots(b, topk: int, recent: int = 0):
    """Boolean [R, S] mask of the depth slots that enter each row's softmax (see
    ``joint_attention``): the last ``recent`` slots, plus the ``topk`` largest
    logits among the others, ties to the lower slot index (a stable sort of -b)."""
    b = np.asarray(b, dtype=np.float64)
    R, S = b.shape
    recent = max(0, min(recent, S))
    n_old = S - recent
    keep = np.zeros((R, S), dtype=bool)
    keep[:, n_old:] = True
    k = max(0, min(topk, n_old))
    if k > 0:
        order = np.argsort(-b[:, :n_old], axis=1, kind="stable")  # descending logit, lower index first
        np.put_along_axis(keep[:, :n_old], order[:, :k], True, axis=1)
    return keep


def joint_rows(q_row, k_seq, v_seq, kd_row, vd_row, scale: float):
    """One output row from explicitly gathered operands (for sampled checks).

    q_row [d]; k_seq, v_seq [J, d]: the visible sequence keys/values of the row;
    kd_row, vd_row [S, d] (S may be 0): the row's own depth slots.
    Returns (o [d], lse).
    """
    q_row, k_seq, v_seq = _f64(q_row), _f64(k_seq), _f64(v_seq)
    kd_row = np.zeros((0, q_row.shape[0])) if kd_row is None else _f64(kd_row)
    vd_row = np.zeros((0, q_row.shape[0])) if vd_row is None else _f64(vd_row)
    a = scale * (k_seq @ q_row)
    b = scale * (kd_row @ q_row)
    M = max(a.max(initial=-np.inf), b.max(initial=-np.inf))
    w, u = np.exp(a - M), np.exp(b - M)
    Z = w.sum() + u.sum()
    o = (w @ v_seq + u @ vd_row) / Z
    return o, M + math.log(Z)


def separate_then_add(q, k, v, k_depth, v_depth, n_depth, causal=True, scale=None, cu_seqlens=None):
    """softmax(a) V + softmax(b) V^depth: NOT the MoDA operator (negative check)."""
    o_s, _ = joint_attention(q, k, v, None, None, 0, causal, scale, cu_seqlens, mode="sequence")
    o_d, _ = joint_attention(q, k, v, k_depth, v_depth, n_depth, causal, scale, cu_seqlens, mode="depth")
    return o_s + o_d


def scalar_ref(q, k, v, k_depth, v_depth, n_depth, causal=True, scale=None, depth_topk=None, depth_recent=0):
    """Pure-Python brute force of the joint equation (batch layout, tiny shapes only).

    math.exp and math.fsum over explicit loops; no numpy reductions. Used to check
    the vectorised oracle above. With ``depth_topk`` the slots are chosen by
    sorting (logit descending, slot index ascending) in plain Python.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    kd, vd = _f64(k_depth), _f64(v_depth)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, T, Hq, d))
    lse = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for t in range(T):
                qt = [float(x) for x in q[b, t, h]]
                logits, values = [], []
                for j in range(T):
                    if causal and j > t:
                        continue
                    logits.append(scale * math.fsum(qt[c] * float(k[b, j, hk, c]) for c in range(d)))
                    values.append([float(x) for x in v[b, j, hk]])
                dl = [scale * math.fsum(qt[c] * float(kd[b, t, i, hk, c]) for c in range(d)) for i in range(n_depth)]
                chosen = range(n_depth)
                if depth_topk is not None:
                    old = n_depth - min(depth_recent, n_depth)
                    ranked = sorted(range(old), key=lambda i: (-dl[i], i))
                    chosen = sorted(ranked[: max(0, depth_topk)] + list(range(old, n_depth)))
                for i in chosen:
                    logits.append(dl[i])
                    values.append([float(x) for x in vd[b, t, i, hk]])
                M = max(logits)
                w = [math.exp(x - M) for x in logits]
                Z = math.fsum(w)
                for c in range(d):
                    out[b, t, h, c] = math.fsum(w[n] * values[n][c] for n in range(len(w))) / Z
                lse[b, h, t] = M + math.log(Z)
    return out, lse


# ---------------------------------------------------------------------------------
# Expanded-query formulation (MoDA deck, backup slide "grouped indexing preserves
# the correct token map", paper Algorithm 1 and Sec. 3.3). The G query heads that
# share one KV head are laid out as T_q = G * T_kv expanded rows, row i_q belonging
# to token floor(i_q / G); depth keys are flattened so that entry j_d belongs to
# token floor(j_d / L) with L slots per token.


def sequence_visible(i_q: int, i_k: int, G: int) -> bool:
    return i_q // G >= i_k


def depth_visible(i_q: int, j_d: int, G: int, L: int) -> bool:
    return i_q // G == j_d // L


def expanded_rows_attention(q, k, v, k_depth, v_depth, n_depth, scale=None):
    """Batch layout, causal. Builds the full expanded-row score matrix for every
    (batch, KV head) with the two visibility predicates above and one softmax per
    expanded row over [sequence keys | flattened depth keys]. Tiny shapes only.
    Returns out [B,T,Hq,d] (row i_q = t*G + g maps to head h_kv*G + g)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    L = n_depth
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros_like(q)
    for b in range(B):
        for hk in range(Hkv):
            Qe = q[b, :, hk * G : (hk + 1) * G].reshape(T * G, d)  # i_q = t*G + g
            Kd = np.asarray(k_depth, dtype=np.float64)[b, :, :L, hk].reshape(T * L, d)  # j_d = t*L + i
            Vd = np.asarray(v_depth, dtype=np.float64)[b, :, :L, hk].reshape(T * L, d)
            Kall = np.concatenate([k[b, :, hk], Kd], axis=0)
            Vall = np.concatenate([v[b, :, hk], Vd], axis=0)
            S = scale * (Qe @ Kall.T)
            vis = np.zeros_like(S, dtype=bool)
            for i_q in range(T * G):
                for i_k in range(T):
                    vis[i_q, i_k] = sequence_visible(i_q, i_k, G)
                for j_d in range(T * L):
                    vis[i_q, T + j_d] = depth_visible(i_q, j_d, G, L)
            S = np.where(vis, S, -np.inf)
            M = S.max(axis=1, keepdims=True)
            W = np.exp(S - M)
            Oe = (W @ Vall) / W.sum(axis=1, keepdims=True)
            out[b, :, hk * G : (hk + 1) * G] = Oe.reshape(T, G, d)
    return out


def depth_utilization(layout: str, T: int, C: int, G: int, L: int) -> float:
    """Fraction of scanned depth entries that a query row may use, counted by brute
    force over one block of C expanded query rows (MoDA deck, slide "Local packing
    avoids scanning irrelevant depth entries", Fig. 4 / Sec. 3.2).

    layout "contiguous": every row scans the whole flattened depth axis (T*L);
    "chunk": a block of C rows (one head, C tokens) scans the C*L entries of its
    tokens; "group": a block of C expanded rows (C/G tokens x G heads) scans the
    (C/G)*L entries of its tokens.
    """
    if layout == "contiguous":
        rows = range(C)  # one head: expanded index == token
        span = range(T * L)
        g = 1
    elif layout == "chunk":
        rows = range(C)
        span = range(C * L)
        g = 1
    elif layout == "group":
        rows = range(C)
        span = range((C // G) * L)
        g = G
    else:
        raise ValueError(layout)
    used = sum(1 for i_q in rows for j_d in span if depth_visible(i_q, j_d, g, L))
    return used / (len(rows) * len(span))


def sequence_only(q, k, v, causal=True, scale=None, cu_seqlens=None):
    """Softmax over the sequence keys alone (the partial state of the sequence blocks)."""
    return joint_attention(q, k, v, None, None, 0, causal, scale, cu_seqlens, mode="sequence")


def depth_only(q, k, v, k_depth, v_depth, n_depth, scale=None, cu_seqlens=None):
    """Softmax over the row's own depth slots alone (the partial state of the depth blocks)."""
    return joint_attention(q, k, v, k_depth, v_depth, n_depth, True, scale, cu_seqlens, mode="depth")

def decode(q, k_cache, v_cache, cache_seqlens, k_depth, v_depth, n_depth, scale=None):
    """One new token per sequence (a decode step) in float64. Returns (out, lse).

    The same joint operator as ``joint_attention`` (deck slide "One denominator
    allocates probability across both memories"), for the one query row of each
    sequence: the paper's Table 1, as the deck quotes it, names the decode-time
    sequence cache and depth cache this reads.

    q [B, Hq, d]: the new token's queries. k_cache, v_cache [B, T_max, Hkv, d]:
    sequence b sees keys/values 0 .. cache_seqlens[b] - 1, the last of them being
    the new token's own. k_depth, v_depth [B, S_cap, Hkv, d]: the new token's depth
    slots, of which [0, n_depth) are read. Query head h reads KV head h // G.
    out [B, Hq, d]; lse [B, Hq] = natural log of the joint denominator.

    Per row the closed form: the maximum over every visible logit, natural
    exponentials, one sum, one division.
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Hq, d = q.shape
    Hkv = kc.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kd = _f64(k_depth) if n_depth > 0 else None
    vd = _f64(v_depth) if n_depth > 0 else None
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(cache_seqlens[b])
        for h in range(Hq):
            hk = h // G
            a = scale * (kc[b, :L, hk] @ q[b, h])
            logits = [a]
            if n_depth > 0:
                logits.append(scale * (kd[b, :n_depth, hk] @ q[b, h]))
            M = np.max(np.concatenate(logits))
            w = np.exp(a - M)
            num = w @ vc[b, :L, hk]
            Z = w.sum()
            if n_depth > 0:
                u = np.exp(logits[1] - M)
                num = num + u @ vd[b, :n_depth, hk]
                Z = Z + u.sum()
            out[b, h] = num / Z
            lse[b, h] = M + math.log(Z)
    return out, lse


def joint_attention_backward(
    q,
    k,
    v,
    k_depth,
    v_depth,
    n_depth: int,
    dout,
    causal: bool = True,
    scale: Optional[float] = None,
    cu_seqlens=None,
    row_block: int = 256,
):
    """Gradients of the MoDA forward in float64: returns (dq, dk, dv, dk_depth, dv_depth).

    The pages define the forward only (deck slide "One denominator allocates
    probability across both memories"); the backward here is its exact derivative
    for an upstream gradient ``dout`` of ``out``, written from the chain rule:

        P_j   = e^{a_j - lse}, P_i = e^{b_i - lse}   (one softmax over both key sets)
        dP_x  = <dout_t, value_x>                     x over every visible key
        dS_x  = P_x (dP_x - sum_y P_y dP_y)            (softmax Jacobian, the sum over
                                                        the row's whole visible set)
        dq_t  = scale (sum_j dS_j k_j + sum_i dS_i k^depth_{t,i})
        dk_j  += scale dS_j q_t,  dv_j += P_j dout_t   (over rows t that see key j)
        dk^depth_{t,i} += scale dS_i q_t,  dv^depth_{t,i} += P_i dout_t

    Grouped heads accumulate the gradients of all G query heads into their KV head.
    Layouts as for ``joint_attention``; dk_depth / dv_depth have the full slot axis
    S_cap, with zeros in slots [n_depth, S_cap), which the operator never reads.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    kd, vd = _f64(k_depth), _f64(v_depth)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    use_depth = n_depth > 0
    qp, kp, vp, kdp, vdp, cu, batch_shape = _as_packed(q, k, v, kd, vd, cu_seqlens)
    dop = do.reshape(qp.shape)
    N, Hq, _ = qp.shape
    Hkv = kp.shape[1]
    G = Hq // Hkv
    dq = np.zeros_like(qp)
    dk = np.zeros_like(kp)
    dv = np.zeros_like(vp)
    dkd = None if kdp is None else np.zeros_like(kdp)
    dvd = None if vdp is None else np.zeros_like(vdp)
    for s in range(len(cu) - 1):
        st, en = int(cu[s]), int(cu[s + 1])
        L = en - st
        if L == 0:
            continue
        for h in range(Hq):
            hk = h // G
            Q, dO = qp[st:en, h], dop[st:en, h]
            K, V = kp[st:en, hk], vp[st:en, hk]
            if use_depth:
                KD = kdp[st:en, :n_depth, hk]  # [L, S, d]: each token's own slots
                VD = vdp[st:en, :n_depth, hk]
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                rows = np.arange(r0, r1)
                kend = r1 if causal else L
                a = scale * (Q[r0:r1] @ K[:kend].T)
                if causal:  # key j visible to row t iff j <= t
                    a = np.where(rows[:, None] >= np.arange(kend)[None, :], a, -np.inf)
                logits = [a]
                if use_depth:
                    logits.append(scale * np.sum(Q[r0:r1][:, None, :] * KD[r0:r1], axis=2))
                M = np.max(np.concatenate(logits, axis=1), axis=1)
                Z = sum(np.exp(lg - M[:, None]).sum(axis=1) for lg in logits)
                Pa = np.exp(a - M[:, None]) / Z[:, None]  # [R, kend], zero where masked
                dPa = dO[r0:r1] @ V[:kend].T
                rowdot = np.sum(Pa * dPa, axis=1)
                if use_depth:
                    Pb = np.exp(logits[1] - M[:, None]) / Z[:, None]  # [R, S]
                    dPb = np.sum(dO[r0:r1][:, None, :] * VD[r0:r1], axis=2)
                    rowdot = rowdot + np.sum(Pb * dPb, axis=1)
                dSa = Pa * (dPa - rowdot[:, None])
                dq[st + r0 : st + r1, h] += scale * (dSa @ K[:kend])
                dk[st : st + kend, hk] += scale * (dSa.T @ Q[r0:r1])
                dv[st : st + kend, hk] += Pa.T @ dO[r0:r1]
                if use_depth:
                    dSb = Pb * (dPb - rowdot[:, None])
                    dq[st + r0 : st + r1, h] += scale * np.sum(dSb[:, :, None] * KD[r0:r1], axis=1)
                    dkd[st + r0 : st + r1, :n_depth, hk] += scale * dSb[:, :, None] * Q[r0:r1][:, None, :]
                    dvd[st + r0 : st + r1, :n_depth, hk] += Pb[:, :, None] * dO[r0:r1][:, None, :]
    if batch_shape is not None:
        B, T = batch_shape
        dq = dq.reshape(B, T, Hq, d)
        dk = dk.reshape(B, T, Hkv, d)
        dv = dv.reshape(B, T, Hkv, d)
        if dkd is not None:
            dkd = dkd.reshape((B, T) + dkd.shape[1:])
            dvd = dvd.reshape((B, T) + dvd.shape[1:])
    return dq, dk, dv, dkd, dvd


def depth_kv_projection(x, w_kv, k_depth, v_depth, slot: int, n_heads_kv: int, head_dim: int):
    """The FFN input's KV projection into one depth slot, in float64 (MoDA deck,
    slide "Reuse attention KV; add a projection for FFN inputs", paper Sec. 2.2:
    step 4 projects the FFN input into additional depth KV slots; the default
    variant reuses the attention KV and adds this extra projection).

    x [N, D_model]: the FFN input of N tokens. w_kv [2 * H_kv * d, D_model]: the
    projection weight in the [out, in] layout of a linear layer, the key rows
    first, then the value rows. k_depth, v_depth [N, S_cap, H_kv, d]: the depth
    cache. Returns new copies of (k_depth, v_depth) whose slot ``slot`` holds
    k = x w_k^T and v = x w_v^T of every token, reshaped [H_kv, d]; every other
    slot is unchanged.
    """
    x, w = _f64(x), _f64(w_kv)
    hd = n_heads_kv * head_dim
    if w.shape != (2 * hd, x.shape[1]):
        raise ValueError(f"w_kv must be [2 * H_kv * d, D_model] = {(2 * hd, x.shape[1])}, got {w.shape}")
    kd, vd = np.array(k_depth, dtype=np.float64), np.array(v_depth, dtype=np.float64)
    kv = x @ w.T  # [N, 2 * H_kv * d]
    kd[:, slot] = kv[:, :hd].reshape(-1, n_heads_kv, head_dim)
    vd[:, slot] = kv[:, hd:].reshape(-1, n_heads_kv, head_dim)
    return kd, vd
