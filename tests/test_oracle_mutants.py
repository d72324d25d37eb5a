"""Plant plausible mistakes in copies of the oracle (CPU only) and check that at
least one pin catches each of them."""
import os
import types

import numpy as np
import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moda_oracle.py")

MUTANTS = {
    "diagonal_key_dropped": ("<= rows[:, None]", "< rows[:, None]"),
    "depth_left_out_of_denominator": ("Z += w.sum(axis=1)", "Z += w.sum(axis=1) if kind == 'seq' else 0.0"),
    "wrong_group_map": ("hk = h // G  # grouped", "hk = h % Hkv  # grouped"),
    "depth_of_previous_token": (
        'np.einsum("rc,rsc->rs", Q[r0:r1], Kd[r0:r1])',
        'np.einsum("rc,rsc->rs", Q[r0:r1], np.roll(Kd, 1, axis=0)[r0:r1])',
    ),
    "depth_logit_unscaled": ('b = scale * np.einsum(', 'b = np.einsum('),
    "keys_used_as_values": ("num += w @ V[:kend]", "num += w @ K[:kend]"),
    "depth_keys_used_as_values": ("Vd = vdp[st:en, :n_depth, hk]", "Vd = kdp[st:en, :n_depth, hk]"),
    "exponent_sign": ("w = np.exp(lg - M[:, None])", "w = np.exp(M[:, None] - lg)"),
    "lse_base_two": ("M + np.log(Z)", "M + np.log2(Z)"),
    "slot_off_by_one": ("Kd = kdp[st:en, :n_depth, hk]", "Kd = kdp[st:en, 1 : n_depth + 1, hk]"),
    "keys_of_first_segment": ("K = kp[st:en, hk]", "K = kp[0 : en - st, hk]"),
    "max_over_sequence_only": (
        "M = np.max(np.concatenate(parts_logit, axis=1), axis=1)",
        "M = np.max(parts_logit[0], axis=1)",
    ),
    "depth_value_of_other_head": ("Vd = vdp[st:en, :n_depth, hk]", "Vd = vdp[st:en, :n_depth, (hk + 1) % Hkv]"),
    "decode_prefix_off_by_one": ("L = int(cache_seqlens[b])", "L = int(cache_seqlens[b]) - 1"),
    "decode_group_map": ("hk = h // G\n            a = scale", "hk = h % Hkv\n            a = scale"),
    "decode_depth_logit_unscaled": ("logits.append(scale * (kd[b", "logits.append((kd[b"),
    "decode_depth_keys_as_values": ("num = num + u @ vd[b, :n_depth, hk]", "num = num + u @ kd[b, :n_depth, hk]"),
    "bwd_rowdot_without_depth": ("rowdot = rowdot + np.sum(Pb * dPb, axis=1)", "rowdot = rowdot + 0.0"),
    "bwd_dq_without_depth": ("dq[st + r0 : st + r1, h] += scale * np.sum(dSb", "dq[st + r0 : st + r1, h] += 0.0 * np.sum(dSb"),
    "bwd_dk_unscaled": ("dk[st : st + kend, hk] += scale * (dSa.T", "dk[st : st + kend, hk] += (dSa.T"),
    "bwd_dvd_from_dS": ("dvd[st + r0 : st + r1, :n_depth, hk] += Pb[", "dvd[st + r0 : st + r1, :n_depth, hk] += dSb["),
    "bwd_jacobian_sign": ("dSa = Pa * (dPa - rowdot[:, None])", "dSa = Pa * (dPa + rowdot[:, None])"),
    "bwd_group_map": ("hk = h // G\n            Q, dO", "hk = h % Hkv\n            Q, dO"),
    "bwd_dkd_of_previous_token": ("scale * dSb[:, :, None] * Q[r0:r1][:, None, :]",
                                  "scale * dSb[:, :, None] * np.roll(Q, 1, axis=0)[r0:r1][:, None, :]"),
    "bwd_dv_from_dS": ("dv[st : st + kend, hk] += Pa.T @ dO[r0:r1]", "dv[st : st + kend, hk] += dSa.T @ dO[r0:r1]"),
    "bwd_diagonal_dropped": ("rows[:, None] >= np.arange(kend)", "rows[:, None] > np.arange(kend)"),
    "bwd_depth_values_as_keys": ("VD = vdp[st:en, :n_depth, hk]", "VD = kdp[st:en, :n_depth, hk]"),
    "rows_depth_logit_unscaled": ("b = scale * (kd_row @ q_row)", "b = kd_row @ q_row"),
    "rows_depth_out_of_max": ("M = max(a.max(initial=-np.inf), b.max(initial=-np.inf))",
                              "M = a.max(initial=-np.inf)"),
    "rows_depth_out_of_denominator": ("Z = w.sum() + u.sum()", "Z = w.sum()"),
    "rows_lse_base_two": ("return o, M + math.log(Z)", "return o, M + math.log2(Z)"),
    "rows_depth_keys_as_values": ("u @ vd_row", "u @ kd_row"),
    "topk_ties_to_higher_index": ('order = np.argsort(-b[:, :n_old], axis=1, kind="stable")',
                                  'order = np.argsort(b[:, :n_old], axis=1, kind="stable")[:, ::-1]'),
    "topk_smallest_logits": ('order = np.argsort(-b[:, :n_old], axis=1, kind="stable")',
                             'order = np.argsort(b[:, :n_old], axis=1, kind="stable")'),
    "topk_by_magnitude": ('order = np.argsort(-b[:, :n_old], axis=1, kind="stable")',
                          'order = np.argsort(-np.abs(b[:, :n_old]), axis=1, kind="stable")'),
    "topk_recent_off_by_one": ("keep[:, n_old:] = True", "keep[:, n_old + 1 :] = True"),
    "topk_one_too_many": ("k = max(0, min(topk, n_old))", "k = max(0, min(topk + 1, n_old))"),
    "projection_key_value_swapped": ("kd[:, slot] = kv[:, :hd]", "kd[:, slot] = kv[:, hd:]"),
    "projection_weight_read_as_in_out": ("kv = x @ w.T", "kv = x @ w.reshape(w.shape[1], -1)"),
    "projection_wrong_slot": ("vd[:, slot] = kv[:, hd:]", "vd[:, (slot + 1) % vd.shape[1]] = kv[:, hd:]"),
}


def load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = load_mutant(*MUTANTS[name])
    caught = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(mod)
            except Exception:  # an AssertionError, or a crash such as NaN indexing
                caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
