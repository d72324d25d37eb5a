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
