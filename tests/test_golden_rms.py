"""The stored whole-output RMS values (tests/golden/output_rms.json, written by
tests/golden/make_output_rms.py from the oracle alone) still belong to the
current input generator and oracle: their fingerprint rows, recomputed here with
the one-row oracle from regenerated operands, match. The full-size GPU checks
take their bf16 bound (2e-2 x RMS of the whole output) from these values."""
import json
import os

import numpy as np
import pytest

import parity_util

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "output_rms.json")


def _stored():
    with open(GOLDEN) as f:
        return {k: v for k, v in json.load(f).items() if not k.startswith("_")}


def _workload(name):
    from workloads import configs

    if name in configs.WORKLOADS:
        return configs.WORKLOADS[name]
    return parity_util.schedule_workload(name)


def test_every_sampled_workload_has_an_rms():
    from workloads import configs

    stored = _stored()
    need = [n for n in configs.ORDER if configs.WORKLOADS[n].bf16]
    need += [c for c, spec in parity_util.SCHEDULE_CASES.items() if not spec.get("whole")]
    missing = [n for n in need if n not in stored]
    assert not missing, f"run tests/golden/make_output_rms.py {' '.join(missing)}"
    for n in need:
        w = _workload(n)
        assert stored[n]["elements"] == w.n_tokens * w.n_heads_q * w.head_dim
        assert 0.0 < stored[n]["rms"] < 1.0


@pytest.mark.parametrize("name", sorted(_stored()))
def test_fingerprint_rows_match(name):
    w = _workload(name)
    for row in _stored()[name]["rows"]:
        o, lse = parity_util.oracle_row(w, row["segment"], row["t"], row["head"])
        assert np.max(np.abs(o[:8] - np.array(row["out_head8"]))) < 1e-12, (name, row)
        assert abs(lse - row["lse"]) < 1e-12
