"""Mutation check of the pins: plausible mistakes planted in a copy of the
oracle's C source (never in the oracle itself) must each break a pin.

Every mutant keeps all memory accesses in bounds (it only changes which
in-bounds element or which arithmetic is used)."""
import os
import shutil

import pytest

import oracle
import oracle_pins

# (name, exact text in kda_oracle.c, replacement)
MUTANTS = [
    ("no_beta", "u[j] = beta_t * ((double)vt[j] - ks);",
     "u[j] = ((double)vt[j] - ks);"),
    ("sign_flip", "u[j] = beta_t * ((double)vt[j] - ks);",
     "u[j] = beta_t * ((double)vt[j] + ks);"),
    ("no_decay", "double alpha = exp((double)gt[i]);", "double alpha = 1.0;"),
    ("inverted_gate", "double alpha = exp((double)gt[i]);",
     "double alpha = exp(-(double)gt[i]);"),
    ("decayed_write_key", "double ki = (double)kt[i];",
     "double ki = (double)kt[i] * exp((double)gt[i]);"),
    ("wrong_column_read", "ks += (double)kt[i] * S[(size_t)i * dv + j];",
     "ks += (double)kt[i] * S[(size_t)i * dv + (dv - 1 - j)];"),
    ("output_uses_key", "acc += (double)qt[i] * S[(size_t)i * dv + j];",
     "acc += (double)kt[i] * S[(size_t)i * dv + j];"),
    ("no_scale", "o[j] = scale * acc;", "o[j] = acc;"),
    ("snapshot_wrong_head",
     "((size_t)(J->snap_base[b] + jsnap) * H + h) * ssz;",
     "((size_t)(J->snap_base[b] + jsnap) * H + (H - 1 - h)) * ssz;"),
    ("decode_wrong_slot",
     "S = J->state + ((size_t)(J->slots ? J->slots[n] : n) * H + h) * ssz;",
     "S = J->state + ((size_t)n * H + h) * ssz;"),
]


def _run_pins(O):
    broken = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            broken.append(pin.__name__)
    return broken


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mutated = tmp_path / "kda_oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(str(mutated), str(tmp_path / f"libmut_{name}.so"))
    broken = _run_pins(oracle.Oracle(lib))
    assert broken, f"mutant {name} passed every pin"
