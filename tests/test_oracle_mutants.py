"""Mutation check of the pins: plausible mistakes planted in a copy of the
oracle's C source (never in the oracle itself) must each break a pin.

Every mutant keeps all memory accesses in bounds (it only changes which
in-bounds element or which arithmetic is used)."""
import os
import shutil

import pytest

import attnres_pins
import frontend_pins
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
    # absolute snapshot positions
    ("abs_ignores_start", "const int64_t s0 = J->start ? J->start[b] : 0;",
     "const int64_t s0 = 0;"),
    ("abs_base_relative",
     "kda_oracle_snapshot_count(1, cu_seqlens + b, start_pos ? start_pos + b : NULL,",
     "kda_oracle_snapshot_count(1, cu_seqlens + b, NULL,"),
    # Attention Residuals aggregation
    ("ar_no_scale", "l[m] = scale * acc;", "l[m] = acc;"),
    ("ar_unnormalised", "        l[m] /= z;", "        l[m] /= 1.0;"),
    ("ar_no_residual", "double acc = x ? (double)x[(size_t)t * d + c] : 0.0;",
     "double acc = 0.0;"),
    ("ar_rms_of_sum", "r = 1.0 / sqrt(ms / d + eps);", "r = 1.0 / sqrt(ms + eps);"),
    ("ar_eps_outside", "r = 1.0 / sqrt(ms / d + eps);", "r = 1.0 / (sqrt(ms / d) + eps);"),
    ("ar_no_gamma", "(gamma ? (double)gamma[c] : 1.0)", "1.0"),
    ("ar_logits_of_first", "const float *s = src + ((size_t)m * T + t) * d;",
     "const float *s = src + ((size_t)0 * T + t) * d;"),
    # q/k front end (short convolution -> Swish -> L2 norm)
    ("fe_taps_reversed", "z += (double)w[ch * W + j] *",
     "z += (double)w[ch * W + (W - 1 - j)] *"),
    ("fe_head_ignored", "z += (double)w[ch * W + j] *", "z += (double)w[(size_t)i * W + j] *"),
    ("fe_no_swish", "a[i] = z / (1.0 + exp(-z));", "a[i] = z;"),
    ("fe_sigmoid_only", "a[i] = z / (1.0 + exp(-z));", "a[i] = 1.0 / (1.0 + exp(-z));"),
    ("fe_eps_outside_root", "a[i] / sqrt(n2 + eps);", "a[i] / (sqrt(n2) + eps);"),
    ("fe_squared_norm", "a[i] / sqrt(n2 + eps);", "a[i] / (n2 + eps);"),
    ("fe_crosses_sequences", "if (u >= start)", "if (u >= 0)"),
    ("fe_history_reversed", "(size_t)((A->W - 1) + (u - start))) * A->C + ch];",
     "(size_t)(-1 - (u - start))) * A->C + ch];"),
    ("fe_state_rows_reversed", "tail[(size_t)r * A.C + ch] = (float)frontend_input(",
     "tail[(size_t)(W - 2 - r) * A.C + ch] = (float)frontend_input("),
]


def _run_pins(O):
    broken = []
    for pin in (oracle_pins.ALL_PINS + frontend_pins.ALL_FRONTEND_PINS +
                attnres_pins.ALL_ATTNRES_PINS):
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
