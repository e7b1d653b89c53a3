"""Planted mistakes in the oracle must be caught by its pins.

Each case edits one line of the oracle's C source (a dropped term, a wrong
sign, a transposed operand, a wrong bound, scale or stride), compiles that
mutant into a temporary library on the CPU, swaps it in, and checks that at
least one pin in test_oracle_pins fails.  The real oracle is never touched.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("decay dropped", "dec[i] = exp((double)clamp_gate(fetch(g, rb + i, in_bf16)));", "dec[i] = 1.0;"),
    ("lower clamp -4", "#define ORACLE_GATE_LO (-5.0f)", "#define ORACLE_GATE_LO (-4.0f)"),
    ("upper clamp missing", "if (x > ORACLE_GATE_HI) x = ORACLE_GATE_HI;", ""),
    ("delta sign", "((double)fetch(v, rb + j, in_bf16) - u[j])", "((double)fetch(v, rb + j, in_bf16) + u[j])"),
    ("beta dropped", "e[j] = b * (", "e[j] = ("),
    ("u transposed", "for (int j = 0; j < d; ++j) u[j] += ki * Sp[(long)i * d + j];",
     "for (int j = 0; j < d; ++j) u[j] += ki * Sp[(long)j * d + i];"),
    ("update transposed", "Sp[(long)i * d + j] += ki * e[j];", "Sp[(long)j * d + i] += ki * e[j];"),
    ("o from pre-update state", "u[j] += qi * Sp[(long)i * d + j];", "u[j] += qi * (double)S[(long)i * d + j];"),
    ("o scale 1/d", "1.0 / sqrt((double)d)", "1.0 / (double)d"),
    ("row stride", "r.row_stride = (long)cs->H * d;", "r.row_stride = d;"),
    ("beta stride", "fetch(beta, (long)t * beta_stride, in_bf16)", "fetch(beta, (long)t, in_bf16)"),
    ("bf16 widen shift", "((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    ("o row stride", "o[(long)t * o_stride + j]", "o[(long)t * d + j]"),
    ("argmax ties to highest index", "if (x > bv) {", "if (x >= bv) {"),
    ("NaN row not flagged", "if (x != x) nan = 1;", ""),
    ("accept stops one draft early", "while (j < t - 1 && drafts[j] == vam[j]) ++j;",
     "while (j < t - 2 && drafts[j] == vam[j]) ++j;"),
    ("accept compares the next row", "drafts[j] == vam[j]) ++j;", "drafts[j] == vam[j + 1]) ++j;"),
    ("bonus from the last accepted row", "out2[1] = vam[j];", "out2[1] = vam[j > 0 ? j - 1 : 0];"),
    ("ring never shifts", "for (int m = 0; m + 1 < ORACLE_RING_ROWS; ++m)",
     "for (int m = 0; m + 1 < 0; ++m)"),
    ("ring appends the previous raw row", "fetch(raw, (l * T_round + r) * C + c, in_bf16)",
     "fetch(raw, (l * T_round + (r > 0 ? r - 1 : 0)) * C + c, in_bf16)"),
    ("ring ignores the layer", "fetch(raw, (l * T_round + r) * C + c, in_bf16)",
     "fetch(raw, (long)r * C + c, in_bf16)"),
    ("conv without SiLU", "y[c] = silu(acc);", "y[c] = acc;"),
    ("conv taps reversed", "(double)wl[c * ORACLE_CONV_TAPS + m] * ring[m * C + c]",
     "(double)wl[c * ORACLE_CONV_TAPS + (ORACLE_RING_ROWS - m)] * ring[m * C + c]"),
    ("conv ring not rolled", "for (long c = 0; c < C; ++c) ring[m * C + c] = ring[(m + 1) * C + c];",
     ""),
    ("norm without epsilon", "1.0 / sqrt(sq + ORACLE_NORM_EPS)", "1.0 / sqrt(sq)"),
    ("norm epsilon 1e-8", "#define ORACLE_NORM_EPS 1e-6", "#define ORACLE_NORM_EPS 1e-8"),
    ("norm epsilon 1e-7", "#define ORACLE_NORM_EPS 1e-6", "#define ORACLE_NORM_EPS 1e-7"),
    ("norm epsilon 1e-5", "#define ORACLE_NORM_EPS 1e-6", "#define ORACLE_NORM_EPS 1e-5"),
    ("q and k blocks swapped", "q[o + j] = (float)(y[h * d + j] * nq);",
     "q[o + j] = (float)(y[HD + h * d + j] * nq);"),
    ("gate bound missing", "if (gg < ORACLE_GATE_LO) gg = ORACLE_GATE_LO;", ""),
    ("gate sign", "double gg = -softplus(", "double gg = softplus("),
    ("beta without sigmoid", "(float)(1.0 / (1.0 + exp(-(double)fetch(b, (l * T + t) * H + h, in_bf16))));",
     "(float)fetch(b, (l * T + t) * H + h, in_bf16);"),
]

PIN_TESTS = [
    lambda: pins.test_identity_beta0_g0_leaves_state_and_reads_it(),
    lambda: pins.test_decay_closed_form(),
    lambda: pins.test_clamp_bounds_are_exactly_minus5_and_0(),
    lambda: pins.test_one_hot_key_writes_value_into_that_key_row(),
    lambda: pins.test_associative_memory_with_orthonormal_keys(),
    lambda: [pins.test_exact_rational_d4(s) for s in range(3)],
    lambda: [pins.test_matrix_form_with_decay(*a) for a in [(4, 6, 0), (8, 9, 2)]],
    lambda: pins.test_chains_are_independent_and_layout_strides_are_right(),
    lambda: pins.test_bf16_widening_matches_ieee_table(),
    lambda: pins.test_accept_argmax_matches_numpy_first_occurrence(),
    lambda: pins.test_accept_tie_break_and_special_values(),
    lambda: [pins.test_accept_prefix_walk(m) for m in (0, 3, 7)],
    lambda: [pins.test_reroll_is_the_last_three_rows_of_snapshot_then_kept_rows(k)
             for k in (1, 2, 4)],
    lambda: pins.test_reroll_composes_and_keeps_layers_apart(),
    lambda: pins.test_row_ops_identity_taps_give_silu_closed_forms(),
    lambda: pins.test_row_ops_taps_reach_back_through_the_ring(),
    lambda: pins.test_row_ops_norms_gate_and_beta_closed_forms(),
    lambda: pins.test_row_ops_norm_epsilon_dominates_small_rows(),
    lambda: pins.test_row_ops_split_rounds_chain_through_the_ring(),
    lambda: pins.test_row_ops_channels_heads_and_layers_stay_apart(),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for '{name}' not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    str(c), "-o", str(so), "-lm", "-lpthread"], check=True)
    return str(so)


def _swap_in(path):
    lib = ctypes.CDLL(path)
    real = oracle.load()
    for fn in ("kda_oracle_scan_rows", "kda_oracle_batched", "kda_oracle_version",
               "kda_oracle_max_threads", "kda_oracle_accept_greedy", "kda_oracle_conv_reroll",
               "kda_oracle_row_ops"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    return lib


def test_unmutated_oracle_passes_every_pin():
    for pin in PIN_TESTS:
        pin()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, monkeypatch, name, old, new):
    lib = _swap_in(_build_mutant(tmp_path, name, old, new))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for pin in PIN_TESTS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin catches the mutant '{name}'"
