"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake into a temporary copy of oracle/kda_ref.c (on the CPU,
built with gcc into a temp directory), swaps it in for the real library and runs a
small set of the pins from the other test_oracle_* files.  Every mutant must fail at
least one pin.  The committed oracle is never modified.
"""
import contextlib
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gated_delta_rule_86_amd import workloads as W
from oracle.chunked import kda_fwd_chunked
from oracle.exact import core_exact

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "kda_ref.c")).read()

DECAY = ("        /* step 4: decay along the key channels */\n"
         "        for (int64_t i = 0; i < V; ++i)\n"
         "            for (int64_t c = 0; c < K; ++c)\n"
         "                S[i * K + c] *= al[c];\n")
READ = "        /* step 7: read-out with the updated state */\n"

MUTANTS = {
    "decay_wrong_index": [("S[i * K + c] *= al[c];", "S[i * K + c] *= al[i];")],
    "residual_sign": [("double r = vt[i] - pred;", "double r = vt[i] + pred;")],
    "beta_dropped": [("S[i * K + c] += bt * r * kt[c];", "S[i * K + c] += r * kt[c];")],
    "readout_transposed": [("acc += S[i * K + c] * qt[c];", "acc += S[c * K + i] * qt[c];")],
    "scale_dropped": [("out[t * V + i] = scale * acc;", "out[t * V + i] = acc;")],
    "gate_bias_sign": [("oracle_sigmoid(exp(A_log) * (g + dt_bias));", "oracle_sigmoid(exp(A_log) * (g - dt_bias));")],
    "l2norm_no_sqrt": [("1.0 / sqrt(ss + eps)", "1.0 / (ss + eps)")],
    "decay_after_update": [(DECAY, ""), (READ, DECAY + READ)],
    "state_load_transposed": [("s = (double)((const float *)initial_state)[sbase + e];",
                               "s = (double)((const float *)initial_state)[sbase + (e % D) * D + e / D];")],
    "beta_sigmoid_sign": [("? oracle_sigmoid(braw) : braw", "? oracle_sigmoid(-braw) : braw")],
    "dt_bias_head_ignored": [("(double)dt_bias[h * D + c]", "(double)dt_bias[c]")],
    "gate_exp_of_A_log_dropped": [("oracle_sigmoid(exp(A_log) * (g + dt_bias));", "oracle_sigmoid(A_log * (g + dt_bias));")],
    "preactivated_gate_not_held_to_range": [("    return a > 0.0 ? 0.0 : a;", "    return g;")],
    "gate_switch_ignored": [("double a = (flags & ORACLE_GATE_IN_KERNEL)", "double a = 1")],
    "l2norm_switch_ignored": [("            if (flags & ORACLE_QK_L2NORM_IN_KERNEL)\n"
                               "                oracle_l2norm(tmp, D, ORACLE_EPS, kn);\n"
                               "            else\n"
                               "                memcpy(kn, tmp, sizeof(double) * D);",
                               "            oracle_l2norm(tmp, D, ORACLE_EPS, kn);")],
    "beta_switch_ignored": [("(flags & ORACLE_BETA_SIGMOID_IN_KERNEL) ? oracle_sigmoid(braw) : braw",
                             "oracle_sigmoid(braw)")],
}


@contextlib.contextmanager
def mutant_oracle(name):
    src = SRC
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, (name, old)
        src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        c, so = os.path.join(d, "m.c"), os.path.join(d, "libm.so")
        open(c, "w").write(src)
        bwd = os.path.join(os.path.dirname(oracle.__file__), "kda_bwd_ref.c")  # unchanged
        subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-o", so, c, bwd, "-lm"],
                       check=True)
        saved_lib, saved_path = oracle._lib, oracle._LIB_PATH
        oracle._lib, oracle._LIB_PATH = None, so
        try:
            yield
        finally:
            oracle._lib, oracle._LIB_PATH = saved_lib, saved_path


def pin_exact_core():
    from test_oracle_exact import as_np, rand_case
    for seed in range(3):
        alpha, beta, kn, qn, v, scale, S0 = rand_case(77 + seed, 3, 4)
        ox, sx = core_exact(alpha, beta, kn, qn, v, scale, S0)
        o, s = oracle.core(as_np(alpha), np.array([float(b) for b in beta]), as_np(kn), as_np(qn),
                           as_np(v), float(scale), as_np(S0))
        if np.abs(o - as_np(ox)).max() > 1e-12 or np.abs(s - as_np(sx)).max() > 1e-12:
            return False
    return True


def pin_chunk_independence():
    w = W.make("m", 1, 33, 2, seed=5, state_dtype="fp32")
    ro, rf = oracle.kda_fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound,
                            w.initial_state)
    co, cf = kda_fwd_chunked(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound,
                             w.initial_state, C=16)
    return np.abs(co - ro).max() <= 1e-12 * np.abs(co).max() and np.abs(cf - rf).max() <= 1e-12 * np.abs(cf).max()


def pin_gate_values():
    import math
    lb, A_log, dt = -2.0, math.log(3.0), 0.25
    return oracle.gate(-dt, A_log, dt, lb) == lb / 2 and oracle.gate(1e6, A_log, dt, lb) == lb


def pin_wiring():
    from test_oracle_dense import test_full_entry_wiring_vs_dense
    try:
        test_full_entry_wiring_vs_dense(False)
        test_full_entry_wiring_vs_dense(True)
    except AssertionError:
        return False
    return True


def pin_l2norm():
    x = np.random.default_rng(1).standard_normal(128)
    return abs(np.linalg.norm(oracle.l2norm(x)) - np.sqrt(x @ x / (x @ x + 1e-6))) <= 1e-15


def pin_switches():
    from test_oracle_flags import (test_all_switches_off_matches_exact_rational,
                                   test_preactivated_gate_pure_decay_closed_form)
    try:
        test_all_switches_off_matches_exact_rational(1)
        test_preactivated_gate_pure_decay_closed_form(0)
    except AssertionError:
        return False
    return True


PINS = [pin_exact_core, pin_chunk_independence, pin_gate_values, pin_wiring, pin_l2norm, pin_switches]


def test_pins_pass_on_the_real_oracle():
    assert all(p() for p in PINS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with mutant_oracle(name):
        results = {p.__name__: p() for p in PINS}
    assert not all(results.values()), f"mutant {name} passed every pin: {results}"
