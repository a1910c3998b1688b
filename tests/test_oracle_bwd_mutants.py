"""The backward oracle's pins must catch plausible mistakes in it.

Each case plants one mistake into a temporary copy of oracle/kda_bwd_ref.c (built with gcc,
together with the unchanged kda_ref.c, into a temp directory), swaps it in for the real
library and runs a few of the pins of test_oracle_bwd.py.  Every mutant must fail one.
"""
import contextlib
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_bwd as P

HERE = os.path.dirname(oracle.__file__)
SRC = open(os.path.join(HERE, "kda_bwd_ref.c")).read()

MUTANTS = {
    "dv_beta_dropped": ("dv[t * V + i] = bt * acc;", "dv[t * V + i] = acc;"),
    "dk_sign": ("dkn[t * K + c] = bt * (a1 - a2);", "dkn[t * K + c] = bt * (a1 + a2);"),
    "carry_decay_dropped": ("D[i * K + c] = dsp * al[c];", "D[i * K + c] = dsp;"),
    "dalpha_wrong_state": ("acc += Sprev[i * K + c] * dsp;", "acc += Sp[i * K + c] * dsp;"),
    "readout_scale_dropped": ("D[i * K + c] += scale * dot[i] * qt[c];", "D[i * K + c] += dot[i] * qt[c];"),
    "dq_before_write": ("acc += S[i * K + c] * dot[i];", "acc += Sp[i * K + c] * dot[i];"),
    "l2norm_projection_dropped": ("(dqn[s * D + c] - qn[s * D + c] * pq) / nq[s]", "dqn[s * D + c] / nq[s]"),
    "gate_sigmoid_derivative": ("da * lower_bound * sg * (1.0 - sg);", "da * lower_bound * sg;"),
    "dA_log_chain": ("pA[chain] += dx * x;", "pA[chain] += dx;"),
    "beta_sigmoid_derivative": ("dbt[s] * bt[s] * (1.0 - bt[s])", "dbt[s] * bt[s]"),
    "dbeta_sign": ("db += acc * r[i];", "db -= acc * r[i];"),
}


@contextlib.contextmanager
def mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, name
    with tempfile.TemporaryDirectory() as d:
        c, so = os.path.join(d, "kda_bwd_ref.c"), os.path.join(d, "libm.so")
        open(c, "w").write(SRC.replace(old, new))
        subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-o", so,
                        os.path.join(HERE, "kda_ref.c"), c, "-lm"], check=True)
        saved_lib, saved_path = oracle._lib, oracle._LIB_PATH
        oracle._lib, oracle._LIB_PATH = None, so
        try:
            yield
        finally:
            oracle._lib, oracle._LIB_PATH = saved_lib, saved_path


def pins():
    for K, seed in ((3, 0), (4, 2)):
        P.test_core_bwd_matches_exact_derivative(K, seed)
    P.test_full_bwd_matches_finite_differences(7)
    P.test_full_bwd_matches_finite_differences(0)
    P.test_beta_zero_closed_form()


def test_pins_pass_on_the_real_oracle():
    pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with mutant(name):
        with pytest.raises(AssertionError):
            pins()
