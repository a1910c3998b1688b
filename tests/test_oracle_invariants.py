"""Closed forms, invariants and special values that pin the oracle's readings.

Each check follows from the definition stated in oracle/kda_ref.c (FlashKDA README
"Kernel API" table and FLA-backend flags; article index "Delta Attention Algorithm",
"lower_bound parameter", "Sigmoid in its gating path"):
  beta = 0            -> pure per-channel decay (closed form)
  q = k, beta = 1     -> the state retrieves the value just written: out_t = scale v_t
  lower_bound = 0, beta = 1, orthonormal keys -> exact delta-rule overwrite (closed form)
  varlen batch        =  its sequences run separately;  B > 1 = varlen with equal lengths
  split + resume      =  one run
  affine segment map  S_end(S0) = S0 P + F, P the run from S0 = I with v = 0, F from S0 = 0
  linearity           (v, S0) -> (2v, 2S0) doubles out and final state exactly
  gate / sigmoid / l2norm special values and ranges
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from gated_delta_rule_86_amd import workloads as W
from gated_delta_rule_86_amd.workloads import f32_to_bf16_bits
from oracle.chunked import bf16_bits_to_f64

D = 128


def run(w, **kw):
    return oracle.kda_fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound,
                          w.initial_state, cu_seqlens=w.cu_seqlens, **kw)


def test_beta_zero_is_pure_decay():
    w = W.make("b0", 1, 40, 2, seed=21, state_dtype="fp32")
    w.beta[:] = f32_to_bf16_bits(np.full(w.beta.shape, -1000.0, np.float32))  # sigmoid -> 0 exactly
    out, fin = run(w)
    for h in range(w.H):
        g = bf16_bits_to_f64(w.g[0, :, h])
        a = np.array([[oracle.gate(g[t, c], w.A_log[h], w.dt_bias[h, c], w.lower_bound) for c in range(D)]
                      for t in range(w.T)])
        cum = np.exp(np.cumsum(a, axis=0))
        S0 = w.initial_state[0, h].astype(np.float64)
        qn = np.array([oracle.l2norm(bf16_bits_to_f64(w.q[0, t, h])) for t in range(w.T)])
        ref = w.scale * np.einsum("vc,tc,tc->tv", S0, cum, qn)
        assert np.abs(out[0, :, h] - ref).max() <= 1e-14 * max(1, np.abs(ref).max()) + 1e-16
        assert np.abs(fin[0, h] - S0 * cum[-1][None, :]).max() <= 1e-14


def test_q_equals_k_beta_one_retrieves_v():
    w = W.make("qk", 1, 50, 2, seed=22, state_dtype="fp32")
    w.q[:] = w.k
    w.beta[:] = f32_to_bf16_bits(np.full(w.beta.shape, 40.0, np.float32))  # sigmoid -> 1.0 in fp64
    out, _ = run(w)
    v = bf16_bits_to_f64(w.v)
    # S_t k^ = rho v_t + (1 - rho) S'_t k^ with rho = |k^|^2 = 1 - O(1e-6/|k|^2)
    assert np.abs(out - w.scale * v).max() <= 1e-6


def hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_orthonormal_keys_exact_overwrite():
    T = 20
    w = W.make("ortho", 1, T, 1, seed=23, state_dtype="fp32", lower_bound=0.0)
    Hd = hadamard(D)
    rows = np.random.default_rng(0).permutation(D)[:T]
    w.k[0, :, 0] = f32_to_bf16_bits(Hd[rows].astype(np.float32))
    w.beta[:] = f32_to_bf16_bits(np.full(w.beta.shape, 40.0, np.float32))
    out, fin = run(w)
    kn = np.array([oracle.l2norm(bf16_bits_to_f64(w.k[0, t, 0])) for t in range(T)])
    v = bf16_bits_to_f64(w.v[0, :, 0])
    S0 = w.initial_state[0, 0].astype(np.float64)
    ref = S0 @ (np.eye(D) - kn.T @ kn) + v.T @ kn
    assert np.abs(fin[0, 0] - ref).max() <= 1e-12


def test_varlen_equals_separate_runs_bit_exact():
    lens = [7, 0, 16, 33, 1]
    w = W.make("vl", 1, 0, 2, lengths=lens, seed=24, state_dtype="bf16")
    out, fin = run(w)
    cu = w.cu_seqlens
    for n in range(len(lens)):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        sl = lambda a: np.ascontiguousarray(a[:, t0:t1])
        o1, f1 = oracle.kda_fwd(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta), w.scale, w.A_log,
                                w.dt_bias, w.lower_bound, np.ascontiguousarray(w.initial_state[n:n + 1]))
        assert np.array_equal(out[:, t0:t1], o1)
        assert np.array_equal(fin[n:n + 1], f1)


def test_batch_equals_varlen_with_equal_lengths():
    w = W.make("bt", 3, 21, 2, seed=25, state_dtype="fp32")
    out, fin = run(w)
    cu = np.arange(0, 4 * 21, 21, dtype=np.int64)
    r = lambda a: np.ascontiguousarray(a.reshape((1, 3 * 21) + a.shape[2:]))
    o2, f2 = oracle.kda_fwd(r(w.q), r(w.k), r(w.v), r(w.g), r(w.beta), w.scale, w.A_log, w.dt_bias,
                            w.lower_bound, w.initial_state, cu_seqlens=cu)
    assert np.array_equal(out.reshape(o2.shape), o2)
    assert np.array_equal(fin, f2)


@pytest.mark.parametrize("split", [1, 16, 17, 40])
def test_split_and_resume(split):
    w = W.make("res", 1, 57, 2, seed=26, state_dtype="fp32")
    out, fin = run(w)
    sl = lambda a, s: np.ascontiguousarray(a[:, s])
    a0, a1 = slice(0, split), slice(split, None)
    o1, f1 = oracle.kda_fwd(sl(w.q, a0), sl(w.k, a0), sl(w.v, a0), sl(w.g, a0), sl(w.beta, a0), w.scale,
                            w.A_log, w.dt_bias, w.lower_bound, w.initial_state)
    o2, f2 = oracle.kda_fwd(sl(w.q, a1), sl(w.k, a1), sl(w.v, a1), sl(w.g, a1), sl(w.beta, a1), w.scale,
                            w.A_log, w.dt_bias, w.lower_bound, f1)  # fp64 carry
    assert np.array_equal(np.concatenate([o1, o2], axis=1), out)
    assert np.array_equal(f2, fin)


@pytest.mark.parametrize("lb", [0.0, -0.05, -1.0])
def test_segment_map_is_affine(lb):
    """The state after a token range is affine in the state before it: with P the range run
    from the identity with v = 0 and F the range run from zero, S_end(S0) = S0 P + F
    (every token's map S -> S Diag(alpha)(I - beta k k^T) + beta v k^T is affine, and so is
    their composition).  The segmented forward pass stands on this."""
    w = W.make("affine", 2, 37, 2, seed=29, lower_bound=lb, state_dtype="fp32")
    S0 = w.initial_state.astype(np.float64)
    eye = np.broadcast_to(np.eye(D), S0.shape).copy()
    _, S_end = run(w)
    _, F = oracle.kda_fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound,
                          None, want_out=False)
    _, P = oracle.kda_fwd(w.q, w.k, np.zeros_like(w.v), w.g, w.beta, w.scale, w.A_log, w.dt_bias,
                          w.lower_bound, eye, want_out=False)
    pred = np.einsum("bhvc,bhcd->bhvd", S0, P) + F
    assert np.abs(pred - S_end).max() <= 1e-13 * max(1.0, np.abs(S_end).max())
    # and P is not trivial here: the initial state still matters at the end
    assert np.abs(np.einsum("bhvc,bhcd->bhvd", S0, P)).max() > 1e-6


def test_linearity_bit_exact():
    w = W.make("lin", 1, 35, 2, seed=27, state_dtype="fp32")
    out, fin = run(w)
    w2 = W.make("lin", 1, 35, 2, seed=27, state_dtype="fp32")
    w2.v[:] = w.v + np.uint16(0x80)  # bf16 exponent + 1 = times 2 (no zeros/denormals at this size)
    assert np.array_equal(bf16_bits_to_f64(w2.v), 2 * bf16_bits_to_f64(w.v))
    w2.initial_state = 2 * w.initial_state
    out2, fin2 = run(w2)
    assert np.array_equal(out2, 2 * out)
    assert np.array_equal(fin2, 2 * fin)
    # with no initial state the output is linear in v alone
    w3 = W.make("lin", 1, 35, 2, seed=27, state_dtype="none", with_initial=False)
    o3, f3 = run(w3)
    w3.v[:] = w3.v + np.uint16(0x80)
    o4, f4 = run(w3)
    assert np.array_equal(o4, 2 * o3) and np.array_equal(f4, 2 * f3)


def test_gate_special_values():
    A_log, dt = math.log(3.0), 0.25
    for lb in (-5.0, -2.0, -0.5):
        assert oracle.gate(1.7, A_log, dt, 0.0) == 0.0
        assert oracle.gate(-dt, A_log, dt, lb) == lb / 2          # sigmoid(0) = 1/2
        assert oracle.gate(1e6, A_log, dt, lb) == lb               # saturates at the lower bound
        assert oracle.gate(-1e6, A_log, dt, lb) == 0.0             # and at zero
        xs = np.linspace(-4, 4, 101)
        a = np.array([oracle.gate(x, A_log, dt, lb) for x in xs])
        assert np.all(np.diff(a) < 0) and np.all(a < 0) and np.all(a > lb)
        # reading R1: a = lb * expit(exp(A_log) (g + dt_bias)), checked against scipy's expit
        ref = lb * scipy.special.expit(3.0 * (xs + dt))
        assert np.abs(a - ref).max() <= 4 * np.finfo(float).eps * abs(lb)  # a few ulp


def test_sigmoid_and_l2norm():
    assert oracle.sigmoid(0.0) == 0.5
    xs = np.linspace(-30, 30, 241)
    s = np.array([oracle.sigmoid(x) for x in xs])
    assert np.abs(s - scipy.special.expit(xs)).max() <= 1e-16
    assert np.abs(s + s[::-1] - 1.0).max() <= 2 * np.finfo(float).eps
    rng = np.random.default_rng(1)
    x = rng.standard_normal(D)
    y = oracle.l2norm(x)
    assert abs(np.linalg.norm(y) - math.sqrt(x @ x / (x @ x + 1e-6))) <= 1e-15
    assert np.abs(oracle.l2norm(4.0 * x) - x / math.sqrt(x @ x + 1e-6 / 16)).max() <= 1e-15
    assert np.array_equal(oracle.l2norm(np.zeros(D)), np.zeros(D))
