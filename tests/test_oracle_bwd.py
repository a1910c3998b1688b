"""Pins of the backward oracle (oracle/kda_bwd_ref.c), CPU only.

The pages print no backward pass; the oracle is the reverse-mode derivative of the token
recurrence (see the header of kda_bwd_ref.c).  It is pinned to things other than itself:
  * the core derivative (already-activated inputs) against exact forward-mode derivatives
    in rational arithmetic: dual numbers over fractions.Fraction pushed through the core
    recurrence (oracle.exact.core_exact_jvp), for random rational directions, with the
    loss L = sum W_o * out + sum W_s * S_T;
  * the full derivative (gate, l2norm, sigmoid, all three switches) against central finite
    differences of a double-precision forward assembled from the forward oracle's own
    exported pieces (oracle.gate, oracle.sigmoid, oracle.l2norm, oracle.core), one
    direction per gradient output;
  * the forward values it recomputes against the forward oracle;
  * a closed form: with beta = 0 the keys and values get no gradient and
    dq^_t = scale S_0 Diag(exp(sum_{j<=t} a_j)) do_t.
"""
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gated_delta_rule_86_amd import workloads as W
from oracle.chunked import bf16_bits_to_f64
from oracle.exact import core_exact, core_exact_jvp
from test_oracle_exact import as_np, rand_case

D = 128


def _rand_like(rng, x, den=7):
    if isinstance(x, list):
        return [_rand_like(rng, a, den) for a in x]
    return Fraction(rng.randint(-5, 5), den)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("seed", range(4))
def test_core_bwd_matches_exact_derivative(K, seed):
    T = 2 + seed % 4
    alpha, beta, kn, qn, v, scale, S0 = rand_case(5000 * K + seed, K, T)
    rng = random.Random(seed + 17 * K)
    Wo = [[Fraction(rng.randint(-3, 3), 4) for _ in range(K)] for _ in range(T)]
    Ws = [[Fraction(rng.randint(-3, 3), 4) for _ in range(K)] for _ in range(K)]
    tan = {"alpha": _rand_like(rng, alpha), "beta": _rand_like(rng, beta), "kn": _rand_like(rng, kn),
           "qn": _rand_like(rng, qn), "v": _rand_like(rng, v), "S0": _rand_like(rng, S0)}
    out, S = core_exact_jvp(alpha, beta, kn, qn, v, scale, S0, tan)
    exact = sum(Wo[t][i] * out[t][i].b for t in range(T) for i in range(K)) + \
        sum(Ws[i][c] * S[i][c].b for i in range(K) for c in range(K))
    g = oracle.core_bwd(as_np(alpha), np.array([float(b) for b in beta]), as_np(kn), as_np(qn), as_np(v),
                        float(scale), as_np(S0), as_np(Wo), as_np(Ws))
    got = (np.sum(g["dalpha"] * as_np(tan["alpha"])) + np.sum(g["dbeta"] * np.array([float(x) for x in tan["beta"]]))
           + np.sum(g["dkn"] * as_np(tan["kn"])) + np.sum(g["dqn"] * as_np(tan["qn"]))
           + np.sum(g["dv"] * as_np(tan["v"])) + np.sum(g["dS0"] * as_np(tan["S0"])))
    assert abs(got - float(exact)) <= 1e-12 * max(1.0, abs(float(exact))), (got, float(exact))
    # the dual numbers carry the plain recurrence in their .a parts
    ox, sx = core_exact(alpha, beta, kn, qn, v, scale, S0)
    assert all(out[t][i].a == ox[t][i] for t in range(T) for i in range(K))


def test_core_bwd_recomputes_the_forward():
    rng = np.random.default_rng(3)
    T, K, V = 9, 5, 4
    alpha = rng.uniform(0.2, 1.0, (T, K))
    beta = rng.uniform(0, 1, T)
    kn = rng.normal(size=(T, K))
    kn /= np.linalg.norm(kn, axis=1, keepdims=True)
    qn = rng.normal(size=(T, K))
    v = rng.normal(size=(T, V))
    S0 = rng.normal(size=(V, K))
    o, S = oracle.core(alpha, beta, kn, qn, v, 0.7, S0)
    g = oracle.core_bwd(alpha, beta, kn, qn, v, 0.7, S0, np.zeros((T, V)), want_out=True)
    assert np.abs(g["out"] - o).max() <= 1e-14 * np.abs(o).max()
    # no loss, no gradient
    for key in ("dalpha", "dbeta", "dkn", "dqn", "dv", "dS0"):
        assert not np.any(g[key])


# ---- full derivative against finite differences of a double-precision forward ----

def _forward_f64(x, flags, lb, scale):
    """Loss of the forward pass on double inputs, assembled from the forward oracle's exported
    pieces (activations per token, then the core recurrence).  x: dict of float64 arrays
    q, k, v, g, b [T, 128] / [T], A_log (scalar), dt [128], S0 [128, 128], Wo [T, 128], Ws."""
    T = x["q"].shape[0]
    qn = np.array([oracle.l2norm(x["q"][t]) if flags & 2 else x["q"][t] for t in range(T)])
    kn = np.array([oracle.l2norm(x["k"][t]) if flags & 2 else x["k"][t] for t in range(T)])
    if flags & 1:
        a = np.array([[oracle.gate(x["g"][t, c], x["A_log"], x["dt"][c], lb) for c in range(D)] for t in range(T)])
    else:
        a = np.array([[oracle.gate_preactivated(x["g"][t, c], lb) for c in range(D)] for t in range(T)])
    beta = np.array([oracle.sigmoid(x["b"][t]) if flags & 4 else x["b"][t] for t in range(T)])
    out, S = oracle.core(np.exp(a), beta, kn, qn, x["v"], scale, x["S0"])
    return float(np.sum(x["Wo"] * out) + np.sum(x["Ws"] * S))


@pytest.mark.parametrize("flags", [7, 0, 5, 2])
def test_full_bwd_matches_finite_differences(flags):
    T, lb = 6, -2.0
    w = W.make(f"fd{flags}", 1, T, 1, seed=600 + flags, lower_bound=lb, flags=flags, state_dtype="fp32")
    if not flags & 1:
        # pre-activated log-decays: keep them away from the kinks of the [lb, 0] limits, where
        # the derivative jumps and a central difference straddles the jump
        gf = W.bf16_bits_to_f32(w.g).copy()
        gf[(gf < lb + 1e-2) | (gf > -1e-2)] = -1.0
        w.g = W.f32_to_bf16_bits(gf)
    rng = np.random.default_rng(flags)
    dout_f = rng.normal(size=(1, T, 1, D)).astype(np.float32)
    dout = W.f32_to_bf16_bits(dout_f)
    dht = rng.normal(size=(1, 1, D, D)).astype(np.float32)
    gA = w.A_log if flags & 1 else None
    gdt = w.dt_bias if flags & 1 else None
    r = oracle.kda_bwd(w.q, w.k, w.v, w.g, w.beta, w.scale, gA, gdt, lb, dout, w.initial_state, dht,
                       flags=flags)
    x = {"q": bf16_bits_to_f64(w.q[0, :, 0]), "k": bf16_bits_to_f64(w.k[0, :, 0]),
         "v": bf16_bits_to_f64(w.v[0, :, 0]), "g": bf16_bits_to_f64(w.g[0, :, 0]),
         "b": bf16_bits_to_f64(w.beta[0, :, 0]), "A_log": float(w.A_log[0]),
         "dt": w.dt_bias[0].astype(np.float64), "S0": w.initial_state[0, 0].astype(np.float64),
         "Wo": bf16_bits_to_f64(dout[0, :, 0]), "Ws": dht[0, 0].astype(np.float64)}
    grads = {"q": r["dq"][0, :, 0], "k": r["dk"][0, :, 0], "v": r["dv"][0, :, 0], "g": r["dg"][0, :, 0],
             "b": r["dbeta"][0, :, 0], "S0": r["dh0"][0, 0]}
    if flags & 1:
        grads["A_log"] = r["dA_log"][0]
        grads["dt"] = r["ddt_bias"][0]
    else:
        assert not np.any(r["dA_log"]) and not np.any(r["ddt_bias"])
    # keep the pre-activated gate away from the kinks of its range limits
    if not flags & 1:
        assert np.all((x["g"] > lb + 1e-3) & (x["g"] < -1e-3))
    for name, gr in grads.items():
        d = rng.normal(size=np.shape(x[name]))
        eps = 1e-5
        xp = dict(x); xm = dict(x)
        xp[name] = x[name] + eps * d
        xm[name] = x[name] - eps * d
        fd = (_forward_f64(xp, flags, lb, w.scale) - _forward_f64(xm, flags, lb, w.scale)) / (2 * eps)
        an = float(np.sum(gr * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_beta_zero_closed_form():
    """beta = 0: no write, so keys and values get no gradient, and the read-out of the decayed
    initial state gives dq^_t = scale Diag(exp(b_t)) S_0^T do_t, b_t = sum_{j<=t} a_j."""
    T = 7
    w = W.make("b0bwd", 1, T, 2, seed=610, state_dtype="fp32")
    w.beta[:] = W.f32_to_bf16_bits(np.full(w.beta.shape, -1000.0, np.float32))
    rng = np.random.default_rng(5)
    dout = W.f32_to_bf16_bits(rng.normal(size=(1, T, 2, D)).astype(np.float32))
    r = oracle.kda_bwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound, dout,
                       w.initial_state)
    assert not np.any(r["dv"]) and not np.any(r["dk"])
    for h in range(2):
        g = bf16_bits_to_f64(w.g[0, :, h])
        a = np.array([[oracle.gate(g[t, c], w.A_log[h], w.dt_bias[h, c], w.lower_bound) for c in range(D)]
                      for t in range(T)])
        bcum = np.cumsum(a, axis=0)
        S0 = w.initial_state[0, h].astype(np.float64)
        do = bf16_bits_to_f64(dout[0, :, h])
        q = bf16_bits_to_f64(w.q[0, :, h])
        for t in range(T):
            dqn = w.scale * np.exp(bcum[t]) * (S0.T @ do[t])
            qn = q[t] / np.sqrt(q[t] @ q[t] + 1e-6)
            dq = (dqn - qn * (qn @ dqn)) / np.sqrt(q[t] @ q[t] + 1e-6)
            assert np.abs(r["dq"][0, t, h] - dq).max() <= 1e-12 * max(1.0, np.abs(dq).max())
