"""Independent NumPy fp64 chunked form of the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

This is a second, independent derivation of what ``kda_ref.c`` computes token by
token: the sequence of every (sequence, head) chain is cut into chunks of ``C``
tokens (any C >= 1; the last chunk of a sequence may be shorter) and each chunk is
processed with intra-chunk matrices and a carried state.  The FlashKDA article
index page ("Delta Attention Algorithm ... processes 16-token chunks") names the
16-token chunking and ("Neumann-series expansion ... matrix inversion") the
inverse; the chunk algebra below follows from the token recurrence:

  within a chunk with inclusive per-channel cumulative log-decay b_r = sum_{j<=r} a_j,
    E[r,s,c] = exp(b[r,c] - b[s,c])
    A_kk[r,s] = beta_r * sum_c k^_rc k^_sc E[r,s,c]        (s < r)
    Tm        = (I + A_kk)^-1
    W = Tm diag(beta) (k^ * exp(b)),   U = Tm diag(beta) v
    V' = U - W S^T                                            (corrected values)
    A_qk[r,s] = scale * sum_c q^_rc k^_sc E[r,s,c]          (s <= r)
    O  = scale (q^ * exp(b)) S^T + A_qk V'
    S <- S diag(exp(b_last)) + V'^T (k^ * exp(b_last - b))

Agreement with the token oracle for every chunk size ("chunk-size independence")
pins this algebra; ``neumann_inverse`` is pinned against a triangular solve.
The activations (l2norm, gate, sigmoid) are re-implemented here from the same
readings as ``kda_ref.c``; the two files share no code.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def bf16_bits_to_f64(a):
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def neumann_inverse(A):
    """(I + A)^-1 for a strictly lower-triangular n x n A by the Neumann product.

    (I + A)^-1 = sum_k (-A)^k = (I - A)(I + A^2)(I + A^4)...(I + A^(2^(m-1))), 2^m >= n,
    exact because A is nilpotent (A^n = 0).
    """
    n = A.shape[0]
    I = np.eye(n)
    T = I - A
    P = A
    span = 2
    while span < n:
        P = P @ P
        T = T @ (I + P)
        span *= 2
    return T


def forward_substitution_inverse(A):
    """(I + A)^-1 for strictly lower-triangular A, column by column (textbook)."""
    n = A.shape[0]
    T = np.zeros((n, n))
    for j in range(n):
        T[j, j] = 1.0
        for i in range(j + 1, n):
            T[i, j] = -np.dot(A[i, j:i], T[j:i, j])
    return T


def _activate(q, k, g, beta, A_log_h, dt_bias_h, lower_bound, flags=7):
    """Activated inputs of one chunk.  flags bit 1: gate from logits (else g is the log-decay,
    held to [lower_bound, 0]); bit 2: l2-normalise q and k (else as given); bit 4: sigmoid of
    the beta logits (else beta as given)."""
    if flags & 2:
        qn = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + EPS)
        kn = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + EPS)
    else:
        qn, kn = q, k
    if flags & 1:
        x = np.exp(A_log_h) * (g + dt_bias_h[None, :])
        a = lower_bound / (1.0 + np.exp(-x))
    else:
        a = np.clip(g, lower_bound, 0.0)
    bt = 1.0 / (1.0 + np.exp(-beta)) if flags & 4 else beta
    return qn, kn, a, bt


def chunk_step(S, qn, kn, v, a, bt, scale, inverse="solve"):
    """One chunk (any length l >= 1).  S: [V, K] state at chunk start.  Returns (O [l, V], S_new)."""
    l = a.shape[0]
    b = np.cumsum(a, axis=0)
    E = np.exp(b[:, None, :] - b[None, :, :])
    G = np.einsum("rc,sc,rsc->rs", kn, kn, E)
    lower_strict = np.tril(np.ones((l, l)), -1)
    lower_incl = np.tril(np.ones((l, l)), 0)
    Akk = bt[:, None] * G * lower_strict
    if inverse == "solve":
        Tm = np.linalg.solve(np.eye(l) + Akk, np.eye(l))
    elif inverse == "neumann":
        Tm = neumann_inverse(Akk)
    else:
        raise ValueError(inverse)
    W = Tm @ (bt[:, None] * kn * np.exp(b))
    U = Tm @ (bt[:, None] * v)
    Vp = U - W @ S.T
    Aqk = scale * np.einsum("rc,sc,rsc->rs", qn, kn, E) * lower_incl
    O = scale * (qn * np.exp(b)) @ S.T + Aqk @ Vp
    S_new = S * np.exp(b[-1])[None, :] + Vp.T @ (kn * np.exp(b[-1][None, :] - b))
    return O, S_new


def kda_fwd_chunked(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state=None,
                    cu_seqlens=None, C=16, inverse="solve", flags=7):
    """Chunked forward pass on host arrays (small sizes only).

    Same argument meaning as ``oracle.kda_fwd`` (``flags``: the activation switches, bit 1
    gate, bit 2 q/k l2norm, bit 4 beta sigmoid); inputs are uint16 bf16 bits, states may be
    uint16 (bf16 bits), float32 or float64.  Returns (out [B, T, H, 128], final [N, H, 128, 128]).
    """
    B, T, H, D = q.shape
    qf, kf, vf, gf = (bf16_bits_to_f64(x) for x in (q, k, v, g))
    bf = bf16_bits_to_f64(beta)
    if flags & 1:
        A_log = np.asarray(A_log, dtype=np.float32).astype(np.float64)
        dt_bias = np.asarray(dt_bias, dtype=np.float32).astype(np.float64)
    else:
        A_log = np.zeros(H)
        dt_bias = np.zeros((H, D))
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(0, int(cu[i]), int(cu[i + 1])) for i in range(cu.size - 1)]
    else:
        seqs = [(b, 0, T) for b in range(B)]
    N = len(seqs)
    if initial_state is None:
        S0 = np.zeros((N, H, D, D))
    elif initial_state.dtype == np.uint16:
        S0 = bf16_bits_to_f64(initial_state)
    else:
        S0 = np.asarray(initial_state).astype(np.float64)
    out = np.zeros((B, T, H, D))
    fin = np.zeros((N, H, D, D))
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = S0[n, h].copy()
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)
                qn, kn, a, bt = _activate(qf[b, c0:c1, h], kf[b, c0:c1, h], gf[b, c0:c1, h],
                                          bf[b, c0:c1, h], A_log[h], dt_bias[h], lower_bound,
                                          flags)
                O, S = chunk_step(S, qn, kn, vf[b, c0:c1, h], a, bt, scale, inverse)
                out[b, c0:c1, h] = O
            fin[n, h] = S
    return out, fin
