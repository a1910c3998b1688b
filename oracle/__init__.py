"""fp64 CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
under ``gated_delta_rule_86_amd/`` and never imports it.

Contents
  kda_ref.c   plain C token-by-token fp64 recurrence (the oracle proper)
  kda_bwd_ref.c  its reverse-mode derivative (gradients of out and final state), fp64
  chunked.py  independent NumPy fp64 chunked form (any chunk size) + Neumann inverse
  exact.py    exact-rational (fractions.Fraction) brute force of the core recurrence

The definition each file follows, and the readings taken where the pages are
silent, are stated in the header of ``kda_ref.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_ref.c")
_SRCS = [_SRC, os.path.join(_HERE, "kda_bwd_ref.c")]
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")

STATE_NONE, STATE_BF16, STATE_FP32, STATE_FP64 = 0, 1, 2, 3
# activation switches (bit mask): gate, q/k l2norm and beta sigmoid computed in the pass
GATE_IN_KERNEL, QK_L2NORM_IN_KERNEL, BETA_SIGMOID_IN_KERNEL = 1, 2, 4
ALL_IN_KERNEL = 7

_lib = None


def build(force: bool = False) -> str:
    """Compile kda_ref.c and kda_bwd_ref.c into libkda_oracle.so with gcc (strict IEEE, OpenMP)."""
    stale = not os.path.exists(_LIB_PATH) or any(os.path.getmtime(_LIB_PATH) < os.path.getmtime(f) for f in _SRCS)
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-std=c11", "-o", tmp, *_SRCS, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_sigmoid.restype = ctypes.c_double
        L.oracle_sigmoid.argtypes = [ctypes.c_double]
        L.oracle_gate.restype = ctypes.c_double
        L.oracle_gate.argtypes = [ctypes.c_double] * 4
        L.oracle_gate_preactivated.restype = ctypes.c_double
        L.oracle_gate_preactivated.argtypes = [ctypes.c_double] * 2
        L.oracle_l2norm.restype = None
        L.oracle_l2norm.argtypes = [dp, i64, ctypes.c_double, dp]
        L.oracle_core.restype = ctypes.c_int
        L.oracle_core.argtypes = [i64, i64, i64, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp]
        L.oracle_kda_fwd.restype = ctypes.c_int
        L.oracle_kda_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.c_double, vp, vp, ctypes.c_double,
                                     ctypes.c_int, vp, ctypes.c_int, vp, i64, i64, i64, i64, vp, i64, vp, vp,
                                     ctypes.c_int]
        L.oracle_kda_fwd_compare.restype = ctypes.c_int
        L.oracle_kda_fwd_compare.argtypes = [vp, vp, vp, vp, vp, ctypes.c_double, vp, vp, ctypes.c_double,
                                             ctypes.c_int, vp, ctypes.c_int, vp, i64, i64, i64, i64, vp, i64,
                                             vp, vp, vp, ctypes.c_int]
        L.oracle_core_bwd.restype = ctypes.c_int
        L.oracle_core_bwd.argtypes = [i64, i64, i64, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp, vp,
                                      dp, dp, dp, dp, dp, dp, vp]
        L.oracle_kda_bwd.restype = ctypes.c_int
        L.oracle_kda_bwd.argtypes = [vp, vp, vp, vp, vp, ctypes.c_double, vp, vp, ctypes.c_double,
                                     ctypes.c_int, vp, ctypes.c_int, vp, i64, i64, i64, i64, vp, vp,
                                     vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def sigmoid(x: float) -> float:
    return lib().oracle_sigmoid(float(x))


def gate(g: float, A_log: float, dt_bias: float, lower_bound: float) -> float:
    """Per-channel log-decay a (natural log) for one token and channel."""
    return lib().oracle_gate(float(g), float(A_log), float(dt_bias), float(lower_bound))


def gate_preactivated(g: float, lower_bound: float) -> float:
    """Log-decay taken from a pre-activated gate (gate switch off): g held to [lb, 0]."""
    return lib().oracle_gate_preactivated(float(g), float(lower_bound))


def l2norm(x, eps: float = 1e-6):
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib().oracle_l2norm(_dptr(x), x.size, float(eps), _dptr(y))
    return y


def core(alpha, beta, kn, qn, v, scale, S0):
    """Steps 4-7 of the recurrence on already-activated inputs (any K, V).

    alpha, kn, qn: [T, K]; beta: [T]; v: [T, V]; S0: [V, K].  Returns (out [T, V], S [V, K]).
    """
    alpha = np.ascontiguousarray(alpha, dtype=np.float64)
    kn = np.ascontiguousarray(kn, dtype=np.float64)
    qn = np.ascontiguousarray(qn, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    T, K = alpha.shape
    V = v.shape[1]
    S = np.array(S0, dtype=np.float64, order="C", copy=True)
    out = np.zeros((T, V), dtype=np.float64)
    rc = lib().oracle_core(T, K, V, _dptr(alpha), _dptr(beta), _dptr(kn), _dptr(qn), _dptr(v),
                           float(scale), _dptr(S), _dptr(out))
    if rc != 0:
        raise ValueError(f"oracle_core failed ({rc})")
    return out, S


def kda_fwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state=None,
            state_dtype=None, cu_seqlens=None, heads=None, want_out=True, want_final=True,
            nthreads=0, flags=ALL_IN_KERNEL):
    """Oracle forward pass on host arrays.

    q, k, v, g: uint16 bf16 bit arrays [B, T, H, 128]; beta: uint16 [B, T, H];
    A_log: float32 [H]; dt_bias: float32 [H, 128] (None allowed with the gate switch off);
    flags: activation switches (GATE_IN_KERNEL | QK_L2NORM_IN_KERNEL | BETA_SIGMOID_IN_KERNEL);
      a switch that is off means that input arrives already activated (see kda_ref.c);
    initial_state: None, or [N, H, 128, 128] uint16 (bf16 bits) / float32 / float64;
    cu_seqlens: None or int64 [N+1] (then B must be 1).
    heads: None (all) or a list of head indices; outputs cover only those heads.
    Returns (out float64 [B, T, n_sel, 128] or None, final float64 [N, n_sel, 128, 128] or None).
    """
    B, T, H, D = q.shape
    assert D == 128
    for a in (q, k, v, g):
        assert a.dtype == np.uint16 and a.shape == (B, T, H, D) and a.flags.c_contiguous
    assert beta.dtype == np.uint16 and beta.shape == (B, T, H) and beta.flags.c_contiguous
    if A_log is not None:
        A_log = np.ascontiguousarray(A_log, dtype=np.float32)
    if dt_bias is not None:
        dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
    if cu_seqlens is not None:
        cu_seqlens = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = cu_seqlens.size - 1
    else:
        N = B
    sd = STATE_NONE
    if initial_state is not None:
        initial_state = np.ascontiguousarray(initial_state)
        assert initial_state.shape == (N, H, D, D)
        sd = {np.dtype(np.uint16): STATE_BF16, np.dtype(np.float32): STATE_FP32,
              np.dtype(np.float64): STATE_FP64}[initial_state.dtype]
    if heads is None:
        hsel = None
        n_sel = H
    else:
        hsel = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        n_sel = hsel.size
    out = np.empty((B, T, n_sel, D), dtype=np.float64) if want_out else None
    fin = np.empty((N, n_sel, D, D), dtype=np.float64) if want_final else None
    rc = lib().oracle_kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                              _ptr(A_log), _ptr(dt_bias), float(lower_bound), int(flags),
                              _ptr(initial_state),
                              sd, _ptr(cu_seqlens), B, T, H, N, _ptr(hsel),
                              n_sel, _ptr(out), _ptr(fin), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_kda_fwd rejected its arguments ({rc})")
    return out, fin


def kda_fwd_compare(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, out_cmp, initial_state=None,
                    cu_seqlens=None, heads=None, want_final=True, nthreads=0, flags=ALL_IN_KERNEL):
    """The oracle forward pass compared token by token with another output, without storing
    the fp64 output (bounded memory for very long sequences).

    Inputs as ``kda_fwd``; out_cmp: uint16 bf16 bits [B, T, H, 128] (every head, whatever
    ``heads`` selects).  Returns (stats float64 [N, n_sel, 3] = max|err|, sum err^2,
    sum ref^2 per chain, final float64 [N, n_sel, 128, 128] or None).
    """
    B, T, H, D = q.shape
    assert out_cmp.dtype == np.uint16 and out_cmp.shape == (B, T, H, D) and out_cmp.flags.c_contiguous
    for a in (q, k, v, g):
        assert a.dtype == np.uint16 and a.shape == (B, T, H, D) and a.flags.c_contiguous
    assert beta.dtype == np.uint16 and beta.shape == (B, T, H) and beta.flags.c_contiguous
    if A_log is not None:
        A_log = np.ascontiguousarray(A_log, dtype=np.float32)
    if dt_bias is not None:
        dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
    N = B
    if cu_seqlens is not None:
        cu_seqlens = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = cu_seqlens.size - 1
    sd = STATE_NONE
    if initial_state is not None:
        initial_state = np.ascontiguousarray(initial_state)
        assert initial_state.shape == (N, H, D, D)
        sd = {np.dtype(np.uint16): STATE_BF16, np.dtype(np.float32): STATE_FP32,
              np.dtype(np.float64): STATE_FP64}[initial_state.dtype]
    hsel = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    n_sel = H if hsel is None else hsel.size
    stats = np.zeros((N, n_sel, 3), dtype=np.float64)
    fin = np.empty((N, n_sel, D, D), dtype=np.float64) if want_final else None
    rc = lib().oracle_kda_fwd_compare(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                      _ptr(A_log), _ptr(dt_bias), float(lower_bound), int(flags),
                                      _ptr(initial_state), sd, _ptr(cu_seqlens), B, T, H, N, _ptr(hsel),
                                      n_sel, _ptr(out_cmp), _ptr(stats), _ptr(fin), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_kda_fwd_compare rejected its arguments ({rc})")
    return stats, fin


def core_bwd(alpha, beta, kn, qn, v, scale, S0, dout, dST=None, want_out=False):
    """Reverse mode of steps 4-7 on already-activated inputs (any K, V).

    alpha, kn, qn: [T, K]; beta: [T]; v, dout: [T, V]; S0, dST: [V, K].  Returns a dict
    of float64 arrays: dalpha, dkn, dqn [T, K]; dbeta [T]; dv [T, V]; dS0 [V, K]
    (and out [T, V], the recomputed read-out, when want_out).
    """
    c = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    alpha, beta, kn, qn, v, S0, dout = map(c, (alpha, beta, kn, qn, v, S0, dout))
    T, K = alpha.shape
    V = v.shape[1]
    dST = None if dST is None else c(dST)
    r = {"dalpha": np.zeros((T, K)), "dkn": np.zeros((T, K)), "dqn": np.zeros((T, K)),
         "dbeta": np.zeros(T), "dv": np.zeros((T, V)), "dS0": np.zeros((V, K))}
    out = np.zeros((T, V)) if want_out else None
    rc = lib().oracle_core_bwd(T, K, V, _dptr(alpha), _dptr(beta), _dptr(kn), _dptr(qn), _dptr(v),
                               float(scale), _dptr(S0), _dptr(dout), _ptr(dST), _dptr(r["dalpha"]),
                               _dptr(r["dbeta"]), _dptr(r["dkn"]), _dptr(r["dqn"]), _dptr(r["dv"]),
                               _dptr(r["dS0"]), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_core_bwd failed ({rc})")
    if want_out:
        r["out"] = out
    return r


def kda_bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, dout, initial_state=None,
            dht=None, cu_seqlens=None, nthreads=0, flags=ALL_IN_KERNEL):
    """Gradients of the oracle forward pass (kda_bwd_ref.c) on host arrays.

    Inputs as ``kda_fwd``; dout: uint16 bf16 bits [B, T, H, 128] (dL/dout); dht: None or
    float32 [N, H, 128, 128] (dL/dfinal_state).  Returns a dict of float64 arrays:
    dq, dk, dv, dg [B, T, H, 128]; dbeta [B, T, H]; dA_log [H]; ddt_bias [H, 128];
    dh0 [N, H, 128, 128].
    """
    B, T, H, D = q.shape
    for a in (q, k, v, g, dout):
        assert a.dtype == np.uint16 and a.shape == (B, T, H, D) and a.flags.c_contiguous
    assert beta.dtype == np.uint16 and beta.shape == (B, T, H) and beta.flags.c_contiguous
    if A_log is not None:
        A_log = np.ascontiguousarray(A_log, dtype=np.float32)
    if dt_bias is not None:
        dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
    N = B
    if cu_seqlens is not None:
        cu_seqlens = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = cu_seqlens.size - 1
    sd = STATE_NONE
    if initial_state is not None:
        initial_state = np.ascontiguousarray(initial_state)
        sd = {np.dtype(np.uint16): STATE_BF16, np.dtype(np.float32): STATE_FP32,
              np.dtype(np.float64): STATE_FP64}[initial_state.dtype]
    if dht is not None:
        dht = np.ascontiguousarray(dht, dtype=np.float32)
        assert dht.shape == (N, H, D, D)
    r = {n: np.zeros((B, T, H, D)) for n in ("dq", "dk", "dv", "dg")}
    r["dbeta"] = np.zeros((B, T, H))
    r["dA_log"] = np.zeros(H)
    r["ddt_bias"] = np.zeros((H, D))
    r["dh0"] = np.zeros((N, H, D, D))
    rc = lib().oracle_kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(A_log),
                              _ptr(dt_bias), float(lower_bound), int(flags), _ptr(initial_state), sd,
                              _ptr(cu_seqlens), B, T, H, N, _ptr(dout), _ptr(dht), _ptr(r["dq"]),
                              _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dg"]), _ptr(r["dbeta"]),
                              _ptr(r["dA_log"]), _ptr(r["ddt_bias"]), _ptr(r["dh0"]), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_kda_bwd failed ({rc})")
    return r


def max_threads() -> int:
    return int(lib().oracle_max_threads())
