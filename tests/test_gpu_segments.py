"""GPU parity of the segmented forward pass where the carried state matters.

Few long equal-length chains run as G segments: pass A (segment 0 from the true initial
state; for the middle segments F = the segment run from S = 0 and P = the run from S = I
with v = 0), a scan S_{g+1} = S_g P_g + F_g, and pass B (segments 1 .. G-1 from S_g, with
out).  With a strong gate (lower_bound -5) the state is forgotten within a few tokens, so
a wrong S_g would show in the first tokens of a segment only; these tests run where the
state persists for hundreds of tokens (lower_bound -0.05) or for the whole sequence
(lower_bound 0, no decay), and also compare F_g, P_g and S_g themselves with the fp64
oracle run over the same token ranges.  Also here: long whole-chain sequences with weak
decay, and isolation of a NaN to its own (sequence, head) chain.

Acceptance as everywhere: out max|err| <= 2e-2, relative L2 <= 5e-3; final_state relative
L2 <= 1e-3 (fp32) / 1e-2 (bf16); the segment states are held to the fp32 bar.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_86_amd import kda
from gated_delta_rule_86_amd import workloads as W
from kda_testutil import (check_final, check_out, rel_l2, run_gpu, run_oracle, segment_bounds,
                          segment_plan, segment_states, to_device)

pytestmark = pytest.mark.gpu


def parity(w, what):
    o, f, ws = run_gpu(w)
    ro, rf = run_oracle(w)
    mx, rl = check_out(o, ro, what)
    msg = f"{what}: out max {mx:.2e} relL2 {rl:.2e}"
    if f is not None:
        msg += f" final relL2 {check_final(f, rf, w.final_dtype, what):.2e}"
    print(msg, flush=True)
    return ws


@pytest.mark.parametrize("B,T,H,lb,sd", [
    (1, 8192, 2, 0.0, "fp32"),
    (1, 8192, 2, -0.05, "fp32"),
    (1, 6000, 2, 0.0, "bf16"),
    (3, 4096, 2, 0.0, "fp32"),
    (2, 5000, 3, -0.05, "bf16"),
    (1, 4103, 1, 0.0, "fp32"),
])
def test_segmented_weak_decay(B, T, H, lb, sd):
    """Segmented runs (G >= 5) where the state persists across segments."""
    G, L = segment_plan(B * H, -(-T // 16))
    assert G >= 5, (B, T, H, G)
    w = W.make(f"segweak_B{B}_T{T}_H{H}_lb{lb}", B, T, H, seed=400 + T + H, lower_bound=lb, state_dtype=sd)
    parity(w, f"segmented G={G} L={L} lb={lb} {sd}")


def _window(w, t0, t1, v_zero=False):
    sl = lambda a: np.ascontiguousarray(a[:, t0:t1])
    v = np.zeros_like(sl(w.v)) if v_zero else sl(w.v)
    return sl(w.q), sl(w.k), v, sl(w.g), sl(w.beta)


def _oracle_state(w, t0, t1, S0, v_zero=False):
    """final state (float64 [B, H, 128, 128]) of the oracle over tokens [t0, t1) of every
    batch row, from S0 (float64 [B, H, 128, 128])."""
    q, k, v, g, b = _window(w, t0, t1, v_zero)
    _, f = oracle.kda_fwd(q, k, v, g, b, w.scale, w.A_log, w.dt_bias, w.lower_bound, S0,
                          want_out=False)
    return f


@pytest.mark.parametrize("lb", [0.0, -0.05])
def test_segment_states_match_oracle(lb):
    """F_g, P_g and S_g as the forward pass left them in its workspace, against the oracle
    over the same token ranges: F_g from zero, P_g from the identity with v = 0, S_g the
    state of the one-shot run at the segment's first token."""
    B, T, H = 1, 4096, 2
    G, L = segment_plan(B * H, T // 16)
    assert G >= 5
    w = W.make(f"segstates{lb}", B, T, H, seed=420, lower_bound=lb, state_dtype="fp32")
    _, _, ws = run_gpu(w)
    S, F, P = segment_states(ws, B, H, G)
    h0 = w.initial_state.astype(np.float64)
    eye = np.broadcast_to(np.eye(128), (B, H, 128, 128)).copy()
    zero = np.zeros((B, H, 128, 128))
    bounds = [min(16 * c, T) for c in segment_bounds(G, L, T // 16)]  # first token of segment g
    worst = {"S": 0.0, "F": 0.0, "P": 0.0}
    for g in range(1, G - 1):
        t0, t1 = bounds[g], bounds[g + 1]
        rF = _oracle_state(w, t0, t1, zero)
        rP = _oracle_state(w, t0, t1, eye, v_zero=True)
        worst["F"] = max(worst["F"], check_final(F[:, :, g], rF, "fp32", f"F_{g}"))
        worst["P"] = max(worst["P"], check_final(P[:, :, g], rP, "fp32", f"P_{g}"))
    for g in range(1, G):
        rS = _oracle_state(w, 0, bounds[g], h0)
        worst["S"] = max(worst["S"], check_final(S[:, :, g], rS, "fp32", f"S_{g}"))
    # the affine hand-off the scan relies on, on the oracle's own states
    g = G // 2
    rSg = _oracle_state(w, 0, bounds[g], h0)
    rF = _oracle_state(w, bounds[g], bounds[g + 1], zero)
    rP = _oracle_state(w, bounds[g], bounds[g + 1], eye, v_zero=True)
    rS1 = _oracle_state(w, 0, bounds[g + 1], h0)
    assert rel_l2(np.einsum("bhvc,bhcd->bhvd", rSg, rP) + rF, rS1) < 1e-12
    print(f"segment states G={G} L={L} lb={lb}: worst relL2 " +
          " ".join(f"{k} {v:.2e}" for k, v in worst.items()), flush=True)


@pytest.mark.parametrize("lb,sd", [(0.0, "fp32"), (-0.05, "fp32"), (0.0, "bf16")])
def test_whole_chain_weak_decay_long(lb, sd):
    """Varlen batches run whole chains: sequences of 4100 and 5003 tokens (257 and 313
    chunks) carried with no or weak decay."""
    w = W.make(f"wholeweak{lb}{sd}", 1, 0, 2, lengths=[4100, 5003], seed=430, lower_bound=lb,
               state_dtype=sd)
    assert kda.forward_launches(1, w.T, w.H, 2, True) == 1
    parity(w, f"whole chains 4100/5003 lb={lb} {sd}")


def _nan_isolation(w, where, what):
    """Poison one (token, head) of v with NaN: that chain's results may change, every other
    chain's out rows and final state stay bit-identical to the clean run."""
    import torch
    d = to_device(w)
    o_clean, f_clean, _ = run_gpu(w, d, keep_device=True)
    o_clean, f_clean = o_clean.clone(), f_clean.clone()
    n_bad, t_bad, h_bad = where  # t_bad counts from the start of sequence n_bad
    lens = w.lengths
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    v = d["v"].clone()
    if w.cu_seqlens is not None:
        v[0, int(starts[n_bad]) + t_bad, h_bad, :] = float("nan")
    else:
        v[n_bad, t_bad, h_bad, :] = float("nan")
    d2 = dict(d, v=v)
    o, f, _ = run_gpu(w, d2, keep_device=True)
    torch.cuda.synchronize()
    for n in range(w.N):
        for h in range(w.H):
            if (n, h) == (n_bad, h_bad):
                continue
            if w.cu_seqlens is not None:
                a = o[0, starts[n]:starts[n] + lens[n], h]
                b = o_clean[0, starts[n]:starts[n] + lens[n], h]
            else:
                a, b = o[n, :, h], o_clean[n, :, h]
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (what, n, h)
            assert torch.equal(f[n, h].view(torch.int32), f_clean[n, h].view(torch.int32)), (what, n, h)
    tb = starts[n_bad] + t_bad if w.cu_seqlens is not None else t_bad
    bad_row = o[0 if w.cu_seqlens is not None else n_bad, tb, h_bad]
    assert torch.isnan(bad_row.float()).any(), what  # the poisoned chain does see it
    print(f"{what}: NaN confined to chain (n={n_bad}, h={h_bad})", flush=True)


def test_nan_confined_to_its_chain_whole():
    w = W.make("nan_whole", 1, 0, 3, lengths=[50, 70, 33, 200], seed=440, state_dtype="fp32")
    _nan_isolation(w, (1, 5, 0), "whole-chain launch")


def test_nan_confined_to_its_chain_segmented():
    w = W.make("nan_seg", 3, 1500, 2, seed=441, state_dtype="fp32")
    assert kda.forward_launches(3, 1500, 2) == 2
    _nan_isolation(w, (1, 700, 1), "segmented launch")
