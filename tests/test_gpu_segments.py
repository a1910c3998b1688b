"""GPU parity of the cut plan where the carried state matters.

Long sequences run under the cut plan: the P workgroups of a head take equal runs of its
chunks, cutting sequences into pieces.  Pass A runs every piece (a sequence's first piece
from the true initial state, the others from S = 0: F_j), transition runs give each cut
piece's P_j (the run from S = I with v = 0), a scan S_{j+1} = S_j P_j + F_j, and pass B
reruns the cut pieces from S_j.  With a strong gate (lower_bound -5) the state is forgotten
within a few tokens, so a wrong S_j would show in the first tokens of a piece only; these
tests run where the state persists for hundreds of tokens (lower_bound -0.05) or for the
whole sequence (lower_bound 0, no decay: no transition run stops early), and also compare
F_j, P_j and S_j themselves with the fp64 oracle run over the same token ranges.  Also
here: long whole-chain sequences with weak decay, and isolation of a NaN to its own
(sequence, head) chain.

Acceptance as everywhere: out max|err| <= 2e-2, relative L2 <= 5e-3; final_state relative
L2 <= 1e-3 (fp32) / 1e-2 (bf16); the segment states are held to the fp32 bar.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_86_amd import kda
from gated_delta_rule_86_amd import workloads as W
from kda_testutil import (check_final, check_out, cut_plan, expected_cuts, rel_l2, run_gpu, run_oracle,
                          segment_states, seq_chunk_offsets, to_device)

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
    """Cut-plan runs (P >= 5 per head) where the state persists across pieces."""
    P = cut_plan(B, T, H)
    assert P >= 5, (B, T, H, P)
    w = W.make(f"segweak_B{B}_T{T}_H{H}_lb{lb}", B, T, H, seed=400 + T + H, lower_bound=lb, state_dtype=sd)
    parity(w, f"cut plan P={P} lb={lb} {sd}")


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
    """F_j, P_j and S_j as the forward pass left them in its workspace, against the oracle
    over the same token ranges: F_j from zero, P_j from the identity with v = 0, S_j the
    state of the one-shot run at cut j (one batch row: the cuts split it evenly)."""
    B, T, H = 1, 4096, 2
    P = cut_plan(B, T, H)
    assert P >= 5
    w = W.make(f"segstates{lb}", B, T, H, seed=420, lower_bound=lb, state_dtype="fp32")
    _, _, ws = run_gpu(w)
    S, F, Pm = segment_states(ws, B, H, P)
    cuts = expected_cuts(seq_chunk_offsets(w), P)
    h0 = w.initial_state.astype(np.float64)
    eye = np.broadcast_to(np.eye(128), (B, H, 128, 128)).copy()
    zero = np.zeros((B, H, 128, 128))
    bounds = [16 * c for _, c in cuts[:P]] + [T]  # first token of the piece at cut j
    worst = {"S": 0.0, "F": 0.0, "P": 0.0}
    for j in range(1, P):
        t0, t1 = bounds[j], bounds[j + 1]
        rF = _oracle_state(w, t0, t1, zero)
        rP = _oracle_state(w, t0, t1, eye, v_zero=True)
        rS = _oracle_state(w, 0, t0, h0)
        worst["F"] = max(worst["F"], check_final(F[:, j], rF[0], "fp32", f"F_{j}"))
        worst["P"] = max(worst["P"], check_final(Pm[:, j], rP[0], "fp32", f"P_{j}"))
        worst["S"] = max(worst["S"], check_final(S[:, j], rS[0], "fp32", f"S_{j}"))
    # the affine hand-off the scan relies on, on the oracle's own states
    j = P // 2
    rSj = _oracle_state(w, 0, bounds[j], h0)
    rF = _oracle_state(w, bounds[j], bounds[j + 1], zero)
    rP = _oracle_state(w, bounds[j], bounds[j + 1], eye, v_zero=True)
    rS1 = _oracle_state(w, 0, bounds[j + 1], h0)
    assert rel_l2(np.einsum("bhvc,bhcd->bhvd", rSj, rP) + rF, rS1) < 1e-12
    print(f"cut states P={P} lb={lb}: worst relL2 " +
          " ".join(f"{k} {v:.2e}" for k, v in worst.items()), flush=True)


@pytest.mark.parametrize("lb,sd", [(0.0, "fp32"), (-0.05, "fp32"), (0.0, "bf16")])
@pytest.mark.parametrize("plan", ["whole", "cut"])
def test_varlen_weak_decay_long(lb, sd, plan):
    """Sequences of 4100 and 5003 tokens (257 and 313 chunks) carried with no or weak decay,
    as whole chains (next to 200 short sequences, which keep the batch on the whole-chain
    plans) and under the cut plan (alone)."""
    lengths = [4100] + [10] * 100 + [5003] + [7] * 100 if plan == "whole" else [4100, 5003]
    w = W.make(f"varlenweak{lb}{sd}{plan}", 1, 0, 2, lengths=lengths, seed=430, lower_bound=lb,
               state_dtype=sd)
    assert kda.forward_launches(1, w.T, w.H, len(lengths), True) == (1 if plan == "whole" else 3)
    parity(w, f"{plan} plan, sequences of 4100/5003 lb={lb} {sd}")


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
    assert kda.forward_launches(3, 1500, 2) == 3
    _nan_isolation(w, (1, 700, 1), "cut-plan launch")
