"""GPU parity of the cut plan, where pieces' start states are dropped.

Long sequences run under the cut plan: the P workgroups of a head take equal runs of its
chunks, cutting sequences into pieces.  For the piece at cut j a transition run from the
identity (v = 0) stops once every entry of its state is below 2^-37 |F_j|_F / B_j, with F_j
the piece's run from zero and B_j = |S_j0|_F + |F_j0|_F + ... + |F_{j-1}|_F; the scan then
takes S_{j+1} = F_j, and pass B reruns only the chunks before the stop.  These tests check
the cut table bit for bit against a replica, that the mechanism fires where the gate
forgets quickly, stays off where it does not (weak decay, switches that lift the
spectral-norm bound), and that out and final_state match the fp64 oracle in every piece,
also when one piece's values are far larger or far smaller than the rest (the stop bound
is relative to the piece's own state), for batch rows and for varlen batches with empty,
short and long sequences.

Acceptance: out max|err| <= 2e-2 and relative L2 <= 5e-3 over the whole tensor, and
relative L2 <= 5e-3 within every piece (per-piece max|err| is not held to 2e-2 where the
test scales a piece's values up); final_state relative L2 <= 1e-3 (fp32) / 1e-2 (bf16).
"""
import numpy as np
import pytest

from gated_delta_rule_86_amd import workloads as W
from kda_testutil import (OUT_REL_L2, check_final, check_out, cut_plan, cut_table, expected_cuts, expected_firsts,
                          pieces, rel_l2, run_gpu, run_oracle, segment_aux, seq_chunk_offsets)

pytestmark = pytest.mark.gpu


def _seq_rows(w, o, i, t0, t1):
    """Rows [t0, t1) of sequence i of an out-shaped array."""
    if w.cu_seqlens is None:
        return o[i, t0:t1]
    s = int(w.cu_seqlens[i])
    return o[0, s + t0:s + t1]


def _run(w, what, whole_bars=True):
    """GPU and oracle; the cut table against its replica; out per piece.  Returns (z, drop,
    cuts, P)."""
    o, f, ws = run_gpu(w)
    ro, rf = run_oracle(w)
    varlen = w.cu_seqlens is not None
    P = cut_plan(w.B, w.T, w.H, w.N, varlen)
    assert P > 1, (w.B, w.T, w.H, w.N)
    seq_off = seq_chunk_offsets(w)
    cuts = expected_cuts(seq_off, P)
    assert cut_table(ws, w.N, P) == (cuts, expected_firsts(cuts))
    if whole_bars:
        mx, rl = check_out(o, ro, what)
    else:
        mx, rl = float(np.abs(o - ro).max()), rel_l2(o, ro)
    lens = w.lengths if varlen else [w.T] * w.B
    worst = 0.0
    for j, i, c0, c1 in pieces(seq_off, cuts):
        t0, t1 = 16 * c0, min(16 * c1, int(lens[i]))
        if t1 <= t0:
            continue
        r = rel_l2(_seq_rows(w, o, i, t0, t1), _seq_rows(w, ro, i, t0, t1))
        worst = max(worst, r)
        assert r <= OUT_REL_L2, f"{what}: piece at cut {j} of sequence {i}, tokens {t0}..{t1}: out relL2 {r:.3e}"
    fr = check_final(f, rf, w.final_dtype, what)
    z, drop, _, _ = segment_aux(ws, w.N, w.H, P)
    inner = [j for j in range(1, P) if cuts[j][1] > 0]
    zi = z[:, inner]
    print(f"{what}: P={P}, {len(inner)} cuts inside sequences; out max {mx:.2e} relL2 {rl:.2e} worst piece "
          f"{worst:.2e} final {fr:.2e}; z min {zi.min(initial=0)} max {zi.max(initial=0)} dropped "
          f"{int(drop[:, inner].sum())}/{zi.size}", flush=True)
    # the scan drops a share exactly where the transition run stopped
    assert np.array_equal(drop[:, inner], (zi >= 0).astype(np.int64))
    return z, drop, cuts, P


@pytest.mark.parametrize("B,T,H,lb,sd", [
    (2, 4096, 16, -5.0, "fp32"),
    (3, 4103, 8, -2.0, "bf16"),
    (1, 8192, 4, -1.0, "fp32"),
])
def test_strong_decay_drops(B, T, H, lb, sd):
    """With a strong gate every transition run stops within a few chunks."""
    w = W.make(f"trunc_B{B}_T{T}_H{H}_lb{lb}", B, T, H, seed=700 + H, lower_bound=lb, state_dtype=sd)
    z, drop, cuts, P = _run(w, f"strong decay B={B} T={T} H={H} lb={lb} {sd}")
    inner = [j for j in range(1, P) if cuts[j][1] > 0]
    assert inner and np.all(z[:, inner] >= 1) and np.all(z[:, inner] <= 12), z[:, inner]


def test_mixed_memory():
    """Head 0 has no decay over the first half of the sequence (its gate pre-activation is
    -30: sigmoid ~ 0), so the transition runs there cannot stop; everywhere else they do.
    The scan mixes computed and dropped steps in one chain."""
    B, T, H = 1, 8192, 2
    w = W.make("trunc_mixed", B, T, H, seed=720, lower_bound=-5.0, state_dtype="fp32")
    g = W.bf16_bits_to_f32(w.g).copy()
    g[0, :T // 2, 0, :] = -30.0
    w.g = W.f32_to_bf16_bits(g)
    z, drop, cuts, P = _run(w, "mixed memory")
    half = T // 32  # chunk where the decay starts
    for j in range(1, P):
        c0, c1 = cuts[j][1], cuts[j + 1][1] if j + 1 < P else T // 16
        if c1 <= half:
            assert z[0, j] == -1, (j, z[0])
        elif c0 >= half:
            assert z[0, j] >= 1, (j, z[0])
        assert z[1, j] >= 1, (j, z[1])


@pytest.mark.parametrize("factor", [1e4, 1e-4])
def test_scaled_piece(factor):
    """The values of one piece scaled by 1e4 (its state dwarfs the next pieces' bound term)
    or by 1e-4 (its own end state is tiny next to the start state it forgets): the stop
    bound is relative to the piece's own end state, so every piece still matches the oracle
    relative to its own scale."""
    B, T, H = 1, 4096, 2
    w = W.make(f"trunc_scaled{factor}", B, T, H, seed=730, lower_bound=-5.0, state_dtype="fp32")
    P = cut_plan(B, T, H)
    cuts = expected_cuts(seq_chunk_offsets(w), P)
    v = W.bf16_bits_to_f32(w.v).copy()
    t0, t1 = 16 * cuts[3][1], 16 * cuts[4][1]
    v[0, t0:t1] *= np.float32(factor)
    w.v = W.f32_to_bf16_bits(v)
    _run(w, f"piece 3 values x{factor:g}", whole_bars=False)


def test_switch_off_keeps_every_share():
    """Without the in-kernel l2norm the transitions need not be contractions: no run stops,
    nothing is dropped, and the path is the exact affine scan."""
    w = W.make("trunc_l2off", 1, 4096, 2, seed=740, lower_bound=-5.0, flags=5, state_dtype="fp32")
    z, drop, cuts, P = _run(w, "l2norm switch off")
    assert np.all(z[:, 1:] == -1) and not np.any(drop[:, 1:])


VARLEN_LENGTHS = [0, 3000, 17, 0, 5000, 1, 2048, 900]


@pytest.mark.parametrize("lb,sd", [(-2.0, "bf16"), (0.0, "fp32"), (-5.0, "fp32")])
def test_varlen_cuts(lb, sd):
    """Varlen batch with empty, one-token, short and long sequences: cuts inside the long
    ones (several per sequence), cuts moved onto nearby sequence boundaries, empty
    sequences at run boundaries.  With no decay (lower_bound 0) nothing is dropped and the
    scan carries states across several cuts of one sequence."""
    w = W.make(f"cuts_varlen{lb}{sd}", 1, 0, 4, lengths=VARLEN_LENGTHS, seed=750, lower_bound=lb,
               state_dtype=sd)
    z, drop, cuts, P = _run(w, f"varlen cuts lb={lb} {sd}")
    inner = [j for j in range(1, P) if cuts[j][1] > 0]
    assert len(inner) >= 20
    if lb == 0.0:
        assert np.all(z[:, inner] == -1)
    else:
        assert np.all(z[:, inner] >= 1)


@pytest.mark.parametrize("T,H,lb", [(65536 + 37, 1, 0.0), (65536 + 37, 1, -1.0), (32768 + 5, 2, -0.05)])
def test_largest_cut_plans(T, H, lb):
    """The largest plans: 256 workgroups per head (H = 1, the cut table at its full 257
    entries) and 128 (H = 2), each run cutting the one sequence; without decay no transition
    run stops and the scan carries the state through 255 affine steps."""
    w = W.make(f"maxcuts_T{T}_H{H}_lb{lb}", 1, T, H, seed=760 + H, lower_bound=lb, state_dtype="fp32")
    z, drop, cuts, P = _run(w, f"largest cut plan T={T} H={H} lb={lb}")
    assert P == 256 // H
    inner = [j for j in range(1, P) if cuts[j][1] > 0]
    assert len(inner) == P - 1
    if lb == 0.0:
        assert np.all(z[:, inner] == -1)
