"""Bit-exact GPU checks: the integer chunk table, coverage, isolation, determinism.

* chunk table (cu_seqlens -> per-sequence chunk offsets, total): equal, bit for bit, to a
  brute-force enumeration of 16-token chunk starts and to sum(ceil(L_i / 16)); invalid
  cu_seqlens set the documented status bits and make every sequence empty.
* the split of a head's sequences into per-workgroup units, bit for bit against a replica
  of each plan: column halves packed longest first (few workgroups and few sequences per
  head), snake order by length (up to 512 sequences), contiguous runs of about equal chunk
  count (brute-force assignment by chunk midpoint) beyond that; for long sequences the cut
  plan's cuts (equal runs of the head's chunks, moved onto nearby sequence boundaries).
* every out element and every final_state element is written (NaN sentinels vanish);
* perturbing one sequence leaves every other sequence's out and final_state bit-identical;
* two runs are bitwise identical, also with a workspace pre-filled with garbage;
* scaling (v, initial_state) by 2 scales out and final_state by exactly 2.
"""
import numpy as np
import pytest

from gated_delta_rule_86_amd import kda
from gated_delta_rule_86_amd import workloads as W
from kda_testutil import (cut_plan, cut_table, expected_cuts, expected_firsts, final_tensor, run_gpu, to_device,
                          torch_dev)

pytestmark = pytest.mark.gpu


def brute_chunk_offsets(cu):
    offs = [0]
    for i in range(len(cu) - 1):
        starts = list(range(int(cu[i]), int(cu[i + 1]), 16))
        offs.append(offs[-1] + len(starts))
    return np.array(offs, dtype=np.int64)


@pytest.mark.parametrize("N", [1, 7, 255, 256, 257, 1000, 3000])
def test_chunk_table_matches_enumeration(N):
    import torch
    rng = np.random.default_rng(N)
    L = rng.integers(0, 70, size=N)
    L[rng.random(N) < 0.2] = 0
    L[rng.random(N) < 0.2] = 16 * rng.integers(1, 4)
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(L)
    T = int(cu[-1])
    seq_off, n_total, status = kda.chunk_table(torch.from_numpy(cu).to(torch_dev()), 1, T, 2)
    ref = brute_chunk_offsets(cu)
    assert status == 0
    assert np.array_equal(seq_off, ref)
    assert n_total == int(ref[-1]) == int(np.sum((L + 15) // 16))


def test_chunk_table_batch_mode():
    for B, T in [(1, 0), (2, 4096), (3, 17), (5, 1)]:
        seq_off, n_total, status = kda.chunk_table(None, B, T, 1)
        assert status == 0 and n_total == B * ((T + 15) // 16)
        assert np.array_equal(seq_off, np.arange(B + 1) * ((T + 15) // 16))


@pytest.mark.parametrize("cu,T,bits", [([1, 5, 9], 9, 1), ([0, 9, 5, 12], 12, 2), ([0, 5, 11], 12, 4),
                                       ([3, 2, 11], 12, 1 | 2 | 4)])
def test_chunk_table_invalid(cu, T, bits):
    import torch
    cu_t = torch.tensor(cu, dtype=torch.int64, device=torch_dev())
    seq_off, n_total, status = kda.chunk_table(cu_t, 1, T, 1)
    assert status == bits
    assert n_total == 0 and not seq_off.any()


def test_invalid_cu_seqlens_leaves_out_and_keeps_state():
    import torch
    w = W.make("bad_cu", 1, 0, 2, lengths=[10, 20], seed=400)
    d = to_device(w)
    d["cu"] = torch.tensor([0, 31, 30], dtype=torch.int64, device=torch_dev())  # decreasing, cu[N] == T
    o, f, ws = run_gpu(w, d, out_fill=7.0)
    assert kda.device_status(ws) == 2
    assert np.all(o == 7.0)
    assert np.array_equal(f, w.initial_state.astype(np.float64))


@pytest.mark.parametrize("bad", ["decreasing", "first", "last"])
def test_invalid_cu_seqlens_under_cut_plan(bad):
    """Long sequences (the cut plan's launch of three passes and the scan): invalid content
    writes no out, final_state equals initial_state and the cut table holds only empty runs."""
    import torch
    lengths = [0, 3000, 17, 0, 5000, 1, 2048, 900]
    w = W.make(f"bad_cu_cut_{bad}", 1, 0, 4, lengths=lengths, seed=401, state_dtype="fp32")
    P = cut_plan(1, w.T, w.H, len(lengths), True)
    assert P > 1 and kda.forward_launches(1, w.T, w.H, len(lengths), True) == 3
    cu = w.cu_seqlens.copy()
    if bad == "decreasing":
        cu[3] = cu[2] - 1
    elif bad == "first":
        cu[0] = -1  # (the first sequence is empty: a positive start would also break monotony)
    else:
        cu[-1] = w.T - 1
    d = to_device(w)
    d["cu"] = torch.tensor(cu, dtype=torch.int64, device=torch_dev())
    o, f, ws = run_gpu(w, d, out_fill=7.0, final_fill=-3.0)
    assert kda.device_status(ws) == {"decreasing": 2, "first": 1, "last": 4}[bad]
    assert np.all(o == 7.0)
    assert np.array_equal(f, w.initial_state.astype(np.float64))
    cuts, firsts = cut_table(ws, len(lengths), P)
    assert cuts == [(0, 0)] + [(len(lengths), 0)] * P and firsts == list(range(P + 1))


def test_every_output_is_written():
    import torch
    w = W.make("cover", 1, 0, 3, lengths=[1, 16, 17, 0, 40, 5], seed=401, state_dtype="bf16")
    out, fin, _ = run_gpu(w, out_fill=float("nan"), final_fill=float("nan"), keep_device=True)
    assert not torch.isnan(out).any()
    assert not torch.isnan(fin).any()


def test_sequences_are_isolated():
    import torch
    lens = [37, 16, 50, 3]
    w = W.make("iso", 1, 0, 2, lengths=lens, seed=402)
    o1, f1, _ = run_gpu(w, keep_device=True)
    cu = w.cu_seqlens
    w2 = W.make("iso", 1, 0, 2, lengths=lens, seed=402)
    t0, t1 = int(cu[1]), int(cu[2])
    for a in (w2.q, w2.k, w2.v, w2.g, w2.beta):
        a[:, t0:t1] = a[:, t0:t1][..., ::-1].copy() if a.ndim == 4 else a[:, t0:t1] ^ np.uint16(0x8000)
    w2.initial_state[1] *= -3.0
    o2, f2, _ = run_gpu(w2, keep_device=True)
    for n in (0, 2, 3):
        a, b = int(cu[n]), int(cu[n + 1])
        assert torch.equal(o1[:, a:b], o2[:, a:b])
        assert torch.equal(f1[n], f2[n])
    assert not torch.equal(o1[:, t0:t1], o2[:, t0:t1])


def test_deterministic_and_workspace_independent():
    import torch
    w = W.make("det", 2, 333, 3, seed=403)
    d = to_device(w)
    o1, f1, ws = run_gpu(w, d, keep_device=True)
    ws.fill_(0xFF)
    o2, f2, _ = run_gpu(w, d, workspace=ws, keep_device=True)
    o3, f3, _ = run_gpu(w, d, keep_device=True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    assert torch.equal(o1, o3) and torch.equal(f1, f3)


def test_power_of_two_scaling_is_exact():
    import torch
    w = W.make("pow2", 1, 0, 2, lengths=[45, 64], seed=404, lower_bound=-2.0)
    d = to_device(w)
    o1, f1, _ = run_gpu(w, d, keep_device=True)
    d2 = dict(d)
    d2["v"] = d["v"] * 2
    d2["h0"] = d["h0"] * 2
    o2, f2, _ = run_gpu(w, d2, keep_device=True)
    assert torch.equal(o2, 2 * o1)
    assert torch.equal(f2, 2 * f1)


def expected_runs(seq_off, P):
    """First sequence of each of the P workgroups of a head: sequence i goes to workgroup
    floor(P * mid_i / total) (at most P - 1) with mid_i its chunk midpoint; all to the last
    workgroup when there are no chunks.  Brute force over the sequences."""
    N = len(seq_off) - 1
    tot = int(seq_off[-1])
    grp = [P - 1 if tot == 0 else min(P - 1, (int(seq_off[i]) + int(seq_off[i + 1])) * P // (2 * tot))
           for i in range(N)]
    return np.array([next((i for i in range(N) if grp[i] >= s), N) for s in range(P)] + [N], dtype=np.int64)


# whole-chain plan with column halves (constants of the chunk-table plan)
SPLIT_MAX_P, SPLIT_MAX_SEQ, SPLIT_MAX_K, WHOLE_W, HALF_W = 16, 32, 8, 100, 82
SNAKE_MAX_SEQ = 512


def split_eligible(H, N):
    return 256 // H <= SPLIT_MAX_P and N <= SPLIT_MAX_SEQ


def whole_chain_groups(H, N):
    units = 2 * N if split_eligible(H, N) else N
    return max(1, min(max(1, 256 // H), units))


def pack_halves(n, order, P, k):
    """Longest first onto P workgroups, the k longest sequences as two halves of weight
    82 n each, the others whole at 100 n; ties take a half first, then the least loaded
    workgroup with the lowest index.  Returns (largest load, [(seq, code, workgroup)])."""
    halves = [(HALF_W * n[order[i // 2]], order[i // 2], 1 + (i & 1)) for i in range(2 * k)]
    wholes = [(WHOLE_W * n[order[i]], order[i], 0) for i in range(k, len(n))]
    load, units, hi, wi = [0] * P, [], 0, 0
    while hi < len(halves) or wi < len(wholes):
        wh = halves[hi][0] if hi < len(halves) else -1
        ww = wholes[wi][0] if wi < len(wholes) else -1
        if wh >= ww:
            w, seq, code = halves[hi]
            hi += 1
        else:
            w, seq, code = wholes[wi]
            wi += 1
        b = min(range(P), key=lambda i: (load[i], i))
        load[b] += w
        units.append((seq, code, b))
    return max(load), units


def expected_plan(seq_off, H):
    """(unit codes, first unit of each workgroup, P) of a head's whole-chain launch."""
    N = len(seq_off) - 1
    P = whole_chain_groups(H, N)
    if not split_eligible(H, N):
        if N > SNAKE_MAX_SEQ or P == 1:
            return np.arange(N, dtype=np.int64) << 2, expected_runs(seq_off, P), P
        # snake order: rank r (longest first, ties by index) -> workgroup r % P in even
        # rounds r // P, P - 1 - r % P in odd ones
        n = [int(seq_off[i + 1] - seq_off[i]) for i in range(N)]
        order = sorted(range(N), key=lambda i: (-n[i], i))
        bins = [[] for _ in range(P)]
        for r, i in enumerate(order):
            rnd, pos = divmod(r, P)
            bins[pos if rnd % 2 == 0 else P - 1 - pos].append(i)
        codes = [i << 2 for b in bins for i in b]
        wg = np.cumsum([0] + [len(b) for b in bins])
        return np.array(codes, dtype=np.int64), wg.astype(np.int64), P
    n = [int(seq_off[i + 1] - seq_off[i]) for i in range(N)]
    order = sorted(range(N), key=lambda i: (-n[i], i))
    mks = [pack_halves(n, order, P, k)[0] for k in range(min(SPLIT_MAX_K, N) + 1)]
    _, units = pack_halves(n, order, P, mks.index(min(mks)))
    codes, wg = [], []
    for b in range(P):
        wg.append(len(codes))
        codes += [(sq << 2) | c for sq, c, bb in units if bb == b]
    wg.append(len(codes))
    return np.array(codes, dtype=np.int64), np.array(wg, dtype=np.int64), P


@pytest.mark.parametrize("N,H,kind", [(1, 1, "rand"), (8, 32, "rand"), (256, 32, "rand"), (300, 1, "rand"),
                                      (1000, 3, "rand"), (5, 4, "empty"), (9, 2, "one_long"),
                                      (40, 8, "bad"), (8, 32, "one_long"), (3, 16, "one_long"),
                                      (32, 16, "rand"), (20, 32, "empty"), (12, 32, "two_long"),
                                      (33, 32, "one_long"), (6, 64, "two_long"), (512, 32, "rand"),
                                      (513, 32, "rand"), (257, 1, "rand"), (100, 3, "empty"),
                                      (8, 32, "long"), (7, 4, "long_empty"), (3, 1, "long"), (20, 2, "long_empty")])
def test_workgroup_runs(N, H, kind):
    """The split of sequences into per-workgroup units (whole-chain plans) or the cut table
    (cut plan), bit for bit."""
    import torch
    rng = np.random.default_rng(N + H)
    L = rng.integers(0, 200, size=N)
    if kind == "empty":
        L[:] = 0
    elif kind == "one_long":
        L[:] = 3
        L[N // 2] = 5000
    elif kind == "two_long":
        L[1] = 3000
        L[N - 2] = 2200
    elif kind.startswith("long"):
        L = rng.integers(1, 8193, size=N)
        if kind == "long_empty":
            L[::3] = 0
            L[1] = 16 * 97
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(L)
    T = int(cu[-1])
    if kind == "bad":
        cu[3] = cu[4] + 1  # decreasing: every sequence becomes empty
    up = lambda x: -(-x // 256) * 256
    ws = torch.empty(kda.workspace_size(1, T, H, N, True), dtype=torch.uint8, device=torch_dev())
    seq_off, _, status = kda.chunk_table(torch.from_numpy(cu).to(torch_dev()), 1, T, H, workspace=ws)
    Pc = cut_plan(1, T, H, N, True)
    assert (Pc > 1) == kind.startswith("long") or kind == "one_long", (N, H, kind, Pc)
    if Pc > 1:
        cuts = expected_cuts(seq_off, Pc)
        got = cut_table(ws, N, Pc)
        assert got == (cuts, expected_firsts(cuts)), (got, cuts)
        assert (status != 0) == (kind == "bad")
        return
    codes, runs_ref, P = expected_plan(seq_off, H)
    off = 256 + 2 * up(8 * N) + up(8 * (N + 1))
    runs = ws[off:off + 8 * (P + 1)].cpu().numpy().view(np.int64)
    assert np.array_equal(runs, runs_ref), (runs, runs_ref)
    off_units = off + up(8 * 257)
    units = ws[off_units:off_units + 4 * int(runs[-1])].cpu().numpy().view(np.int32)
    assert np.array_equal(units.astype(np.int64), codes), (units, codes)
    # every sequence appears once whole or as both halves
    seen = sorted((int(c) >> 2, int(c) & 3) for c in units)
    for i in range(N):
        mine = [c for sq, c in seen if sq == i]
        assert mine in ([0], [1, 2]), (i, mine)
    assert (status != 0) == (kind == "bad")
    if kind in ("one_long", "two_long") and split_eligible(H, N) and whole_chain_groups(H, N) > 1:
        assert any(int(c) & 3 for c in units)  # the long sequences run as column halves


def test_segmented_workspace_garbage():
    """Cut-plan batch rows (pass A, transition runs, scan, pass B) with a workspace
    pre-filled with garbage: the status word reads 0, the chunk total is right, and out and
    final_state are bit-identical to a run on a fresh workspace."""
    import torch
    w = W.make("segws", 2, 1100, 2, seed=405)
    assert kda.forward_launches(2, 1100, 2) == 3
    d = to_device(w)
    o1, f1, _ = run_gpu(w, d, keep_device=True)
    ws = torch.full((kda.workspace_size(2, 1100, 2),), 0xFF, dtype=torch.uint8, device=torch_dev())
    o2, f2, _ = run_gpu(w, d, workspace=ws, keep_device=True)
    assert kda.device_status(ws) == 0
    assert int(ws[8:16].cpu().numpy().view(np.int64)[0]) == 2 * ((1100 + 15) // 16)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
