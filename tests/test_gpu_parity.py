"""GPU parity: kda_fwd (HIP, through the C ABI) against the fp64 oracle.

Acceptance (fp64 oracle on the same seeded inputs): out max|err| <= 2e-2 and relative
L2 <= 5e-3; final_state relative L2 <= 1e-3 (fp32 states) or <= 1e-2 (bf16 states).
Covers the five reference workloads (the 1M-token one in full, every token of every head),
ragged lengths around the 16-token chunk,
every state-dtype combination, zero-length sequences, B > 1, T = 0, lower_bound in
{-5, -2, -0.05, 0}, in-place state carry, the activation switches (pre-activated gate,
caller-normalised q/k, pre-activated beta) in all eight settings, whole-chain and segmented,
and long sequences run as two column halves.
"""
import numpy as np
import pytest

from gated_delta_rule_86_amd import workloads as W
from kda_testutil import (check_final, check_out, final_tensor, run_gpu, run_oracle, state_tensor,
                          to_device)

pytestmark = pytest.mark.gpu


def parity(w, what):
    o, f, _ = run_gpu(w)
    ro, rf = run_oracle(w)
    mx, rl = check_out(o, ro, what)
    msg = f"{what}: out max {mx:.2e} relL2 {rl:.2e}"
    if f is not None:
        msg += f" final relL2 {check_final(f, rf, w.final_dtype, what):.2e}"
    print(msg, flush=True)


@pytest.mark.parametrize("cfg", [0, 1, 2, 4])
def test_reference_workload(cfg):
    w = W.config(cfg)
    parity(w, w.name)


def test_long_context_workload():
    """B=1, T=2^20, H=8 (cut plan: pass A, transition runs, scan, pass B), compared in full: every output
    token of every head against the oracle run from the true initial state (streamed, the
    fp64 output is never stored), and the final state."""
    import os
    import torch
    import oracle
    w = W.config(3)
    out, fin, _ = run_gpu(w, keep_device=True)
    o_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    f = fin.cpu().numpy().astype(np.float64)
    del out, fin
    threads = min(w.H, len(os.sched_getaffinity(0)))
    stats, rf = oracle.kda_fwd_compare(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias,
                                       w.lower_bound, o_bits, w.initial_state, nthreads=threads)
    mx = float(stats[..., 0].max())
    rl = float(np.sqrt(stats[..., 1].sum() / stats[..., 2].sum()))
    per_head = np.sqrt(stats[..., 1] / stats[..., 2]).ravel()
    print(f"T=2^20 H=8 full: out max {mx:.2e} relL2 {rl:.2e} (per head {per_head.min():.2e}.."
          f"{per_head.max():.2e}); final relL2 {check_final(f, rf, 'fp32', 'T=2^20'):.2e}", flush=True)
    assert mx <= 2e-2 and rl <= 5e-3, (mx, rl)
    assert np.all(per_head <= 5e-3), per_head


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 33, 47, 64, 4097])
def test_lengths_around_chunks(T):
    parity(W.make(f"T{T}", 1, T, 2, seed=300 + T), f"T={T}")


@pytest.mark.parametrize("B,T,H,lengths", [(2, 100, 129, None), (1, 70, 256, None), (1, 0, 300, [33, 0, 50]),
                                          (1, 0, 200, [1100, 17])])
def test_many_heads(B, T, H, lengths):
    """More heads than the cut plan takes (128) and than CUs (256): whole chains, one
    workgroup per head and more workgroups than CUs; varlen with an empty sequence and with
    one long sequence."""
    w = W.make(f"heads{H}_{T}_{lengths}", B, T, H, lengths=lengths, seed=600 + H, state_dtype="fp32")
    parity(w, f"B={B} T={T} H={H} lengths={lengths}")


def test_batch_and_heads():
    parity(W.make("B3_T100_H3", 3, 100, 3, seed=301), "B=3 T=100 H=3")


@pytest.mark.parametrize("init,final", [("none", "none"), ("none", "fp32"), ("none", "bf16"),
                                        ("fp32", "fp32"), ("bf16", "bf16"), ("fp32", "none"),
                                        ("bf16", "none")])
def test_state_dtype_combinations(init, final):
    w = W.make(f"st_{init}_{final}", 2, 40, 2, seed=302, state_dtype=init if init != "none" else "none",
               with_initial=init != "none", final_dtype=final)
    parity(w, f"init={init} final={final}")


@pytest.mark.parametrize("lb", [-5.0, -2.0, -0.05, 0.0])
def test_lower_bounds(lb):
    parity(W.make(f"lb{lb}", 1, 300, 2, seed=303, lower_bound=lb), f"lb={lb}")


def test_varlen_with_empty_sequences():
    w = W.make("varlen_empty", 1, 0, 3, lengths=[0, 5, 0, 16, 33, 0, 1, 70], seed=304, state_dtype="bf16")
    parity(w, "varlen with empty sequences")


def test_varlen_fp32_many():
    L = np.random.default_rng(7).integers(0, 90, size=40)
    parity(W.make("varlen40", 1, 0, 2, lengths=L, seed=305), "varlen N=40")


def test_varlen_many_short_contiguous_runs():
    """More than 512 sequences: the whole-chain launch splits them into contiguous runs of
    about equal chunk count (above the snake-order limit)."""
    L = np.random.default_rng(8).integers(0, 40, size=600)
    parity(W.make("varlen600", 1, 0, 1, lengths=L, seed=309, state_dtype="bf16"), "varlen N=600")


def test_T_zero():
    w = W.make("T0", 2, 0, 2, seed=306)
    o, f, _ = run_gpu(w)
    assert o.size == 0
    assert np.array_equal(f, w.initial_state.astype(np.float64))


def test_scale_values():
    for sc in (0.3, 0.0, -1.5):
        parity(W.make(f"scale{sc}", 1, 50, 1, seed=307, scale=sc), f"scale={sc}")


def test_in_place_state_carry():
    import torch
    w = W.make("inplace", 1, 0, 2, lengths=[20, 37], seed=308)
    d = to_device(w)
    ro, rf = run_oracle(w)
    buf = d["h0"].clone()
    o, f, _ = run_gpu(w, d, h0=buf, final=buf)
    check_out(o, ro, "in-place")
    check_final(buf.cpu().numpy().astype(np.float64), rf, "fp32", "in-place")


def segments_of(B, T, H):
    """Workgroups per head of the cut plan (1: whole-chain plans); the host ABI tests check
    this replica against the library's workspace size."""
    from kda_testutil import cut_plan
    return cut_plan(B, T, H)


@pytest.mark.parametrize("B,T,H,init,final", [
    (1, 1100, 1, "fp32", "fp32"),
    (1, 1200, 2, "bf16", "bf16"),
    (2, 2000, 3, "none", "fp32"),
    (1, 5000, 4, "fp32", "none"),
    (3, 1100, 5, "fp32", "fp32"),
])
def test_segmented_chains(B, T, H, init, final):
    P = segments_of(B, T, H)
    assert P >= 2, (B, T, H, P)
    w = W.make(f"seg_B{B}_T{T}_H{H}", B, T, H, seed=310 + T, state_dtype=init if init != "none" else "none",
               with_initial=init != "none", final_dtype=final)
    parity(w, f"cut plan P={P}")


def test_segmented_in_place_state():
    w = W.make("seg_inplace", 1, 1100, 2, seed=311)
    assert segments_of(1, 1100, 2) >= 2
    d = to_device(w)
    ro, rf = run_oracle(w)
    buf = d["h0"].clone()
    o, f, _ = run_gpu(w, d, h0=buf, final=buf)
    check_out(o, ro, "segmented in-place")
    check_final(buf.cpu().numpy().astype(np.float64), rf, "fp32", "segmented in-place")


@pytest.mark.parametrize("flags", range(8))
def test_activation_switches(flags):
    """Each of the eight switch settings, on two chunk-crossing ragged sequences and a
    1-token one with an initial state (whole-chain launch)."""
    w = W.make(f"sw{flags}", 1, 0, 3, lengths=[45, 1, 130], seed=320 + flags, flags=flags,
               lower_bound=-3.0, state_dtype="fp32")
    parity(w, f"flags={flags}")


@pytest.mark.parametrize("flags", [0, 3, 6])
def test_activation_switches_segmented(flags):
    """Switches under the cut plan (pass A, transition runs, scan, pass B: the transition
    runs use the same gates; with l2norm or sigmoid off they never stop early)."""
    assert segments_of(1, 1500, 2) >= 2
    w = W.make(f"swseg{flags}", 1, 1500, 2, seed=330 + flags, flags=flags, state_dtype="bf16")
    parity(w, f"cut plan flags={flags}")


def test_preactivated_gate_held_to_range():
    """Pre-activated log-decays outside [lower_bound, 0] are held to the range on both sides
    (the oracle does the same); lower_bound 0 turns every decay off."""
    from gated_delta_rule_86_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits
    for lb in (-2.0, 0.0):
        w = W.make(f"clamp{lb}", 1, 90, 2, seed=340, flags=0, lower_bound=lb)
        g = bf16_bits_to_f32(w.g).copy()
        g[0, ::3, 0, :64] = -4.5
        g[0, 1::5, 1, 30:] = 0.75
        w.g = f32_to_bf16_bits(g)
        parity(w, f"pre-activated gate held to [{lb}, 0]")


def plan_has_halves(w):
    """True when the chunk table runs some sequence of w as two column halves."""
    import torch
    from gated_delta_rule_86_amd import kda
    from kda_testutil import torch_dev
    N = len(w.cu_seqlens) - 1
    up = lambda x: -(-x // 256) * 256
    ws = torch.zeros(kda.workspace_size(1, w.T, w.H, N, True), dtype=torch.uint8, device=torch_dev())
    kda.chunk_table(torch.from_numpy(w.cu_seqlens).to(torch_dev()), 1, w.T, w.H, workspace=ws)
    off = 256 + 2 * up(8 * N) + up(8 * (N + 1))
    off_units = off + up(8 * 257)
    units = ws[off_units:off_units + 4 * 2 * N].cpu().numpy().view(np.int32)
    return bool(np.any((units & 3) != 0))  # entries past the list stay zero (whole)


@pytest.mark.parametrize("H,lens,sd,flags", [
    (32, [600, 40, 30, 50, 20, 10, 70, 25], "bf16", 7),
    (16, [900, 33, 17], "fp32", 7),
    (32, [1000, 517, 3, 200], "none", 7),
    (16, [700, 20], "fp32", 0),
    (24, [500, 30, 70], "fp32", 7),     # 10 workgroups per head
])
def test_column_halves(H, lens, sd, flags):
    """Few long sequences on heads with few workgroups each: the longest run as two units
    of 64 value columns (the consumers take 16 columns each), whole-chain launch."""
    w = W.make(f"halves_H{H}", 1, 0, H, lengths=lens, seed=350 + H + len(lens), flags=flags,
               state_dtype=sd, with_initial=sd != "none", final_dtype="fp32" if sd == "none" else None)
    assert plan_has_halves(w)
    parity(w, f"column halves H={H} flags={flags}")


def test_column_halves_in_place_state():
    w = W.make("halves_inplace", 1, 0, 32, lengths=[640, 30, 45], seed=360)
    assert plan_has_halves(w)
    d = to_device(w)
    ro, rf = run_oracle(w)
    buf = d["h0"].clone()
    o, f, _ = run_gpu(w, d, h0=buf, final=buf)
    check_out(o, ro, "column halves in-place")
    check_final(buf.cpu().numpy().astype(np.float64), rf, "fp32", "column halves in-place")
