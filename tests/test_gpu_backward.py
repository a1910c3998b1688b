"""GPU parity of the backward pass (kda_bwd, through the C ABI) against the fp64 backward
oracle (oracle/kda_bwd_ref.c) on the same seeded inputs.

Tolerance: every gradient tensor within relative L2 <= 1e-4 of the oracle, and its max
|err| <= 1e-4 of the oracle's largest magnitude.  The kernels work in fp32 end to end (the
inputs and dL/dout are bf16 on both sides, so both see the same values); fp32 rounding
of the carried state gradient over a few thousand tokens stays near 1e-6 relative (measured
1e-7 to 5e-6), and the bar leaves an order of magnitude above that.  Covers batch rows, varlen with empty
and ragged sequences, bf16/fp32/no initial state, a final-state gradient, weak decay
(lower_bound 0), every activation switch setting, and T = 0.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_86_amd import kda
from gated_delta_rule_86_amd import workloads as W
from kda_testutil import bf16_tensor, bwd_piece_len, rel_l2, state_tensor, torch_dev

pytestmark = pytest.mark.gpu
REL = 1e-4


def grads_parity(w, seed, with_dht, what):
    import torch
    rng = np.random.default_rng(seed)
    dout = W.f32_to_bf16_bits(rng.normal(size=(w.B, w.T, w.H, 128)).astype(np.float32))
    dht = rng.normal(size=(w.N, w.H, 128, 128)).astype(np.float32) if with_dht else None
    gate_in = bool(w.flags & 1)
    dev = torch_dev()
    d = {n: bf16_tensor(getattr(w, n)) for n in ("q", "k", "v", "g", "beta")}
    A_log = torch.from_numpy(w.A_log).to(dev) if gate_in else None
    dt_bias = torch.from_numpy(w.dt_bias).to(dev) if gate_in else None
    cu = None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens).to(dev)
    r = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, A_log, dt_bias, w.lower_bound,
                bf16_tensor(dout), state_tensor(w.initial_state),
                None if dht is None else torch.from_numpy(dht).to(dev), cu,
                use_gate_in_kernel=gate_in, use_qk_l2norm_in_kernel=bool(w.flags & 2),
                use_beta_sigmoid_in_kernel=bool(w.flags & 4))
    torch.cuda.synchronize()
    ref = oracle.kda_bwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log if gate_in else None,
                         w.dt_bias if gate_in else None, w.lower_bound, dout, w.initial_state, dht,
                         cu_seqlens=w.cu_seqlens, flags=w.flags)
    pairs = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
             ("dinitial_state", "dh0")]
    if gate_in:
        pairs += [("dA_log", "dA_log"), ("ddt_bias", "ddt_bias")]
    msg = []
    for gk, rk in pairs:
        got = r[gk].cpu().numpy().astype(np.float64)
        exp = ref[rk]
        if exp.size == 0:
            continue
        rl = rel_l2(got, exp)
        mx = float(np.abs(got - exp).max())
        scale_ = float(np.abs(exp).max())
        msg.append(f"{gk} {rl:.1e}")
        assert np.isfinite(got).all(), (what, gk)
        assert rl <= REL and mx <= REL * max(scale_, 1e-30), (what, gk, rl, mx, scale_)
    print(f"{what}: relL2 " + " ".join(msg), flush=True)


def test_backward_batch_rows():
    w = W.make("bwd_batch", 2, 50, 2, seed=700, state_dtype="fp32")
    grads_parity(w, 1, True, "B=2 T=50 H=2 fp32 state, dL/dfinal")


def test_backward_varlen_ragged_and_empty():
    w = W.make("bwd_varlen", 1, 0, 3, lengths=[37, 0, 300, 16, 5], seed=701, state_dtype="bf16")
    grads_parity(w, 2, False, "varlen 37/0/300/16/5 H=3 bf16 state")


def test_backward_no_initial_state():
    w = W.make("bwd_noh0", 1, 70, 2, seed=702, state_dtype="none", with_initial=False)
    grads_parity(w, 3, True, "T=70 no initial state")


@pytest.mark.parametrize("lb", [0.0, -0.05, -5.0])
def test_backward_lower_bounds(lb):
    w = W.make(f"bwd_lb{lb}", 1, 200, 2, seed=703, lower_bound=lb, state_dtype="fp32")
    grads_parity(w, 4, True, f"T=200 lb={lb}")


@pytest.mark.parametrize("flags", [0, 1, 2, 3, 4, 5, 6])
def test_backward_activation_switches(flags):
    w = W.make(f"bwd_sw{flags}", 1, 0, 2, lengths=[45, 1, 33], seed=710 + flags, flags=flags,
               lower_bound=-3.0, state_dtype="fp32")
    grads_parity(w, 5 + flags, True, f"flags={flags}")


@pytest.mark.parametrize("B,H", [(2, 16), (4, 16), (5, 13)])
def test_backward_chain_splits(B, H):
    """2 B H (chain, role) units: 64 and 128 (the chain kernel splits each unit's channels over
    two waves, up to 128 units), 130 (no split)."""
    w = W.make(f"bwd_split{B}x{H}", B, 40, H, seed=720 + B, state_dtype="fp32")
    grads_parity(w, 20 + B, True, f"B={B} T=40 H={H}: {2 * B * H} chain units")


def test_backward_many_heads():
    """160 heads: 320 chain units (the two-workgroup split of the chain kernel), more chunk
    workgroups than CUs."""
    w = W.make("bwd_heads160", 1, 0, 160, lengths=[50, 20], seed=707, state_dtype="fp32")
    grads_parity(w, 13, True, "varlen 50/20 H=160")


def test_backward_long_chains():
    """Two chains of 2100 tokens (132 chunks of checkpoints each) with weak decay."""
    w = W.make("bwd_long", 1, 2100, 2, seed=705, lower_bound=-0.05, state_dtype="fp32")
    grads_parity(w, 9, True, "T=2100 H=2 lb=-0.05")


def _pieces(w, L):
    lens = np.diff(w.cu_seqlens) if w.cu_seqlens is not None else [w.T] * w.B
    return [max(1, -(-(-(-int(n) // 16)) // L)) for n in lens]


@pytest.mark.parametrize("lb", [0.0, -0.05, -2.0, -5.0])
def test_backward_cut_plan_lower_bounds(lb):
    """One long sequence per row cut into pieces (pass A, transition runs, scan, pass B):
    without decay no transition run stops and the scan composes every piece; with a strong
    gate the runs stop within a few chunks and pass B reruns only those."""
    w = W.make(f"bwd_cut_lb{lb}", 1, 2048, 2, seed=730, lower_bound=lb, state_dtype="fp32")
    L = bwd_piece_len(w.B, w.T, w.H)
    assert L > 0 and _pieces(w, L) == [16]
    grads_parity(w, 30, True, f"cut plan T=2048 H=2 lb={lb} (16 pieces)")


def test_backward_cut_plan_batch_rows():
    """Two batch rows of 1100 tokens (9 pieces each, the last one 5 chunks), bf16 initial
    state, three heads."""
    w = W.make("bwd_cut_rows", 2, 1100, 3, seed=731, state_dtype="bf16")
    L = bwd_piece_len(w.B, w.T, w.H)
    assert L == 8 and _pieces(w, L) == [9, 9]
    grads_parity(w, 31, True, "cut plan B=2 T=1100 H=3")


@pytest.mark.parametrize("flags,lb", [(7, -0.05), (1, -2.0)])
def test_backward_cut_plan_varlen(flags, lb):
    """Varlen batch on the cut plan with an empty, a one-token and a two-chunk sequence among
    two long ones; weak decay (scan through every piece), and the l2norm and sigmoid
    switched off (no transition run may stop: the bound needs them)."""
    w = W.make(f"bwd_cut_var{flags}", 1, 0, 2, lengths=[3500, 0, 17, 2600, 1], seed=732 + flags,
               lower_bound=lb, flags=flags, state_dtype="fp32")
    L = bwd_piece_len(w.B, w.T, w.H, w.N, True)
    assert L == 8 and _pieces(w, L) == [28, 1, 1, 21, 1]
    grads_parity(w, 32 + flags, True, f"cut plan varlen flags={flags} lb={lb}")


def test_backward_cut_plan_short_walks():
    """Sequences of two pieces (pass B joins them without a scan step) and of three (one scan
    step) beside a long one and an empty one, moderate decay."""
    w = W.make("bwd_cut_short", 1, 0, 2, lengths=[4000, 200, 300, 0], seed=736, lower_bound=-0.5,
               state_dtype="bf16")
    L = bwd_piece_len(w.B, w.T, w.H, w.N, True)
    assert L == 8 and _pieces(w, L) == [32, 2, 3, 1]
    grads_parity(w, 36, True, "cut plan varlen, walks of 32 / 2 / 3 / 1 pieces")


def test_backward_cut_plan_no_states():
    """Cut plan without an initial state or a final-state gradient (both chains start from
    zero)."""
    w = W.make("bwd_cut_none", 1, 1600, 2, seed=733, state_dtype="none", with_initial=False)
    assert bwd_piece_len(w.B, w.T, w.H) > 0
    grads_parity(w, 34, False, "cut plan T=1600 H=2, no states")


def test_backward_T_zero():
    import torch
    w = W.make("bwd_T0", 2, 0, 2, seed=704)
    dev = torch_dev()
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)
    dht = torch.randn(2, 2, 128, 128, device=dev)
    r = kda.bwd(e(2, 0, 2, 128), e(2, 0, 2, 128), e(2, 0, 2, 128), e(2, 0, 2, 128), e(2, 0, 2),
                w.scale, torch.from_numpy(w.A_log).to(dev), torch.from_numpy(w.dt_bias).to(dev),
                w.lower_bound, e(2, 0, 2, 128), state_tensor(w.initial_state), dht)
    torch.cuda.synchronize()
    assert torch.equal(r["dinitial_state"], dht)      # nothing happens between the two states
    assert not torch.any(r["dA_log"]) and not torch.any(r["ddt_bias"])


def test_backward_invalid_cu_seqlens():
    """cu_seqlens that decreases (found on the device): every sequence is empty, the status
    word reports it, dA_log and dt_bias are zero and dL/dinitial_state = dL/dfinal_state."""
    import torch
    w = W.make("bwd_bad_cu", 1, 0, 2, lengths=[40, 0, 70], seed=706, state_dtype="fp32")
    dev = torch_dev()
    rng = np.random.default_rng(12)
    dout = W.f32_to_bf16_bits(rng.normal(size=(w.B, w.T, w.H, 128)).astype(np.float32))
    dht = torch.randn(w.N, w.H, 128, 128, device=dev)
    d = {n: bf16_tensor(getattr(w, n)) for n in ("q", "k", "v", "g", "beta")}
    cu = w.cu_seqlens.copy()
    cu[1] = cu[2] + 1  # 41 > 40: decreasing
    r = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, torch.from_numpy(w.A_log).to(dev),
                torch.from_numpy(w.dt_bias).to(dev), w.lower_bound, bf16_tensor(dout),
                state_tensor(w.initial_state), dht, torch.from_numpy(cu).to(dev))
    torch.cuda.synchronize()
    assert kda.device_status(r["workspace"]) == 2
    assert not torch.any(r["dA_log"]) and not torch.any(r["ddt_bias"])
    assert torch.equal(r["dinitial_state"], dht)


@pytest.mark.parametrize("case", ["whole", "cut"])
def test_backward_deterministic_and_workspace_independent(case):
    """Two kda_bwd calls give bitwise identical gradients (fixed summation orders, no atomics),
    also when the second one gets a workspace pre-filled with garbage: every per-chunk state,
    operand and row region it reads was written by the same call -- with whole-chain walks,
    and on the cut plan (piece table, start states, F, Phi, norms and stop counts)."""
    import torch
    if case == "whole":
        w = W.make("bwd_det", 1, 0, 3, lengths=[333, 17, 0, 120], seed=708, state_dtype="fp32")
        assert bwd_piece_len(w.B, w.T, w.H, w.N, True) == 0
    else:
        w = W.make("bwd_det_cut", 1, 0, 2, lengths=[3000, 0, 1500, 40], seed=709, lower_bound=-1.0,
                   state_dtype="fp32")
        assert bwd_piece_len(w.B, w.T, w.H, w.N, True) > 0
    dev = torch_dev()
    rng = np.random.default_rng(14)
    dout = bf16_tensor(W.f32_to_bf16_bits(rng.normal(size=(w.B, w.T, w.H, 128)).astype(np.float32)))
    dht = torch.randn(w.N, w.H, 128, 128, device=dev)
    d = {n: bf16_tensor(getattr(w, n)) for n in ("q", "k", "v", "g", "beta")}
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, torch.from_numpy(w.A_log).to(dev),
            torch.from_numpy(w.dt_bias).to(dev), w.lower_bound, dout, state_tensor(w.initial_state), dht,
            torch.from_numpy(w.cu_seqlens).to(dev))
    r1 = kda.bwd(*args)
    ws = r1["workspace"]
    r1 = {k: v.clone() for k, v in r1.items() if k != "workspace"}
    ws.fill_(0xA5)
    r2 = kda.bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    for k, v in r1.items():
        assert torch.equal(v, r2[k]), k
