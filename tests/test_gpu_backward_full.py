"""Backward parity at the full sizes of the workloads the backward bench times (B=2 T=4096
H=16 fp32 state; varlen N=8 up to 8192 tokens H=32 bf16 state, lower_bound -2; varlen N=256
up to 512 tokens H=32 fp32 state; B=1 T=2^20 H=8 fp32 state, in windows), in the launch
configuration ``bench.py --backward`` uses: one kda_bwd call over the whole batch with a
random dL/dout and dL/dfinal_state.

The gradients of one chain (sequence, head) depend on that chain's inputs alone, so sampled
chains -- the longest sequence among them -- are compared with the fp64 backward oracle run
on the chain by itself (the inputs sliced out of the batch); bars as in test_gpu_backward.py:
relative L2 1e-4 and max |err| 1e-4 of the largest magnitude on every sampled gradient.
dA_log and dt_bias sum over every chain; they are checked against their definition in terms
of the gate (x = e^A_log (g + dt_bias)): dL/ddt_bias[h, c] = sum_t dL/dg[t, h, c] and
dL/dA_log[h] = sum_{t, c} dL/dg[t, h, c] (g[t, h, c] + dt_bias[h, c]), summed in fp64 from the
GPU's dg (whose values the sampled chains pin), each entry within 1e-4 of the sum of its
terms' magnitudes.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_86_amd import kda
from gated_delta_rule_86_amd import workloads as W
from kda_testutil import bf16_tensor, rel_l2, state_tensor, torch_dev

pytestmark = pytest.mark.gpu
REL = 1e-4


def _check(got, exp, what):
    rl = rel_l2(got, exp)
    mx = float(np.abs(got - exp).max(initial=0.0))
    scale = float(np.abs(exp).max(initial=0.0))
    assert np.isfinite(got).all(), what
    assert rl <= REL and mx <= REL * max(scale, 1e-30), (what, rl, mx, scale)
    return rl


@pytest.mark.parametrize("wl,picks", [
    (1, [(0, 0), (1, 15)]),
    (2, [("longest", 5), ("shortest", 31), (3, 17)]),
    (4, [(0, 0), (128, 9), (255, 31), ("longest", 20)]),
])
def test_backward_full_size_sampled_chains(wl, picks):
    import torch
    w = W.config(wl)
    dev = torch_dev()
    rng = np.random.default_rng(900 + wl)
    dout = W.f32_to_bf16_bits(rng.standard_normal((w.B, w.T, w.H, 128), dtype=np.float32))
    dht = rng.standard_normal((w.N, w.H, 128, 128), dtype=np.float32)
    d = {n: bf16_tensor(getattr(w, n)) for n in ("q", "k", "v", "g", "beta")}
    A_log = torch.from_numpy(w.A_log).to(dev)
    dt_bias = torch.from_numpy(w.dt_bias).to(dev)
    cu = None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens).to(dev)
    print(f"case {w.name}: kda_bwd over {w.head_tokens} head-tokens", flush=True)
    r = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, A_log, dt_bias, w.lower_bound,
                bf16_tensor(dout), state_tensor(w.initial_state), torch.from_numpy(dht).to(dev), cu)
    torch.cuda.synchronize()
    lens = w.lengths
    starts = np.zeros(w.N, dtype=np.int64) if w.cu_seqlens is None else w.cu_seqlens[:-1]
    for n, h in picks:
        if n == "longest":
            n = int(np.argmax(lens))
        elif n == "shortest":
            n = int(np.argmin(lens))
        L = int(lens[n])
        row, t0 = (n, 0) if w.cu_seqlens is None else (0, int(starts[n]))
        sl = lambda a: np.ascontiguousarray(a[row:row + 1, t0:t0 + L, h:h + 1])
        h0 = None if w.initial_state is None else np.ascontiguousarray(w.initial_state[n:n + 1, h:h + 1])
        ref = oracle.kda_bwd(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta), w.scale,
                             np.ascontiguousarray(w.A_log[h:h + 1]), np.ascontiguousarray(w.dt_bias[h:h + 1]),
                             w.lower_bound, sl(dout), h0, np.ascontiguousarray(dht[n:n + 1, h:h + 1]),
                             flags=w.flags)
        msg = []
        for name, key in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg")):
            got = r[name][row, t0:t0 + L, h].double().cpu().numpy()
            rl = _check(got, ref[key][0, :, 0], f"{w.name} chain ({n}, {h}) {name}")
            msg.append(f"{name} {rl:.1e}")
        got = r["dbeta"][row, t0:t0 + L, h].double().cpu().numpy()
        rl = _check(got, ref["dbeta"][0, :, 0], f"{w.name} chain ({n}, {h}) dbeta")
        msg.append(f"dbeta {rl:.1e}")
        got = r["dinitial_state"][n, h].double().cpu().numpy()
        rl = _check(got, ref["dh0"][0, 0], f"{w.name} chain ({n}, {h}) dinitial_state")
        msg.append(f"dh0 {rl:.1e}")
        print(f"{w.name} chain (seq {n}, {L} tokens, head {h}): relL2 " + " ".join(msg), flush=True)
    # dt_bias and A_log gradients: their definition from the GPU's dg, summed in fp64; each entry
    # within 1e-4 of the sum of its terms' magnitudes (fp32 summation: runs of a few hundred
    # terms per thread, n eps ~ 3e-5, then 128 partial sums in a fixed order)
    dg = r["dg"].double()
    x = d["g"].double() + dt_bias.double()[None, None]
    for name, exp, mag in (("ddt_bias", dg.sum(dim=(0, 1)), dg.abs().sum(dim=(0, 1))),
                           ("dA_log", (dg * x).sum(dim=(0, 1, 3)), (dg * x).abs().sum(dim=(0, 1, 3)))):
        got = r[name].double()
        err = (got - exp).abs()
        assert bool((err <= 1e-4 * mag).all()), (w.name, name, float((err / mag).max()))
        print(f"{w.name} {name}: max |err| / sum |terms| = {float((err / mag).max()):.1e}", flush=True)


def test_backward_long_context_windows():
    """The 2^20-token workload (B=1 T=1,048,576 H=8, fp32 state, lower_bound -5), one kda_bwd
    call as ``bench.py --backward --workload 3`` makes it: the backward walks run on the cut
    plan (24 pieces of 2,731 chunks per chain and direction, the last one 2,723).  A 1M-token chain is beyond the
    fp64 oracle, so windows are compared: the oracle runs on tokens [t0 - M, t1 + M) of a chain
    from a zero state (the true initial state where t0 - M <= 0) and with a zero dL/dS at its
    end (the true dL/dfinal_state where t1 + M reaches T); with this gate every token scales
    the carried state by at most e^(-5 sigmoid(x)), so over M = 512 tokens the cut-off parts
    fall far below fp64 rounding, and the gradients of [t0, t1) must match as for a whole
    chain.  Windows: the first tokens (with dL/dinitial_state), one across a cut between
    pieces, one inside a piece, and the last tokens."""
    import torch
    w = W.config(3)
    dev = torch_dev()
    rng = np.random.default_rng(903)
    dout = W.f32_to_bf16_bits(rng.standard_normal((w.B, w.T, w.H, 128), dtype=np.float32))
    dht = rng.standard_normal((w.N, w.H, 128, 128), dtype=np.float32)
    d = {n: bf16_tensor(getattr(w, n)) for n in ("q", "k", "v", "g", "beta")}
    A_log = torch.from_numpy(w.A_log).to(dev)
    dt_bias = torch.from_numpy(w.dt_bias).to(dev)
    print(f"case {w.name}: kda_bwd over {w.head_tokens} head-tokens", flush=True)
    r = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, A_log, dt_bias, w.lower_bound,
                bf16_tensor(dout), state_tensor(w.initial_state), torch.from_numpy(dht).to(dev))
    torch.cuda.synchronize()
    T, M, piece = w.T, 512, 2731 * 16
    windows = [(0, 1024, 0), (3 * piece - 600, 3 * piece + 600, 5), (20 * piece + 4000, 20 * piece + 5000, 7),
               (T - 1024, T, 3)]
    for t0, t1, h in windows:
        a0, a1 = max(0, t0 - M), min(T, t1 + M)
        sl = lambda x: np.ascontiguousarray(x[0:1, a0:a1, h:h + 1])
        h0 = np.ascontiguousarray(w.initial_state[0:1, h:h + 1]) if a0 == 0 else None
        dh = np.ascontiguousarray(dht[0:1, h:h + 1]) if a1 == T else None
        ref = oracle.kda_bwd(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta), w.scale,
                             np.ascontiguousarray(w.A_log[h:h + 1]), np.ascontiguousarray(w.dt_bias[h:h + 1]),
                             w.lower_bound, sl(dout), h0, dh, flags=w.flags)
        msg = []
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            got = r[name][0, t0:t1, h].double().cpu().numpy()
            rl = _check(got, ref[name][0, t0 - a0:t1 - a0, 0], f"window [{t0}, {t1}) head {h} {name}")
            msg.append(f"{name} {rl:.1e}")
        if a0 == 0:
            got = r["dinitial_state"][0, h].double().cpu().numpy()
            msg.append(f"dh0 {_check(got, ref['dh0'][0, 0], f'head {h} dinitial_state'):.1e}")
        print(f"{w.name} window [{t0}, {t1}) head {h}: relL2 " + " ".join(msg), flush=True)
    dg = r["dg"].double()
    x = d["g"].double() + dt_bias.double()[None, None]
    for name, exp, mag in (("ddt_bias", dg.sum(dim=(0, 1)), dg.abs().sum(dim=(0, 1))),
                           ("dA_log", (dg * x).sum(dim=(0, 1, 3)), (dg * x).abs().sum(dim=(0, 1, 3)))):
        got = r[name].double()
        err = (got - exp).abs()
        assert bool((err <= 1e-4 * mag).all()), (w.name, name, float((err / mag).max()))
        print(f"{w.name} {name}: max |err| / sum |terms| = {float((err / mag).max()):.1e}", flush=True)
