"""The stage-timed entry points, kda_fwd_timed and kda_fwd_recurrent_timed, on the GPU.

They run the same launches as kda_fwd / kda_fwd_recurrent with HIP events recorded between
them, so on the same inputs their out and final_state are bitwise those of the untimed
calls.  The events are recorded in order on the launch stream: every interval between
consecutive events is non-negative and the intervals add up to the first-to-last one.
Cases: a whole-chain plan, the cut plan (on a non-default stream), and the recurrent
evaluation of a decode step and of a short varlen batch.
"""
import ctypes

import pytest

from gated_delta_rule_86_amd import kda
from gated_delta_rule_86_amd import workloads as W
from kda_testutil import cut_plan, final_tensor, to_device

pytestmark = pytest.mark.gpu


def _hip():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def _call(w, d, recurrent, events=None, stream=None):
    import torch
    out = torch.empty_like(d["q"]).fill_(7.0)
    fin = final_tensor(w, fill=7.0)
    if stream is not None:  # the inputs and the fills above were queued on the current stream
        stream.wait_stream(torch.cuda.current_stream())
    entry = kda.fwd_recurrent if recurrent else kda.fwd
    entry(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, out, d["A_log"], d["dt_bias"],
          w.lower_bound, d["h0"], fin, d["cu"], stream=stream, stage_events=events)
    (stream or torch.cuda.current_stream()).synchronize()
    return out, fin


@pytest.mark.parametrize("case", ["whole_chain", "cut_plan", "recurrent_decode", "recurrent_varlen"])
def test_timed_matches_untimed(case):
    import torch
    if case == "whole_chain":
        w, recurrent = W.make("timed_whole", 2, 333, 3, seed=811, state_dtype="fp32"), False
        assert cut_plan(w.B, w.T, w.H) == 1
    elif case == "cut_plan":
        w, recurrent = W.make("timed_cut", 1, 6000, 4, seed=812, lower_bound=-2.0), False
        assert cut_plan(w.B, w.T, w.H) > 1
    elif case == "recurrent_decode":
        w, recurrent = W.make("timed_decode", 48, 1, 4, seed=813, state_dtype="fp32"), True
    else:
        w, recurrent = W.make("timed_rvar", 1, 0, 3, lengths=[5, 0, 17, 1], seed=814), True
    n_ev = 3 if recurrent else 5
    print(f"case {case}: B={w.B} T={w.T} H={w.H} N={w.N}, {n_ev} events", flush=True)
    d = to_device(w)
    hip = _hip()
    evs = []
    for _ in range(n_ev):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    try:
        stream = torch.cuda.Stream() if case == "cut_plan" else None
        o_ref, f_ref = _call(w, d, recurrent)
        o, f = _call(w, d, recurrent, events=evs, stream=stream)
        assert torch.equal(o, o_ref)
        assert torch.equal(f, f_ref)
        ms = ctypes.c_float()
        iv = []
        for j in range(n_ev - 1):
            assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[j], evs[j + 1]) == 0
            iv.append(ms.value)
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[-1]) == 0
        total = ms.value
        assert all(x >= 0.0 for x in iv), iv
        assert abs(sum(iv) - total) <= 1e-3 + 1e-3 * total, (iv, total)
        print(f"case {case}: intervals (ms) {[round(x, 4) for x in iv]}, total {total:.4f}", flush=True)
    finally:
        for e in evs:
            hip.hipEventDestroy(e)
