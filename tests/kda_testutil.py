"""Helpers shared by the GPU tests: host->device marshalling, one kda_fwd call through
the C ABI (via the thin binding), oracle reference, and the acceptance metrics."""
import numpy as np

import oracle
from gated_delta_rule_86_amd import kda
from oracle.chunked import bf16_bits_to_f64

# acceptance bars for floating point (fp64 oracle as the reference)
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
FINAL_REL_L2 = {"fp32": 1e-3, "bf16": 1e-2}


def torch_dev():
    import torch
    return torch.device("cuda:0")


def bf16_tensor(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch_dev())


def state_tensor(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return bf16_tensor(a)
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dev())


def to_device(w):
    import torch
    d = {k: bf16_tensor(getattr(w, k)) for k in ("q", "k", "v", "g", "beta")}
    gate_in = bool(w.flags & 1)  # A_log / dt_bias feed only the in-pass gate
    d["A_log"] = torch.from_numpy(w.A_log).to(torch_dev()) if gate_in else None
    d["dt_bias"] = torch.from_numpy(w.dt_bias).to(torch_dev()) if gate_in else None
    d["h0"] = state_tensor(w.initial_state)
    d["cu"] = None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens).to(torch_dev())
    return d


def final_tensor(w, fill=None):
    import torch
    if w.final_dtype == "none":
        return None
    dt = torch.float32 if w.final_dtype == "fp32" else torch.bfloat16
    t = torch.empty((w.N, w.H, 128, 128), dtype=dt, device=torch_dev())
    if fill is not None:
        t.fill_(fill)
    return t


def run_gpu(w, d=None, out_fill=None, final_fill=None, workspace=None, h0=None, final=None,
            keep_device=False, recurrent=False):
    """One kda_fwd call.  Returns (out, final, workspace) -- host float64 arrays unless keep_device."""
    import torch
    if d is None:
        d = to_device(w)
    out = torch.empty_like(d["q"])
    if out_fill is not None:
        out.fill_(out_fill)
    fin = final if final is not None else final_tensor(w, final_fill)
    h0t = d["h0"] if h0 is None else h0
    entry = kda.fwd_recurrent if recurrent else kda.fwd
    ws = entry(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, out, d["A_log"], d["dt_bias"],
                 w.lower_bound, h0t, fin, d["cu"], workspace=workspace,
                 use_gate_in_kernel=bool(w.flags & 1), use_qk_l2norm_in_kernel=bool(w.flags & 2),
                 use_beta_sigmoid_in_kernel=bool(w.flags & 4))
    torch.cuda.synchronize()
    if keep_device:
        return out, fin, ws
    o = out.float().cpu().numpy().astype(np.float64)
    f = None if fin is None else fin.float().cpu().numpy().astype(np.float64)
    return o, f, ws


def run_oracle(w, heads=None, initial_state="default", nthreads=0):
    h0 = w.initial_state if isinstance(initial_state, str) else initial_state
    gate_in = bool(w.flags & 1)
    return oracle.kda_fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log if gate_in else None,
                          w.dt_bias if gate_in else None, w.lower_bound, h0, cu_seqlens=w.cu_seqlens,
                          heads=heads, nthreads=nthreads, flags=w.flags)


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def check_out(o, ro, what=""):
    mx = float(np.abs(o - ro).max(initial=0.0))
    rl = rel_l2(o, ro) if o.size else 0.0
    assert mx <= OUT_MAX_ABS and rl <= OUT_REL_L2, f"{what} out: max|err| {mx:.3e} relL2 {rl:.3e}"
    return mx, rl


def check_final(f, rf, dtype, what=""):
    rl = rel_l2(f, rf)
    assert rl <= FINAL_REL_L2[dtype], f"{what} final ({dtype}): relL2 {rl:.3e}"
    return rl


def bf16_round_f64(x):
    """Round float64 values to bf16 (via fp32) and return them as float64."""
    from gated_delta_rule_86_amd.workloads import f32_to_bf16_bits
    return bf16_bits_to_f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


# ---- segment plan of few long equal-length chains (replica of the host plan) ----
PLAN_CUS = 256


SEG_MIN_CHUNKS = 16       # shortest segment the plan makes
TRUNC_TAU = 2.0 ** -50    # entry bound at which a segment's transition run stops
TRUNC_M = 4096.0          # Frobenius bound on a segment's start state for dropping its share


def segment_plan(chains, nch):
    """(G, L): segments per chain and chunks per segment (the last one shorter) that the
    forward pass picks for `chains` equal-length chains of `nch` chunks (G = 1: whole
    chains).  G fills the 256 CUs with one round of pass A units (segments of every chain)
    of at least 16 chunks, with no empty segment."""
    cdiv = lambda a, b: -(-a // b)
    if chains <= 0 or chains > PLAN_CUS // 2:
        return 1, nch
    G = min(PLAN_CUS // chains, nch // SEG_MIN_CHUNKS)
    while G >= 2 and (G - 1) * cdiv(nch, G) >= nch:
        G -= 1
    if G < 2:
        return 1, nch
    return G, cdiv(nch, G)


def segment_bounds(G, L, nch):
    """First chunk of each segment 0 .. G-1, and nch at the end: G + 1 entries."""
    return [min(g * L, nch) for g in range(G)] + [nch]


def table_bytes(N):
    """Workspace bytes before the segment states: header, per-sequence tables, the
    workgroup-run table and the unit list."""
    up = lambda x: -(-x // 256) * 256
    return 256 + up(8 * N) + up(8 * N) + up(8 * (N + 1)) + up(8 * 257) + up(8 * N)


def segment_states(ws, B, H, G):
    """The fp32 segment states S, F, P of a segmented call, read back from its workspace:
    three float64 arrays [B, H, G, 128, 128] (V-major).  S_g (g >= 2) is written only where
    the scan computed it; F_g, P_g (g >= 1) hold the runs from zero and from the identity
    (P_g only where its run went the whole segment)."""
    n = B * H * G * 128 * 128
    off = table_bytes(B)
    raw = ws[off:off + 3 * 4 * n].cpu().numpy().view(np.float32).astype(np.float64)
    S, F, P = (raw[i * n:(i + 1) * n].reshape(B, H, G, 128, 128) for i in range(3))
    return S, F, P


def segment_aux(ws, B, H, G):
    """Per segment of a segmented call: z (chunks its transition run took before it
    stopped, -1: the whole segment), drop (1 where the scan dropped the segment's start
    state's share of the next one) and the squared norms of pass A's end states (per
    consumer wavefront): int64 [B, H, G], int64 [B, H, G], float64 [B, H, G, 4]."""
    units = B * H * G
    off = table_bytes(B) + 3 * 4 * units * 128 * 128
    raw = ws[off:off + units * 24].cpu().numpy()
    z = raw[:4 * units].view(np.int32).astype(np.int64).reshape(B, H, G)
    drop = raw[4 * units:8 * units].view(np.int32).astype(np.int64).reshape(B, H, G)
    nrm = raw[8 * units:24 * units].view(np.float32).astype(np.float64).reshape(B, H, G, 4)
    return z, drop, nrm
