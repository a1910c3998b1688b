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


# ---- cut plan (replica of the host plan and of the chunk table's cuts) ----
PLAN_CUS = 256
SEG_MIN_CHUNKS = 16   # shortest run of the cut plan
CUT_MIN_AVG = 64      # average chunks per sequence for the cut plan
SNAP_CHUNKS = 8
TRUNC_REL = 2.0 ** -37


def cut_plan(B, T, H, N=0, varlen=False):
    """Workgroups per head of the cut plan for these sizes, 1 for the whole-chain plans."""
    if H < 1 or H > PLAN_CUS // 2:
        return 1
    nseq = N if varlen else B
    C = -(-T // 16) if varlen else B * -(-T // 16)
    if nseq < 1 or C < nseq * CUT_MIN_AVG:
        return 1
    P = min(PLAN_CUS // H, C // SEG_MIN_CHUNKS)
    return P if P >= 2 else 1


# ---- backward cut plan (replica of the host decision) ----
BWD_CUT_MIN_AVG = 64   # average chunks per sequence
BWD_PIECE_MIN = 8      # chunks per piece, at least
BWD_TARGET_WGS = 768   # pass A workgroups aimed at


def bwd_piece_len(B, T, H, N=0, varlen=False):
    """Chunks per piece of the backward cut plan for these sizes, 0 for whole chains."""
    nseq = N if varlen else B
    chunks = -(-T // 16) + N if varlen else B * -(-T // 16)
    if nseq < 1 or H < 1 or chunks < nseq * BWD_CUT_MIN_AVG:
        return 0
    L = max(BWD_PIECE_MIN, -(-(chunks * H * 4) // BWD_TARGET_WGS))
    return L if chunks >= 2 * L * nseq else 0


def expected_cuts(seq_off, P):
    """The cuts (sequence, chunk offset) j = 0 .. P the chunk table computes from the chunk
    offsets: x_j = floor(j C / P), moved to the nearest sequence boundary within
    min(8, C // (4P)) chunks; the sequence of chunk x is the first one ending after x."""
    seq_off = [int(x) for x in seq_off]
    N, C = len(seq_off) - 1, seq_off[-1]
    snap = min(SNAP_CHUNKS, C // (4 * P))

    def holder(x):
        return next((i for i in range(N) if seq_off[i + 1] > x), N)

    cuts = []
    for j in range(P + 1):
        if j == 0:
            i, x = 0, 0
        elif j == P:
            i, x = N, C
        else:
            x = j * C // P
            i = holder(x)
            if i < N:
                dlo, dhi = x - seq_off[i], seq_off[i + 1] - x
                if 0 < dlo <= snap:
                    x -= dlo
                elif dlo > 0 and dhi <= snap:
                    x += dhi
                i = holder(x)
        cuts.append((i, x - seq_off[i] if i < N else 0))
    return cuts


def pieces(seq_off, cuts):
    """Pieces of the cut plan: (cut j or -1, sequence, c0, c1) for every run's pieces; a piece
    that starts at a cut inside a sequence carries that cut's index."""
    out = []
    P = len(cuts) - 1
    for w in range(P):
        (i0, o0), (i1, o1) = cuts[w], cuts[w + 1]
        i = i0
        while i < i1 or (i == i1 and o1 > 0):
            n = int(seq_off[i + 1] - seq_off[i])
            c0 = o0 if i == i0 else 0
            c1 = o1 if i == i1 else n
            if not (c0 == c1 and n > 0):
                out.append((w if c0 > 0 else -1, i, c0, c1))
            i += 1
    return out


def table_bytes(N):
    """Workspace bytes before the cut-plan states: header, per-sequence tables, the
    workgroup-run table, the unit list and the cut table."""
    up = lambda x: -(-x // 256) * 256
    return 256 + up(8 * N) + up(8 * N) + up(8 * (N + 1)) + up(8 * 257) + up(8 * N) + up(12 * 257)


def cut_table(ws, N, P):
    """The cuts the chunk table wrote: list of (sequence, chunk offset), j = 0 .. P, and the
    first-cut column (list of P + 1)."""
    up = lambda x: -(-x // 256) * 256
    off = 256 + up(8 * N) + up(8 * N) + up(8 * (N + 1)) + up(8 * 257) + up(8 * N)
    raw = ws[off:off + 12 * 257].cpu().numpy().view(np.int32)
    return [(int(raw[j]), int(raw[257 + j])) for j in range(P + 1)], [int(raw[514 + j]) for j in range(P + 1)]


def expected_firsts(cuts):
    """First of the cuts inside cut j's sequence (j for a cut at a sequence boundary)."""
    out = []
    for j, (i, o) in enumerate(cuts):
        j0 = j
        if o > 0:
            while j0 > 1 and cuts[j0 - 1][0] == i and cuts[j0 - 1][1] > 0:
                j0 -= 1
        out.append(j0)
    return out


def segment_states(ws, N, H, P):
    """The fp32 cut states S, F, P of a cut-plan call, read back from its workspace: three
    float64 arrays [H, P, 128, 128] (V-major), slot j = cut j.  S_j is written where pass A
    (a sequence's first cut) or the scan computed it; F_j, P_j hold the piece's run from zero
    and from the identity (P_j only where its transition run went the whole piece)."""
    n = H * P * 128 * 128
    off = table_bytes(N)
    raw = ws[off:off + 3 * 4 * n].cpu().numpy().view(np.float32).astype(np.float64)
    S, F, Pm = (raw[i * n:(i + 1) * n].reshape(H, P, 128, 128) for i in range(3))
    return S, F, Pm


def segment_aux(ws, N, H, P):
    """Per head and cut of a cut-plan call: z (chunks its transition run took before it
    stopped, -1: the whole piece), drop (1 where the scan dropped S_j's share) and the
    squared norms of S_j and F_j (per consumer wavefront): int64 [H, P] twice, float64
    [H, P, 4] twice."""
    slots = H * P
    off = table_bytes(N) + 3 * 4 * slots * 128 * 128
    raw = ws[off:off + slots * 40].cpu().numpy()
    z = raw[:4 * slots].view(np.int32).astype(np.int64).reshape(H, P)
    drop = raw[4 * slots:8 * slots].view(np.int32).astype(np.int64).reshape(H, P)
    nS = raw[8 * slots:24 * slots].view(np.float32).astype(np.float64).reshape(H, P, 4)
    nF = raw[24 * slots:40 * slots].view(np.float32).astype(np.float64).reshape(H, P, 4)
    return z, drop, nS, nF


def seq_chunk_offsets(w):
    """Chunk offset of every sequence of a workload (the chunk table's seq_off)."""
    lens = w.lengths if w.cu_seqlens is not None else [w.T] * w.B
    return np.concatenate([[0], np.cumsum([-(-int(n) // 16) for n in lens])]).astype(np.int64)
