"""Host-side checks of the C ABI (no GPU needed).

* libkda.so loads and exports every function include/kda.h declares.
* Every validation error of kda_fwd is returned before anything touches the device:
  the pointers below are never dereferenced, so fake aligned addresses are fine.
* kda_fwd_workspace_size covers the status word, the per-sequence chunk table, the
  table of whole-chain workgroup runs (257 int64) and the whole-chain unit list (2 int32
  per sequence), plus,
  for few long equal-length chains run as segments, three fp32 states per chain and segment.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from gated_delta_rule_86_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(kda.EXPORTS)
    L = ctypes.CDLL(kda.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = kda.lib()
    assert L.kda_version() >= 100
    for code, name in kda.STATUS_NAMES.items():
        assert L.kda_status_string(code).decode().startswith(name)
    assert L.kda_status_string(999).decode() == "KDA_ERR_UNKNOWN"


def ws_size(B, T, H, N=0, varlen=False):
    return kda.workspace_size(B, T, H, N, varlen)


def table_bytes(N):
    up = lambda x: -(-x // 256) * 256
    return 256 + up(8 * N) + up(8 * N) + up(8 * (N + 1)) + up(8 * 257) + up(8 * N) + up(12 * 257)


def cut_extra(H, P):
    """Workspace beyond the tables with the cut plan: three fp32 128 x 128 states per head and
    cut, then 40 bytes of per-cut words (z, drop, two norms of 4 floats) rounded up to 256."""
    return 0 if P == 1 else 3 * H * P * 128 * 128 * 4 + -(-H * P * 40 // 256) * 256


def test_workspace_size_formula():
    # many heads or short sequences: tables only, independent of T and H
    for B, T, H in [(1, 64, 1), (3, 17, 5), (1, 0, 4), (2, 300, 100), (1, 1 << 20, 200), (64, 1000, 4)]:
        assert ws_size(B, T, H) == table_bytes(B)
    # long sequences: plus the cut plan's states, P = min(256 / H, C / 16) per head
    for B, T, H, P in [(2, 4096, 16, 16), (1, 1 << 20, 8, 32), (1, 1100, 1, 4), (2, 2048, 128, 2)]:
        assert ws_size(B, T, H) == table_bytes(B) + cut_extra(H, P), (B, T, H)
    for N, T, H, P in [(8, 32000, 32, 8), (1, 1 << 20, 2, 128), (3, 3100, 4, 12)]:
        assert ws_size(1, T, H, N, True) == table_bytes(N) + cut_extra(H, P), (N, T, H)
    # with cu_seqlens and short sequences on average: tables only
    for N, T in [(256, 65000), (3, 5), (40, 32000)]:
        assert ws_size(1, T, 2, N, True) == table_bytes(N)
        assert ws_size(1, 2 * T // 3, 5, N, True) == table_bytes(N)
    assert ws_size(0, 10, 1) == 0            # B < 1
    assert ws_size(2, 10, 1, 3, True) == 0   # cu_seqlens needs B == 1
    assert ws_size(1, -1, 1) == 0


class Args:
    """A consistent set of arguments whose pointers are fake but aligned and disjoint."""

    def __init__(self, B=1, T=16, H=1, varlen=False, N=0):
        self.B, self.T, self.H = B, T, H
        tok = max(B * T * H * 128 * 2, 16)
        base = 1 << 32
        step = 1 << 28
        self.q, self.k, self.v, self.g, self.beta, self.out = (base + i * step for i in range(6))
        self.A_log = base + 6 * step
        self.dt_bias = base + 7 * step
        self.h0, self.h0_dt = base + 8 * step, kda.STATE_FP32
        self.ht, self.ht_dt = base + 9 * step, kda.STATE_FP32
        self.cu = base + 10 * step if varlen else None
        self.cu_host = None
        self.N = N if varlen else B
        self.K = self.V = 128
        self.scale, self.lb = 0.125, -5.0
        self.ws = base + 11 * step
        self.ws_bytes = ws_size(B, T, H, self.N if varlen else B, varlen)
        self.flags = None  # None: kda_fwd; else kda_fwd_ex with this switch mask
        assert tok < step

    def call(self):
        L = kda.lib()
        cu_host = None if self.cu_host is None else self.cu_host.ctypes.data
        args = (self.q, self.k, self.v, self.g, self.beta, self.scale, self.out, self.A_log,
                self.dt_bias, self.lb, self.h0, self.h0_dt, self.ht, self.ht_dt, self.cu, cu_host,
                self.B, self.T, self.H, self.N, self.K, self.V, self.ws, self.ws_bytes, None)
        if self.flags is None:
            return L.kda_fwd(*args)
        return L.kda_fwd_ex(*args, self.flags)


def expect(code, **changes):
    a = Args(**{k: changes.pop(k) for k in list(changes) if k in ("B", "T", "H", "varlen", "N")})
    for k, val in changes.items():
        setattr(a, k, val)
    assert a.call() == code, (changes, kda.STATUS_NAMES.get(a.call()))


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "out", "A_log", "dt_bias"])
def test_null_pointers(name):
    expect(1, **{name: None})


def test_shape_errors():
    expect(2, B=0)
    expect(2, T=-1)
    expect(2, H=0)
    expect(2, B=2, varlen=True, N=2)   # cu_seqlens requires B == 1
    expect(2, varlen=True, N=0)        # cu_seqlens with N < 1
    a = Args(B=2)
    a.N = 3                            # without cu_seqlens N must be B (or 0)
    assert a.call() == 2


def test_head_dim_errors():
    expect(3, K=64)
    expect(3, V=256)


def test_dtype_errors():
    expect(4, h0_dt=kda.STATE_BF16)                    # both given, dtypes differ
    expect(4, h0_dt=7)                                 # unknown dtype
    expect(4, h0=None)                                 # NULL pointer with a dtype
    expect(4, ht_dt=kda.STATE_NONE)                    # pointer without a dtype


def test_lower_bound_and_scale_errors():
    for lb in (-5.01, 0.01, float("nan"), float("-inf")):
        expect(5, lb=lb)
    for sc in (float("nan"), float("inf")):
        expect(6, scale=sc)


def test_alignment_errors():
    expect(7, q=Args().q + 8)
    expect(7, out=Args().out + 2)
    expect(7, beta=Args().beta + 1)
    expect(7, dt_bias=Args().dt_bias + 4)
    expect(7, ws=Args().ws + 128)
    expect(7, h0=Args().h0 + 8)


def test_alias_errors():
    a = Args()
    expect(11, out=a.q)
    expect(11, out=a.beta)
    expect(11, ht=a.v)
    expect(11, ht=a.out)
    expect(11, h0=a.out)
    expect(11, ht=a.h0 + 4096)    # overlapping but distinct state buffers


def test_workspace_errors():
    expect(8, ws=None)
    a = Args()
    expect(8, ws_bytes=a.ws_bytes - 1)


def test_cu_seqlens_host_checks():
    for cu in ([1, 8, 16], [0, 9, 8, 16], [0, 8, 15]):
        a = Args(T=16, varlen=True, N=len(cu) - 1)
        a.ws_bytes = ws_size(1, 16, 1, a.N, True)
        a.cu_host = np.array(cu, dtype=np.int64)
        assert a.call() == 9, cu


def test_chunk_table_argument_errors():
    L = kda.lib()
    p = ctypes.c_void_p(1 << 32)
    assert L.kda_chunk_table(None, 0, 16, 1, 0, p, 1 << 20, None, None, None, None) == 2
    assert L.kda_chunk_table(None, 1, 16, 1, 0, p, 16, None, None, None, None) == 8
    assert L.kda_chunk_table(None, 1, 16, 1, 0, ctypes.c_void_p((1 << 32) + 64), 1 << 20, None, None,
                             None, None) == 7
    assert L.kda_fwd_device_status(None, None, None) == 1


def test_activation_switch_errors():
    expect(12, flags=8)
    expect(12, flags=0xFFFFFFFF)
    # in-pass gate: A_log and dt_bias are required and checked for alignment
    expect(1, flags=kda.ALL_IN_KERNEL, A_log=None)
    expect(1, flags=kda.GATE_IN_KERNEL, dt_bias=None)
    expect(7, flags=kda.GATE_IN_KERNEL, dt_bias=Args().dt_bias + 4)
    # pre-activated gate: they are not read, so NULL or misaligned pass validation (the
    # too-small workspace, checked later, is then the first error)
    a = Args()
    for flags in (0, kda.QK_L2NORM_IN_KERNEL | kda.BETA_SIGMOID_IN_KERNEL):
        expect(8, flags=flags, A_log=None, dt_bias=None, ws_bytes=a.ws_bytes - 1)
        expect(8, flags=flags, A_log=a.A_log + 1, dt_bias=a.dt_bias + 4, ws_bytes=a.ws_bytes - 1)
        expect(5, flags=flags, A_log=None, dt_bias=None, lb=0.5)  # lower_bound still checked
    # the other switches do not change what is required
    expect(1, flags=kda.GATE_IN_KERNEL, q=None)


def test_forward_launches_of_reference_workloads():
    """One forward launch for the whole-chain plans, three (pass A, transition runs, pass B)
    for the cut plan; the helper reads the workspace size, so it tracks the layout."""
    assert kda.forward_launches(1, 64, 1) == 1                 # B=1 T=64 H=1
    assert kda.forward_launches(2, 4096, 16) == 3              # long batch rows: cut plan
    assert kda.forward_launches(1, 31094, 32, 8, True) == 3    # varlen, long on average: cut plan
    assert kda.forward_launches(1, 1 << 20, 8) == 3
    assert kda.forward_launches(1, 66285, 32, 256, True) == 1  # many short sequences: whole
    assert kda.forward_launches(256, 1, 32) == 1


def test_timed_entry_points_check_their_events():
    """kda_fwd_timed (5 handles) and kda_fwd_recurrent_timed (3) return KDA_ERR_NULL for a
    NULL handle array or a NULL handle among those they record, and otherwise validate their
    arguments as kda_fwd does, before any HIP call (the fake handles are never used)."""
    L = kda.lib()
    a = Args(T=16)
    base = (a.q, a.k, a.v, a.g, a.beta, a.scale, a.out, a.A_log, a.dt_bias, a.lb, a.h0, a.h0_dt,
            a.ht, a.ht_dt, a.cu, None, a.B, a.T, a.H, a.N, a.K, a.V, a.ws, a.ws_bytes, None)
    fake = [(1 << 33) + 256 * i for i in range(5)]

    def timed(n, handles, lb=None):
        args = list(base)
        if lb is not None:
            args[9] = lb
        evs = None if handles is None else (ctypes.c_void_p * len(handles))(*handles)
        if n == 5:
            return L.kda_fwd_timed(*args, evs)
        return L.kda_fwd_recurrent_timed(*args, kda.ALL_IN_KERNEL, evs)

    for n in (5, 3):
        assert timed(n, None) == 1, n
        for i in range(n):
            h = list(fake[:n])
            h[i] = None
            assert timed(n, h) == 1, (n, i)
        assert timed(n, fake[:n], lb=0.5) == 5, n          # lower_bound out of range
    # the recurrent entry reads only its first three handles
    assert timed(3, fake[:3] + [None, None], lb=0.5) == 5


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """kda_fwd_noalloc checks the workspace its sizes need against its static scratch
    (KDA_NOALLOC_SCRATCH_BYTES) before any HIP call: KDA_ERR_SCRATCH, nothing launched."""
    L = kda.lib()
    cap = kda.NOALLOC_SCRATCH_BYTES
    a = Args(T=16)
    for N in (1 << 21, 1 << 22):
        T = 2 * N
        assert ws_size(1, T, 1, N, True) > cap
        st = L.kda_fwd_noalloc(a.q, a.k, a.v, a.g, a.beta, a.scale, a.out, a.A_log, a.dt_bias, a.lb,
                               None, kda.STATE_NONE, None, kda.STATE_NONE, 1 << 33, None, 1, T, 1, N,
                               128, 128, None, 7)
        assert st == 13, st  # KDA_ERR_SCRATCH
    # every reference workload fits (the 2^20-token one, segmented, needs the most)
    for B, T, H, N, varlen in [(1, 1 << 20, 8, 0, False), (2, 4096, 16, 0, False), (1, 31094, 32, 8, True),
                               (1, 66285, 32, 256, True), (256, 1, 32, 0, False)]:
        assert ws_size(B, T, H, N, varlen) <= cap, (B, T, H)
    assert L.kda_status_string(13).decode().startswith("KDA_ERR_SCRATCH")


def test_cut_plan_replica():
    """The tests' replica of the cut plan (kda_testutil.cut_plan) picks the same number of
    workgroups per head as the library, read off the workspace size."""
    from kda_testutil import cut_plan
    for B, T, H, N, varlen in [(1, 700, 1, 0, False), (1, 8192, 2, 0, False), (3, 4096, 2, 0, False),
                               (2, 5000, 3, 0, False), (1, 4103, 1, 0, False), (2, 4096, 16, 0, False),
                               (1, 1 << 20, 8, 0, False), (3, 1500, 2, 0, False), (1, 1 << 20, 1, 0, False),
                               (1, 100, 4, 0, False), (5, 4000, 40, 0, False), (1, 1023, 1, 0, False),
                               (1, 1024, 1, 0, False), (130, 9000, 1, 0, False), (1, 9000, 128, 0, False),
                               (1, 9000, 129, 0, False), (300, 2000, 1, 0, False),
                               (1, 31094, 32, 8, True), (1, 66285, 32, 256, True), (1, 5000, 3, 5, True),
                               (1, 1024, 2, 1, True), (1, 1023, 2, 1, True), (1, 100000, 64, 20, True)]:
        P = cut_plan(B, T, H, N, varlen)
        assert ws_size(B, T, H, N, varlen) == table_bytes(N if varlen else B) + cut_extra(H, P), \
            (B, T, H, N, varlen, P)
        # a run is at least 16 chunks
        C = -(-T // 16) * (1 if varlen else B)
        assert P == 1 or (2 <= P <= 256 // H and C // P >= 16), (B, T, H, N, P)


def test_sequence_count_limit():
    """Unit codes hold the sequence index in 29 bits: N >= 2^29 is a shape error, and the
    workspace size is 0 for it."""
    assert ws_size(1, 100, 1, (1 << 29) - 1, True) > 0
    assert ws_size(1, 100, 1, 1 << 29, True) == 0
    a = Args(T=16, varlen=True, N=1)
    a.N = 1 << 29
    # no states: their fake ranges at this N would overlap the other fake buffers
    a.h0, a.h0_dt, a.ht, a.ht_dt = None, kda.STATE_NONE, None, kda.STATE_NONE
    assert a.call() == 2  # KDA_ERR_SHAPE


def _bwd_call(**over):
    """kda_bwd with fake but aligned, disjoint pointers; `over` replaces arguments by name."""
    base, step = 1 << 32, 1 << 28
    p = {n: base + i * step for i, n in enumerate(
        ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "h0", "dout", "dht", "dq", "dk", "dv", "dg",
         "dbeta", "dA_log", "ddt", "dh0", "cu", "ws"])}
    a = dict(q=p["q"], k=p["k"], v=p["v"], g=p["g"], beta=p["beta"], scale=0.125, A_log=p["A_log"],
             dt_bias=p["dt_bias"], lb=-5.0, h0=p["h0"], h0_dt=kda.STATE_FP32, dout=p["dout"], dht=p["dht"],
             dq=p["dq"], dk=p["dk"], dv=p["dv"], dg=p["dg"], dbeta=p["dbeta"], dA_log=p["dA_log"],
             ddt=p["ddt"], dh0=p["dh0"], cu=None, cu_host=None, B=1, T=16, H=1, N=1, K=128, V=128,
             ws=p["ws"], ws_bytes=None, flags=7)
    a.update(over)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = kda.bwd_workspace_size(a["B"], a["T"], a["H"], a["N"], a["cu"] is not None)
    L = kda.lib()
    return L.kda_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["scale"], a["A_log"], a["dt_bias"], a["lb"],
                     a["h0"], a["h0_dt"], a["dout"], a["dht"], a["dq"], a["dk"], a["dv"], a["dg"], a["dbeta"],
                     a["dA_log"], a["ddt"], a["dh0"], a["cu"], a["cu_host"], a["B"], a["T"], a["H"], a["N"],
                     a["K"], a["V"], a["ws"], a["ws_bytes"], None, a["flags"])


def test_bwd_error_paths():
    """kda_bwd validates everything on the host before any launch."""
    for name in ("q", "k", "v", "g", "beta", "dout", "dq", "dk", "dv", "dg", "dbeta", "A_log", "dt_bias"):
        assert _bwd_call(**{name: None}) == 1, name                      # KDA_ERR_NULL
    assert _bwd_call(flags=0, A_log=None, dt_bias=None, ws_bytes=0) == 8  # gate off: no A_log needed
    assert _bwd_call(B=0) == 2 and _bwd_call(H=0) == 2 and _bwd_call(T=-1) == 2
    assert _bwd_call(K=64) == 3
    assert _bwd_call(h0_dt=kda.STATE_NONE) == 4
    assert _bwd_call(lb=0.5) == 5 and _bwd_call(scale=float("nan")) == 6
    assert _bwd_call(dq=(1 << 32) + 10 * (1 << 28) + 4) == 7                # misaligned fp32 output
    assert _bwd_call(dk=(1 << 32) + 10 * (1 << 28)) == 11                   # dk on top of dq
    assert _bwd_call(dq=1 << 32) == 11                                       # an output on top of q
    assert _bwd_call(ws_bytes=100) == 8
    assert _bwd_call(flags=8) == 12
    # with the gate switch off dA_log / dt_bias are not needed
    assert kda.bwd_workspace_size(1, 16, 1) > kda.workspace_size(1, 16, 1)
    assert kda.bwd_workspace_size(0, 16, 1) == 0
