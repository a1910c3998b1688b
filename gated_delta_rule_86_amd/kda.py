"""Thin Python binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: every step of the forward pass runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  If libkda.so is
missing or cannot be loaded, every call raises; there is no fallback path.

``fwd`` mirrors the FlashKDA README "Kernel API" entry point:

    fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
        initial_state=None, final_state=None, cu_seqlens=None)

plus the keyword switches use_gate_in_kernel, use_qk_l2norm_in_kernel and
use_beta_sigmoid_in_kernel (README, "Using FlashKDA as an FLA backend"); turning one
off means that input arrives already activated (kda_fwd_ex in include/kda.h).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_OK = 0
STATUS_NAMES = {
    0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_HEAD_DIM", 4: "KDA_ERR_DTYPE",
    5: "KDA_ERR_LOWER_BOUND", 6: "KDA_ERR_SCALE", 7: "KDA_ERR_ALIGN", 8: "KDA_ERR_WORKSPACE",
    9: "KDA_ERR_CU_SEQLENS", 10: "KDA_ERR_HIP", 11: "KDA_ERR_ALIAS", 12: "KDA_ERR_FLAGS",
    13: "KDA_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # KDA_NOALLOC_SCRATCH_BYTES
# activation switches of kda_fwd_ex (include/kda.h)
GATE_IN_KERNEL, QK_L2NORM_IN_KERNEL, BETA_SIGMOID_IN_KERNEL = 1, 2, 4
ALL_IN_KERNEL = 7
STATE_NONE, STATE_BF16, STATE_FP32 = 0, 1, 2

# every symbol include/kda.h declares
EXPORTS = ("kda_fwd", "kda_fwd_ex", "kda_fwd_recurrent", "kda_fwd_recurrent_timed", "kda_fwd_timed",
           "kda_fwd_noalloc", "kda_fwd_workspace_size", "kda_bwd", "kda_bwd_workspace_size",
           "kda_status_string",
           "kda_fwd_device_status", "kda_chunk_table", "kda_version")


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str = "kda_fwd"):
        self.status = status
        super().__init__(f"{what} failed: {STATUS_NAMES.get(status, status)}")


_lib = None


def lib():
    """Load libkda.so (built in-tree by ``python -m gated_delta_rule_86_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gated_delta_rule_86_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    L.kda_fwd.restype = ctypes.c_int
    L.kda_fwd.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, f32, vp, ctypes.c_int, vp,
                          ctypes.c_int, vp, vp, i64, i64, i64, i64, i64, i64, vp, ctypes.c_size_t, vp]
    L.kda_fwd_ex.restype = ctypes.c_int
    L.kda_fwd_ex.argtypes = L.kda_fwd.argtypes + [ctypes.c_uint32]
    L.kda_fwd_recurrent.restype = ctypes.c_int
    L.kda_fwd_recurrent.argtypes = L.kda_fwd.argtypes + [ctypes.c_uint32]
    L.kda_fwd_recurrent_timed.restype = ctypes.c_int
    L.kda_fwd_recurrent_timed.argtypes = L.kda_fwd_recurrent.argtypes + [ctypes.POINTER(ctypes.c_void_p)]
    L.kda_fwd_timed.restype = ctypes.c_int
    L.kda_fwd_timed.argtypes = L.kda_fwd.argtypes + [ctypes.POINTER(ctypes.c_void_p)]
    L.kda_fwd_noalloc.restype = ctypes.c_int
    L.kda_fwd_noalloc.argtypes = L.kda_fwd.argtypes[:22] + [vp, ctypes.c_uint32]
    L.kda_bwd.restype = ctypes.c_int
    L.kda_bwd.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, f32, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                          vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, ctypes.c_size_t, vp,
                          ctypes.c_uint32]
    L.kda_bwd_workspace_size.restype = ctypes.c_size_t
    L.kda_bwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    L.kda_fwd_workspace_size.restype = ctypes.c_size_t
    L.kda_fwd_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_fwd_device_status.restype = ctypes.c_int
    L.kda_fwd_device_status.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), vp]
    L.kda_chunk_table.restype = ctypes.c_int
    L.kda_chunk_table.argtypes = [vp, i64, i64, i64, i64, vp, ctypes.c_size_t,
                                  ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                  ctypes.POINTER(ctypes.c_int32), vp]
    L.kda_version.restype = ctypes.c_int
    L.kda_version.argtypes = []
    _lib = L
    return L


def workspace_size(B: int, T: int, H: int, N: int = 0, varlen: bool = False) -> int:
    return int(lib().kda_fwd_workspace_size(B, T, H, N, 1 if varlen else 0))


def forward_launches(B: int, T: int, H: int, N: int = 0, varlen: bool = False) -> int:
    """Launches of the forward kernel per call: 3 (pass A, the transition runs, pass B) with
    the cut plan, else 1.  The cut plan shows in the workspace size (states per head and cut
    beyond the chunk table, the workgroup runs, the unit list and the cut table)."""
    n = N if varlen else B
    up = lambda x: -(-x // 256) * 256
    table = 256 + up(8 * n) + up(8 * n) + up(8 * (n + 1)) + up(8 * 257) + up(8 * n) + up(12 * 257)
    return 3 if workspace_size(B, T, H, N, varlen) > table else 1


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _state_code(t) -> int:
    import torch
    if t is None:
        return STATE_NONE
    if t.dtype == torch.bfloat16:
        return STATE_BF16
    if t.dtype == torch.float32:
        return STATE_FP32
    raise ValueError(f"state dtype must be bf16 or fp32, got {t.dtype}")


def fwd_recurrent(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state=None,
                  final_state=None, cu_seqlens=None, **kw):
    """The same forward pass evaluated token by token (kda_fwd_recurrent): for the decode
    step (one token per sequence, state in and out) and other short sequences.  Same
    arguments and keywords as ``fwd``; stage_events takes 3 handles here (before the chunk
    table, before the recurrent kernel, after it; kda_fwd_recurrent_timed)."""
    return fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
               final_state, cu_seqlens, _recurrent=True, **kw)


def fwd_noalloc(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state=None,
                final_state=None, cu_seqlens=None, **kw):
    """The same forward pass through kda_fwd_noalloc: no workspace, the library's static
    device scratch (NOALLOC_SCRATCH_BYTES per GPU) instead; calls that overlap on one GPU
    race.  Same arguments and keywords as ``fwd`` except workspace and stage_events.
    Raises KDAError(KDA_ERR_SCRATCH) for problems whose workspace would exceed the scratch."""
    for bad in ("workspace", "stage_events"):
        if kw.get(bad) is not None:
            raise ValueError(f"fwd_noalloc takes no {bad}")
    return fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
               final_state, cu_seqlens, _noalloc=True, **kw)


def fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state=None,
        final_state=None, cu_seqlens=None, *, cu_seqlens_host=None, workspace=None, stream=None,
        stage_events=None, use_gate_in_kernel=True, use_qk_l2norm_in_kernel=True,
        use_beta_sigmoid_in_kernel=True, _recurrent=False, _noalloc=False):
    """KDA forward pass on torch device tensors; writes ``out`` and ``final_state`` in place.

    q, k, v, g: bf16 [B, T, H, 128]; beta: bf16 [B, T, H]; out: bf16 [B, T, H, 128];
    A_log: fp32 [H]; dt_bias: fp32 [H, 128]; states: bf16/fp32 [N, H, 128, 128] or None;
    cu_seqlens: int64 [N+1] device tensor or None (then N = B).
    cu_seqlens_host: optional host copy (sequence or CPU tensor) for a synchronous check.
    workspace: optional uint8 device tensor of at least workspace_size(...) bytes.
    stage_events: optional sequence of 5 raw hipEvent_t handles (ints); when given the call
    goes through kda_fwd_timed, which records them around each launch (see include/kda.h).
    use_*_in_kernel: activation switches.  With use_gate_in_kernel=False, g is the natural-log
    decay itself and A_log / dt_bias may be None; with use_qk_l2norm_in_kernel=False q and k
    are used as given; with use_beta_sigmoid_in_kernel=False beta is the write strength.
    """
    import torch
    L = lib()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("g", g)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (B, T, H, K) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 [B, T, H, K] tensor")
    for name, t in (("v", v), ("out", out)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (B, T, H, V) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 [B, T, H, V] tensor")
    if beta.dtype != torch.bfloat16 or tuple(beta.shape) != (B, T, H) or not beta.is_contiguous():
        raise ValueError("beta must be a contiguous bf16 [B, T, H] tensor")
    flags = ((GATE_IN_KERNEL if use_gate_in_kernel else 0) |
             (QK_L2NORM_IN_KERNEL if use_qk_l2norm_in_kernel else 0) |
             (BETA_SIGMOID_IN_KERNEL if use_beta_sigmoid_in_kernel else 0))
    if use_gate_in_kernel or A_log is not None:
        if A_log is None or A_log.dtype != torch.float32 or A_log.numel() != H or not A_log.is_contiguous():
            raise ValueError("A_log must be a contiguous fp32 [H] tensor")
    if use_gate_in_kernel or dt_bias is not None:
        if (dt_bias is None or dt_bias.dtype != torch.float32 or tuple(dt_bias.shape) != (H, K)
                or not dt_bias.is_contiguous()):
            raise ValueError("dt_bias must be a contiguous fp32 [H, K] tensor")
    if initial_state is not None and final_state is not None and initial_state.dtype != final_state.dtype:
        raise ValueError("initial_state and final_state dtypes must match")
    N = B
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous int64 [N+1] tensor")
        N = cu_seqlens.numel() - 1
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and (tuple(t.shape) != (N, H, V, K) or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [N, H, V, K] tensor")
    host_cu = None
    if cu_seqlens_host is not None:
        import numpy as np
        host_cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int64))
    if _noalloc:
        st = L.kda_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
                               _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                               _state_code(initial_state), _ptr(final_state), _state_code(final_state),
                               _ptr(cu_seqlens), None if host_cu is None else host_cu.ctypes.data,
                               B, T, H, N if cu_seqlens is not None else B, K, V,
                               _stream_handle(stream, q.device), flags)
        if st != KDA_OK:
            raise KDAError(st, "kda_fwd_noalloc")
        return None
    ws_bytes = workspace_size(B, T, H, N if cu_seqlens is not None else B, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
        # allocated on the current stream; the kernels run on `stream`: keep the caching
        # allocator from reusing the block before they have finished
        if stream is not None and stream != torch.cuda.current_stream(q.device):
            workspace.record_stream(stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
            _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
            _state_code(initial_state), _ptr(final_state), _state_code(final_state),
            _ptr(cu_seqlens), None if host_cu is None else host_cu.ctypes.data,
            B, T, H, N if cu_seqlens is not None else B, K, V, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream_handle(stream, q.device))
    if _recurrent:
        if stage_events is None:
            st = L.kda_fwd_recurrent(*args, flags)
        else:
            evs = (ctypes.c_void_p * 3)(*[ctypes.c_void_p(int(e)) for e in stage_events[:3]])
            st = L.kda_fwd_recurrent_timed(*args, flags, evs)
    elif stage_events is None:
        st = L.kda_fwd(*args) if flags == ALL_IN_KERNEL else L.kda_fwd_ex(*args, flags)
    else:
        if flags != ALL_IN_KERNEL:
            raise ValueError("stage_events (kda_fwd_timed) runs with every activation in the pass")
        evs = (ctypes.c_void_p * 5)(*[ctypes.c_void_p(int(e)) for e in stage_events])
        st = L.kda_fwd_timed(*args, evs)
    if st != KDA_OK:
        raise KDAError(st)
    return workspace


def bwd_workspace_size(B: int, T: int, H: int, N: int = 0, varlen: bool = False) -> int:
    return int(lib().kda_bwd_workspace_size(B, T, H, N, 1 if varlen else 0))


def bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, dout, initial_state=None,
        dfinal_state=None, cu_seqlens=None, *, cu_seqlens_host=None, workspace=None, stream=None,
        use_gate_in_kernel=True, use_qk_l2norm_in_kernel=True, use_beta_sigmoid_in_kernel=True):
    """Gradients of ``fwd``'s out and final_state (kda_bwd in include/kda.h).

    Inputs as ``fwd``; dout: bf16 [B, T, H, 128] (dL/dout); dfinal_state: None or fp32
    [N, H, 128, 128] (dL/dfinal_state).  Returns a dict of fp32 device tensors: dq, dk, dv,
    dg [B, T, H, 128]; dbeta [B, T, H]; dA_log [H] and dt_bias [H, 128] (with the gate
    switch on); dinitial_state [N, H, 128, 128]; and the workspace used.
    """
    import torch
    L = lib()
    B, T, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("g", g), ("v", v), ("dout", dout)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (B, T, H, K) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 [B, T, H, K] tensor")
    if beta.dtype != torch.bfloat16 or tuple(beta.shape) != (B, T, H) or not beta.is_contiguous():
        raise ValueError("beta must be a contiguous bf16 [B, T, H] tensor")
    flags = ((GATE_IN_KERNEL if use_gate_in_kernel else 0) |
             (QK_L2NORM_IN_KERNEL if use_qk_l2norm_in_kernel else 0) |
             (BETA_SIGMOID_IN_KERNEL if use_beta_sigmoid_in_kernel else 0))
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if dfinal_state is not None and (dfinal_state.dtype != torch.float32 or tuple(dfinal_state.shape) != (N, H, V, K)
                                     or not dfinal_state.is_contiguous()):
        raise ValueError("dfinal_state must be a contiguous fp32 [N, H, V, K] tensor")
    dev = q.device
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    r = {"dq": f32(B, T, H, K), "dk": f32(B, T, H, K), "dv": f32(B, T, H, V), "dg": f32(B, T, H, K),
         "dbeta": f32(B, T, H), "dinitial_state": f32(N, H, V, K)}
    if use_gate_in_kernel:
        r["dA_log"] = f32(H)
        r["ddt_bias"] = f32(H, K)
    host_cu = None
    if cu_seqlens_host is not None:
        import numpy as np
        host_cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int64))
    ws_bytes = bwd_workspace_size(B, T, H, N if cu_seqlens is not None else B, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        if stream is not None and stream != torch.cuda.current_stream(dev):
            workspace.record_stream(stream)
    st = L.kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(A_log), _ptr(dt_bias),
                   float(lower_bound), _ptr(initial_state), _state_code(initial_state), _ptr(dout),
                   _ptr(dfinal_state), _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dg"]),
                   _ptr(r["dbeta"]), _ptr(r.get("dA_log")), _ptr(r.get("ddt_bias")),
                   _ptr(r["dinitial_state"]), _ptr(cu_seqlens),
                   None if host_cu is None else host_cu.ctypes.data, B, T, H,
                   N if cu_seqlens is not None else B, K, V, _ptr(workspace),
                   workspace.numel() * workspace.element_size(), _stream_handle(stream, dev), flags)
    if st != KDA_OK:
        raise KDAError(st, "kda_bwd")
    r["workspace"] = workspace
    return r


def device_status(workspace, stream=None) -> int:
    """Read the device status word after a call (synchronises the stream)."""
    out = ctypes.c_int32(-1)
    st = lib().kda_fwd_device_status(_ptr(workspace), ctypes.byref(out),
                                     _stream_handle(stream, workspace.device))
    if st != KDA_OK:
        raise KDAError(st, "kda_fwd_device_status")
    return int(out.value)


def chunk_table(cu_seqlens, B: int, T: int, H: int, workspace=None, stream=None):
    """Run only the chunk-table stage; returns (seq_off int64 [N+1], n_total, status)."""
    import numpy as np
    import torch
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dev = cu_seqlens.device if cu_seqlens is not None else torch.device("cuda")
    ws_bytes = workspace_size(B, T, H, N if cu_seqlens is not None else B, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        if stream is not None and stream != torch.cuda.current_stream(dev):
            workspace.record_stream(stream)
    seq_off = np.zeros(N + 1, dtype=np.int64)
    n_total = ctypes.c_int64(-1)
    status = ctypes.c_int32(-1)
    st = lib().kda_chunk_table(_ptr(cu_seqlens), B, T, H, N if cu_seqlens is not None else 0,
                               _ptr(workspace), workspace.numel(),
                               seq_off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                               ctypes.byref(n_total), ctypes.byref(status),
                               _stream_handle(stream, dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_table")
    return seq_off, int(n_total.value), int(status.value)
