"""gated_delta_rule_86_amd -- Kimi Delta Attention (KDA) chunked forward pass for MI355X (gfx950).

The compute path is libkda.so (hand-written HIP kernels behind the C ABI in include/kda.h);
``kda.fwd`` is its thin Python binding.  ``workloads`` draws the seeded synthetic inputs.
"""
from . import kda
from .kda import KDAError, fwd, workspace_size

__all__ = ["kda", "fwd", "workspace_size", "KDAError"]
