"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random numbers and packs them into the layouts the
``kda_fwd`` argument table fixes (FlashKDA README, "Kernel API": bf16
q/k/v/g ``[B, T, H, 128]``, bf16 beta ``[B, T, H]``, fp32 ``A_log [H]`` and
``dt_bias [H, 128]``, optional bf16/fp32 states ``[N, H, 128, 128]``, int64
``cu_seqlens [N+1]``).  It holds none of the method's arithmetic, so both the
oracle side and the HIP side of the tests use it.

Recipe (all draws are fp32, then rounded to bf16 with round-to-nearest-even
where the argument is bf16; the second parameter of N(mu, s) is the standard
deviation):
  q, k, v, g, beta logits ~ N(0, 1)
  A_log[h] = log(U[1, 16]);  dt_bias ~ N(0, 0.1)
  initial state ~ N(0, 0.05)
  varlen lengths ~ U[1, Lmax] (inclusive); a draw is kept only if some length is
  not a multiple of 16 and the total is within 10% of N * (1 + Lmax) / 2,
  otherwise the next seed attempt is used.
Inputs that arrive already activated (a switch of the forward pass turned off):
  gate switch off:   g = lower_bound * U[0, 1]      (a per-token natural-log decay)
  l2norm switch off: q, k ~ N(0, 1/128)            (norms close to 1, not exactly 1)
  sigmoid switch off: beta ~ U[0, 1]
Seeds: numpy SeedSequence([config_id, attempt]).spawn(9) in the order
  [lengths, q, k, v, g, beta, A_log, dt_bias, initial_state]; each tensor is drawn
  in blocks of 2^24 values, block i from child i of that tensor's seed (PCG64).
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional

import numpy as np

D = 128
STATE_NONE, STATE_BF16, STATE_FP32 = "none", "bf16", "fp32"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).copy()
    nan = np.isnan(x)
    u += ((u >> 16) & 1) + np.uint32(0x7FFF)
    r = (u >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    lower_bound: float
    scale: float
    initial_state: Optional[np.ndarray]  # uint16 bf16 bits or float32, [N, H, 128, 128]
    state_dtype: str  # dtype of both initial and final state ("none" -> no initial, fp32 final)
    final_dtype: str
    cu_seqlens: Optional[np.ndarray]  # int64 [N+1]
    flags: int = 7  # activation switches of the forward pass (1 gate, 2 q/k l2norm, 4 beta sigmoid)

    @property
    def N(self) -> int:
        return self.B if self.cu_seqlens is None else int(self.cu_seqlens.size - 1)

    @property
    def lengths(self) -> np.ndarray:
        if self.cu_seqlens is None:
            return np.full(self.B, self.T, dtype=np.int64)
        return np.diff(self.cu_seqlens)

    @property
    def head_tokens(self) -> int:
        return int(self.lengths.sum()) * self.H

    def describe(self) -> dict:
        d = {"workload": self.name, "B": self.B, "T": self.T, "H": self.H, "N": self.N,
             "K": D, "V": D, "lower_bound": self.lower_bound,
             "initial_state": self.state_dtype if self.initial_state is not None else "none",
             "final_state": self.final_dtype, "varlen": self.cu_seqlens is not None}
        if self.flags != 7:
            d["activation_flags"] = self.flags
        return d


_BLOCK = 1 << 24


def _fill_normal(seq: np.random.SeedSequence, n: int, std: float, to_bf16: bool,
                 uniform=None) -> np.ndarray:
    """n draws of N(0, std) (or of U[lo, hi] when uniform = (lo, hi)) in float32 (or bf16
    bits), in fixed blocks of 2^24 with one spawned child seed per block, so the values do not
    depend on the thread count."""
    out = np.empty(n, dtype=np.uint16 if to_bf16 else np.float32)
    nblk = max(1, -(-n // _BLOCK))
    kids = seq.spawn(nblk)

    def work(i):
        lo = i * _BLOCK
        m = min(_BLOCK, n - lo)
        if m <= 0:
            return
        gen = np.random.Generator(np.random.PCG64(kids[i]))
        if uniform is not None:
            x = gen.uniform(uniform[0], uniform[1], size=m).astype(np.float32)
        else:
            x = gen.standard_normal(m, dtype=np.float32)
            if std != 1.0:
                x *= np.float32(std)
        out[lo:lo + m] = f32_to_bf16_bits(x) if to_bf16 else x

    if nblk == 1:
        work(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(16, nblk, os.cpu_count() or 1)) as ex:
            list(ex.map(work, range(nblk)))
    return out


def _normal_bf16(seq, shape, std=1.0) -> np.ndarray:
    return _fill_normal(seq, int(np.prod(shape)), std, True).reshape(shape)


def _uniform_bf16(seq, shape, lo, hi) -> np.ndarray:
    return _fill_normal(seq, int(np.prod(shape)), 1.0, True, uniform=(lo, hi)).reshape(shape)


def _lengths(config_id: int, N: int, Lmax: int):
    attempt = 0
    while True:
        ss = np.random.SeedSequence([config_id, attempt]).spawn(9)
        rng = np.random.Generator(np.random.PCG64(ss[0]))
        L = rng.integers(1, Lmax, size=N, endpoint=True).astype(np.int64)
        target = N * (1 + Lmax) / 2.0
        if np.any(L % 16 != 0) and abs(L.sum() - target) <= 0.1 * target:
            return L, ss
        attempt += 1


def make(name: str, B: int, T: int, H: int, *, lengths=None, lower_bound=-5.0,
         scale=None, state_dtype=STATE_FP32, with_initial=True, final_dtype=None,
         seed=0, seeds=None, flags=7) -> Workload:
    """General generator.  ``lengths`` (list) switches to varlen with B = 1, T = sum(lengths).
    ``flags``: activation switches of the forward pass; an input whose switch is off is drawn
    already activated (see the recipe above)."""
    if seeds is None:
        seeds = np.random.SeedSequence([seed, 0]).spawn(9)
    cu = None
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(lengths.size + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lengths)
        B, T = 1, int(cu[-1])
    N = B if cu is None else lengths.size
    qk_std = 1.0 if flags & 2 else 1.0 / math.sqrt(D)
    q = _normal_bf16(seeds[1], (B, T, H, D), qk_std)
    k = _normal_bf16(seeds[2], (B, T, H, D), qk_std)
    v = _normal_bf16(seeds[3], (B, T, H, D))
    if flags & 1:
        g = _normal_bf16(seeds[4], (B, T, H, D))
    else:
        g = _uniform_bf16(seeds[4], (B, T, H, D), float(lower_bound), 0.0)
    if flags & 4:
        beta = _normal_bf16(seeds[5], (B, T, H))
    else:
        beta = _uniform_bf16(seeds[5], (B, T, H), 0.0, 1.0)
    A_log = np.log(np.random.Generator(np.random.PCG64(seeds[6])).uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = _fill_normal(seeds[7], H * D, 0.1, False).reshape(H, D)
    h0 = None
    if with_initial and state_dtype != STATE_NONE:
        h0 = _fill_normal(seeds[8], N * H * D * D, 0.05, state_dtype == STATE_BF16).reshape(N, H, D, D)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    if final_dtype is None:
        final_dtype = STATE_FP32 if state_dtype == STATE_NONE else state_dtype
    return Workload(name, B, T, H, q, k, v, g, beta, A_log, dt_bias, float(np.float32(lower_bound)),
                    float(np.float32(scale)), h0, state_dtype, final_dtype, cu, int(flags))


CONFIG_NAMES = [
    "B1_T64_H1_nostate",
    "B2_T4096_H16_fp32state",
    "varlen_N8_Lmax8192_H32_bf16state_lb-2",
    "B1_T1048576_H8_fp32state",
    "varlen_N256_Lmax512_H32_fp32state",
    "decode_B256_T1_H32_fp32state",
]


def config(i: int) -> Workload:
    """The five reference workloads (index 0..4), and a decode step (index 5: 256 sequences,
    one token each, 32 heads, fp32 state in and out)."""
    seeds = np.random.SeedSequence([i, 0]).spawn(9)
    name = CONFIG_NAMES[i]
    if i == 0:
        return make(name, 1, 64, 1, state_dtype=STATE_NONE, with_initial=False,
                    final_dtype=STATE_FP32, seeds=seeds)
    if i == 1:
        return make(name, 2, 4096, 16, state_dtype=STATE_FP32, seeds=seeds)
    if i == 2:
        L, seeds = _lengths(2, 8, 8192)
        return make(name, 1, 0, 32, lengths=L, lower_bound=-2.0, state_dtype=STATE_BF16, seeds=seeds)
    if i == 3:
        return make(name, 1, 1 << 20, 8, state_dtype=STATE_FP32, seeds=seeds)
    if i == 4:
        L, seeds = _lengths(4, 256, 512)
        return make(name, 1, 0, 32, lengths=L, state_dtype=STATE_FP32, seeds=seeds)
    if i == 5:
        return make(name, 256, 1, 32, state_dtype=STATE_FP32, seeds=seeds)
    raise ValueError(i)
