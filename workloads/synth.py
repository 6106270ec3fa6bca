"""Seeded synthetic inputs for the AttnRes depth-routing workloads.

This module only draws and rounds numbers.  It holds none of the routing
arithmetic (no normalisation, scoring, softmax or weighted sum), so both the
CPU oracle and the HIP path can consume what it produces without sharing any
of the method's code.

Every tensor is drawn from its own PCG64 stream, keyed by
``SeedSequence(seed, spawn_key=(tensor_id, index))``.  Streams are therefore
independent of draw order and of how many threads fill them, and a given
(seed, tensor, index) always yields the same values.

Notation follows the pages: T tokens, d hidden width, sources v_i, block
representations b_n, intra-block outputs f, pseudo-queries w_l, RMSNorm gain g,
H heads.  Distributions are written N(mean, variance) throughout, so
``std = sqrt(variance)``.

bf16 workloads are drawn in float32 and rounded once to bfloat16 with
round-to-nearest-even; the rounded values are kept as float32 arrays whose
low 16 mantissa bits are zero, so the same numbers upcast exactly to float64
for the oracle and convert exactly to torch.bfloat16 for the device.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Tensor ids used in the spawn key of each stream.
_TID_SOURCES = 1
_TID_F = 2
_TID_W = 3
_TID_GAIN = 4
_TID_DH = 5
_TID_CONV = 6
_TID_MIX = 7

_CHUNK = 1 << 24  # elements per stream chunk; chunks are separate sub-streams


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bfloat16 (ties to even), in place.

    Returns the same array; values are float32 with the low 16 bits cleared.
    Inputs are finite draws, so NaN/Inf handling is not needed.
    """
    assert x.dtype == np.float32 and x.flags.c_contiguous
    u = x.reshape(-1).view(np.uint32)

    def work(lo: int, hi: int) -> None:
        seg = u[lo:hi]
        lsb = seg >> np.uint32(16)
        lsb &= np.uint32(1)
        lsb += np.uint32(0x7FFF)
        seg += lsb
        seg &= np.uint32(0xFFFF0000)

    n = u.size
    step = max(_CHUNK, (n + _threads() - 1) // _threads())
    spans = [(lo, min(n, lo + step)) for lo in range(0, n, step)]
    if len(spans) <= 1:
        for lo, hi in spans:
            work(lo, hi)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda s: work(*s), spans))
    return x


def _normal_into(out: np.ndarray, seed: int, tid: int, index: int) -> None:
    """Fill ``out`` (float32, contiguous) with standard normals from stream (seed, tid, index).

    The stream is split into fixed chunks of _CHUNK elements, chunk k drawn from
    ``SeedSequence(seed, spawn_key=(tid, index, k))``; the result does not
    depend on the number of worker threads.
    """
    flat = out.reshape(-1)
    n = flat.size
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def work(k: int) -> None:
        lo, hi = k * _CHUNK, min(n, (k + 1) * _CHUNK)
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(tid, index, k))
        g = np.random.Generator(np.random.PCG64(ss))
        g.standard_normal(out=flat[lo:hi], dtype=np.float32)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))


def normal_stack(count: int, shape: tuple, stds, seed: int, tid: int) -> np.ndarray:
    """[count, *shape] float32, slice k ~ N(0, stds[k]^2), each slice its own stream."""
    out = np.empty((count,) + tuple(shape), dtype=np.float32)
    for k in range(count):
        _normal_into(out[k], seed, tid, k)
        s = np.float32(stds[k])
        if s != 1.0:
            out[k] *= s
    return out


@dataclass
class Workload:
    """One synthetic workload.  Arrays are float32 (bf16-exact when dtype == 'bf16').

    kind: 'full' or 'block'.
      full : src [n_src, T, d], w [n_dst, d]; destination j reads sources
             0 .. n_src - n_dst + j.
      block: reps [N, T, d], partials [S-1, T, d], w [S, d]; dh [S, T, d] if
             a backward is part of the workload.
      (full workloads with a backward carry dout [n_dst, T, d] in dh.)
    gain: [n_dst, d] (one per destination), [d] (shared) or None (all ones).
    """

    name: str
    kind: str
    dtype: str  # 'f32' or 'bf16'
    T: int
    d: int
    H: int
    eps: float
    w: np.ndarray
    gain: Optional[np.ndarray]
    src: Optional[np.ndarray] = None
    n_dst: int = 0
    reps: Optional[np.ndarray] = None
    partials: Optional[np.ndarray] = None
    dh: Optional[np.ndarray] = None
    f: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return 0 if self.reps is None else self.reps.shape[0]

    @property
    def S(self) -> int:
        return self.w.shape[0]


def _maybe_round(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else x


def _pseudo_queries(n: int, d: int, seed: int) -> np.ndarray:
    # w_l ~ N(0, 1/d): std 1/sqrt(d).  Parameters stay float32 (never rounded).
    return normal_stack(n, (d,), [1.0 / math.sqrt(d)] * n, seed, _TID_W)


def _gain(n: int, d: int, seed: int, variance: float) -> np.ndarray:
    # g = 1 + N(0, variance), one [d] vector per destination sublayer.
    g = normal_stack(n, (d,), [math.sqrt(variance)] * n, seed, _TID_GAIN)
    g += np.float32(1.0)
    return g


def full_workload(T: int, d: int, L: int, std_step: float, dtype: str, seed: int = 0,
                  gain_variance: Optional[float] = None, eps: float = 1e-6, H: int = 1,
                  n_dst: Optional[int] = None, name: str = "full", with_dout: bool = False) -> Workload:
    """Full AttnRes: L sources v_i ~ N(0, (1 + std_step*i)^2), i = 0..L-1.

    With n_dst = L (default) destination l = 1..L reads v_0..v_{l-1}.
    gain_variance None means gain = 1 (passed as None).  With with_dout, the
    upstream gradient dout [n_dst, T, d] ~ N(0, 1) is stored in dh.
    """
    n_dst = L if n_dst is None else n_dst
    src = normal_stack(L, (T, d), [1.0 + std_step * i for i in range(L)], seed, _TID_SOURCES)
    src = _maybe_round(src, dtype)
    w = _pseudo_queries(n_dst, d, seed)
    gain = None if gain_variance is None else _gain(n_dst, d, seed, gain_variance)
    dout = _maybe_round(normal_stack(n_dst, (T, d), [1.0] * n_dst, seed, _TID_DH), dtype) if with_dout else None
    return Workload(name=name, kind="full", dtype=dtype, T=T, d=d, H=H, eps=eps, w=w,
                    gain=gain, src=src, n_dst=n_dst, dh=dout,
                    meta=dict(L=L, std_step=std_step, seed=seed, gain_variance=gain_variance))


def block_workload(T: int, d: int, N: int, S: int, H: int, rep_std_step: float, dtype: str,
                   seed: int = 0, gain_variance: Optional[float] = 0.02, eps: float = 1e-6,
                   with_dh: bool = False, name: str = "block", with_f: bool = False) -> Workload:
    """Block AttnRes inputs for one block.

    reps b_0..b_{N-1} ~ N(0, (1 + rep_std_step*n)^2); intra-block outputs
    f_1..f_{S-1} ~ N(0, 1); partials[k] = f_1 + ... + f_{k+1} accumulated in
    float32 and rounded once; w [S, d] ~ N(0, 1/d); gain [S, d] = 1 + N(0,
    gain_variance); dh [S, T, d] ~ N(0, 1) when with_dh.  With with_f the
    outputs themselves, each rounded to dtype, are kept in f [S-1, T, d] (the
    inputs of the fused partial-sum update).
    """
    reps = normal_stack(N, (T, d), [1.0 + rep_std_step * n for n in range(N)], seed, _TID_SOURCES)
    reps = _maybe_round(reps, dtype)
    if S > 1:
        f = normal_stack(S - 1, (T, d), [1.0] * (S - 1), seed, _TID_F)
        f_out = _maybe_round(f.copy(), dtype) if with_f else None
        np.cumsum(f, axis=0, out=f)  # running intra-block sum, float32
        partials = _maybe_round(f, dtype)
    else:
        partials = np.zeros((0, T, d), dtype=np.float32)
        f_out = np.zeros((0, T, d), dtype=np.float32) if with_f else None
    w = _pseudo_queries(S, d, seed)
    gain = None if gain_variance is None else _gain(S, d, seed, gain_variance)
    dh = None
    if with_dh:
        dh = _maybe_round(normal_stack(S, (T, d), [1.0] * S, seed, _TID_DH), dtype)
    return Workload(name=name, kind="block", dtype=dtype, T=T, d=d, H=H, eps=eps, w=w,
                    gain=gain, reps=reps, partials=partials, dh=dh, f=f_out,
                    meta=dict(N=N, S=S, rep_std_step=rep_std_step, seed=seed,
                              gain_variance=gain_variance))


def msar_workload(T: int, d: int, n_src: int, n_dst: int, dtype: str, seed: int = 0, std_step: float = 0.1,
                  eps: float = 1e-6, name: str = "msar") -> Workload:
    """MSAR inputs: sources v_i ~ N(0, (1 + std_step*i)^2), i = 0..n_src-1;
    pseudo-queries w [n_dst, 4, d] ~ N(0, 1/d); convolution taps conv [24, d]
    with stream r's K_r taps ~ N(0, 1/K_r) (K = 4, 8, 12), so every stream keeps
    roughly the source's scale; mixer P [n_dst, 4 d, 4] ~ N(0, 1/(4 d)).
    The taps and P are kept in meta['conv'] and meta['mix']."""
    src = normal_stack(n_src, (T, d), [1.0 + std_step * i for i in range(n_src)], seed, _TID_SOURCES)
    src = _maybe_round(src, dtype)
    w = _pseudo_queries(n_dst * 4, d, seed).reshape(n_dst, 4, d)
    conv = np.concatenate([normal_stack(1, (K, d), [1.0 / math.sqrt(K)], seed, _TID_CONV + 16 * r)[0]
                           for r, K in enumerate((4, 8, 12))])
    mix = normal_stack(n_dst, (4 * d, 4), [1.0 / math.sqrt(4 * d)] * n_dst, seed, _TID_MIX)
    return Workload(name=name, kind="msar", dtype=dtype, T=T, d=d, H=1, eps=eps, w=w, gain=None, src=src,
                    n_dst=n_dst, meta=dict(conv=conv, mix=mix, std_step=std_step, seed=seed))


def block_msar_workload(T: int, d: int, N: int, S: int, seed: int = 0, rep_std_step: float = 0.3,
                        eps: float = 1e-6, name: str = "block_msar") -> Workload:
    """Block MSAR inputs: the block reps and partial sums of block_workload
    (bf16), with MSAR parameters as in msar_workload: w [S, 4, d] ~ N(0, 1/d),
    taps conv [24, d] (stream r's K_r taps ~ N(0, 1/K_r)), one mixer per
    sublayer P [S, 4 d, 4] ~ N(0, 1/(4 d))."""
    wl = block_workload(T=T, d=d, N=N, S=S, H=1, rep_std_step=rep_std_step, dtype="bf16", seed=seed,
                        gain_variance=None, eps=eps, name=name)
    w = _pseudo_queries(S * 4, d, seed).reshape(S, 4, d)
    conv = np.concatenate([normal_stack(1, (K, d), [1.0 / math.sqrt(K)], seed, _TID_CONV + 16 * r)[0]
                           for r, K in enumerate((4, 8, 12))])
    mix = normal_stack(S, (4 * d, 4), [1.0 / math.sqrt(4 * d)] * S, seed, _TID_MIX)
    wl.w = w
    wl.kind = "block_msar"
    wl.meta.update(conv=conv, mix=mix)
    return wl


# ---------------------------------------------------------------------------
# The five named workloads (shapes and distributions of the benchmark configs).
# ---------------------------------------------------------------------------

def config_full_fp32_small(seed: int = 0) -> Workload:
    """Full AttnRes, fp32: T=64, d=64, L=8, v_i ~ N(0,(1+0.2i)^2), gain 1, eps 1e-6."""
    return full_workload(T=64, d=64, L=8, std_step=0.2, dtype="f32", seed=seed,
                         gain_variance=None, eps=1e-6, name="full_fp32_T64_d64_L8")


def config_full_bf16(seed: int = 0, T: int = 4096) -> Workload:
    """Full AttnRes, bf16: T=4096, d=2048, L=32, v_i ~ N(0,(1+0.1i)^2), gain 1+N(0,0.02)."""
    return full_workload(T=T, d=2048, L=32, std_step=0.1, dtype="bf16", seed=seed,
                         gain_variance=0.02, eps=1e-6, name=f"full_bf16_T{T}_d2048_L32")


def config_full_fwd_bwd(seed: int = 0, T: int = 4096) -> Workload:
    """Full AttnRes fwd+bwd, bf16: the Full bf16 workload (d=2048, L=32) with dout ~ N(0,1)."""
    return full_workload(T=T, d=2048, L=32, std_step=0.1, dtype="bf16", seed=seed,
                         gain_variance=0.02, eps=1e-6, name=f"full_bwd_bf16_T{T}_d2048_L32", with_dout=True)


def config_block_two_phase(seed: int = 0, T: int = 16384) -> Workload:
    """Block two-phase, bf16: T=16384, d=4096, N=8, S=4, H=1, b_n ~ N(0,(1+0.3n)^2)."""
    return block_workload(T=T, d=4096, N=8, S=4, H=1, rep_std_step=0.3, dtype="bf16",
                          seed=seed, name=f"block_bf16_T{T}_d4096_N8_S4")


def config_mhar(seed: int = 0, T: int = 32768, H: int = 8) -> Workload:
    """MHAR Block routing, bf16: T=32768, d=4096, H=8, N=8, S=4, b_n ~ N(0,(1+0.1n)^2)."""
    return block_workload(T=T, d=4096, N=8, S=4, H=H, rep_std_step=0.1, dtype="bf16",
                          seed=seed, name=f"mhar_bf16_T{T}_d4096_H{H}_N8_S4")


def config_block_fwd_bwd(seed: int = 0, T: int = 8192) -> Workload:
    """Block fwd+bwd, bf16: T=8192, d=4096, N=8, S=4, dh ~ N(0,1)."""
    return block_workload(T=T, d=4096, N=8, S=4, H=1, rep_std_step=0.3, dtype="bf16",
                          seed=seed, with_dh=True, name=f"block_bwd_bf16_T{T}_d4096_N8_S4")


def config_mhar_fwd_bwd(seed: int = 0, T: int = 8192, H: int = 8) -> Workload:
    """MHAR Block fwd+bwd, bf16: the MHAR workload (d=4096, H=8, N=8, S=4) at T=8192 with dh ~ N(0,1)."""
    return block_workload(T=T, d=4096, N=8, S=4, H=H, rep_std_step=0.1, dtype="bf16",
                          seed=seed, with_dh=True, name=f"mhar_bwd_bf16_T{T}_d4096_H{H}_N8_S4")


def take_tokens(x: Optional[np.ndarray], idx: np.ndarray) -> Optional[np.ndarray]:
    """Select tokens (axis -2) of a [k, T, d] array; None passes through."""
    if x is None:
        return None
    return np.ascontiguousarray(x[:, idx, :])


def sample_tokens(T: int, count: int, seed: int = 1234) -> np.ndarray:
    """Sorted token sample: first, last and `count - 2` random distinct others."""
    if T <= count:
        return np.arange(T)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(99,))))
    mid = g.choice(np.arange(1, T - 1), size=count - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], mid]))
