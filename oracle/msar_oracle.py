"""CPU oracle for MSAR, multi-stream depth attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  The product path
(the HIP library and its Python binding) never calls it, and it imports
nothing from the product path.

Plain, slow, float64 numpy, written from the onedev.kr summary of the MSAR
paper ("Extending depth-wise attention to multiple streams"), sections "How it
differs" (the streams, the per-stream depth softmax, the H^pre mixer) and "How
to use it" (Block MSAR keeps one stream per source and expands the others on
demand).

The method, as computed here:
  * Each residual source v_i [T, d] expands into m = 4 full-width streams:
    stream 0 is v_i itself, streams 1..3 are causal depthwise 1-D
    convolutions of v_i along the token axis with kernel sizes 4, 8 and 12.
  * Each stream runs its own depth softmax with its own pseudo-query:
    s_i^(r) = w^(r) . RMSNorm(v_i^(r)),  alpha^(r) = softmax_i(s^(r)),
    Z^(r) = sum_i alpha_i^(r) v_i^(r)  (the weights of each stream sum to 1).
  * The H^pre mixer: beta = sigmoid(RMSNorm(Flatten(Z)) P), P [m d, m];
    h = sum_r beta_r Z^(r).

Readings where the summary is silent (each also listed in the design notes):
  * Tap k of a stream's kernel multiplies the source k tokens back (tap 0 is
    the current token); tokens before the first one of the call are zero.  No
    bias.
  * One set of three convolutions serves every source: the summary applies
    "the" convolution r to each source and writes the streams v_i^(r) with no
    destination index, while the pseudo-queries w_l^(r) carry one.  The taps
    are packed as conv [24, d]: rows 0-3 for stream 1, 4-11 for stream 2 and
    12-23 for stream 3.  Pseudo-queries and mixer belong to the destination:
    w [n_dst, 4, d], P [n_dst, 4 d, 4].  A model whose layers own different
    taps makes one call per layer.
  * RMSNorm as in AttnRes (x / sqrt(mean x^2 + eps)), with no gain in either
    place: a gain folds exactly into w (scores) and into P (mixer).
  * Flatten(Z) concatenates the streams in order: [Z^(0), Z^(1), Z^(2), Z^(3)].
  * The mixer has no bias term (the summary names RMSNorm, the md x m
    projection and the sigmoid only).
  * Destinations read causal prefixes of the sources as in Full AttnRes:
    destination j of n_dst reads sources 0 .. n_src - n_dst + j.  A Block
    MSAR sublayer is the n_dst = 1 call over its block reps and partial sum.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attnres_oracle import rms_normalise

MSAR_STREAMS = 4
MSAR_KERNEL_SIZES = (4, 8, 12)     # streams 1, 2, 3
MSAR_TAP_OFFSETS = (0, 4, 12)      # first packed row of each conv stream
MSAR_TAPS = 24


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def msar_expand(v, conv) -> np.ndarray:
    """Streams of one source: v [T, d], conv [24, d] -> [4, T, d].

    Stream r >= 1 at token t is sum_k conv[off_r + k] * v[t - k] over its
    K_r taps, with v[t - k] = 0 before the first token."""
    v = _f64(v)
    conv = _f64(conv)
    T, d = v.shape
    out = np.zeros((MSAR_STREAMS, T, d))
    out[0] = v
    for r in range(1, MSAR_STREAMS):
        K, off = MSAR_KERNEL_SIZES[r - 1], MSAR_TAP_OFFSETS[r - 1]
        for k in range(min(K, T)):
            out[r, k:] += conv[off + k] * v[:T - k]
    return out


def sigmoid(x) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-_f64(x)))


def msar_fwd(src, w, conv, P, eps: float = 1e-6, return_parts: bool = False):
    """MSAR routing for n_dst destinations with causal-prefix source sets.

    src [n_src, T, d]; w [n_dst, 4, d]; conv [24, d]; P [n_dst, 4 d, 4].
    Returns h [n_dst, T, d]; with return_parts also Z [n_dst, 4, T, d] and
    beta [n_dst, T, 4]."""
    src = _f64(src)
    w = _f64(w)
    P = _f64(P)
    n_src, T, d = src.shape
    n_dst = w.shape[0]
    assert w.shape == (n_dst, MSAR_STREAMS, d) and P.shape == (n_dst, MSAR_STREAMS * d, MSAR_STREAMS)
    assert 1 <= n_dst <= n_src and np.shape(conv) == (MSAR_TAPS, d)
    streams = np.stack([msar_expand(src[i], conv) for i in range(n_src)])      # [n_src, 4, T, d]
    h = np.zeros((n_dst, T, d))
    Z = np.zeros((n_dst, MSAR_STREAMS, T, d))
    beta = np.zeros((n_dst, T, MSAR_STREAMS))
    for j in range(n_dst):
        n = n_src - n_dst + j + 1
        for r in range(MSAR_STREAMS):
            vals = streams[:n, r]                                  # [n, T, d]
            keys = rms_normalise(vals, eps)
            s = np.einsum("itc,c->it", keys, w[j, r])
            s = s - s.max(axis=0, keepdims=True)
            a = np.exp(s)
            a /= a.sum(axis=0, keepdims=True)
            Z[j, r] = np.einsum("it,itc->tc", a, vals)
        flat = np.concatenate([Z[j, r] for r in range(MSAR_STREAMS)], axis=-1)   # [T, 4 d]
        beta[j] = sigmoid(rms_normalise(flat, eps) @ P[j])
        h[j] = np.einsum("tr,rtc->tc", beta[j], Z[j])
    if return_parts:
        return h, Z, beta
    return h


def _mixer(Z, P, eps):
    """h = sum_r beta_r Z^(r), beta = sigmoid(RMSNorm(Flatten(Z)) P); Z [4, T, d], P [4 d, 4]."""
    flat = np.concatenate([Z[r] for r in range(MSAR_STREAMS)], axis=-1)
    beta = sigmoid(rms_normalise(flat, eps) @ _f64(P))
    return np.einsum("tr,rtc->tc", beta, Z)


def block_msar_phase1(reps, w, conv, P1, eps: float = 1e-6):
    """Block MSAR, Phase 1 ([MSAR] "How to use it": AttnRes's two-phase
    computation carries over): the block's S sublayers' per-stream queries
    against the N cached reps, each rep's streams expanded once for all of them.

    reps [N, T, d]; w [S, 4, d]; conv [24, d]; P1 [4 d, 4] (sublayer 1's mixer).
    Returns (h1 [T, d], o [S-1, 4, T, d], lse [S-1, 4, T]): sublayer 1 reads the
    reps only, so its output is final; sublayers 2..S keep, per stream, the
    softmax-weighted state over the reps and its log-sum-exp."""
    reps = _f64(reps)
    w = _f64(w)
    N, T, d = reps.shape
    S = w.shape[0]
    streams = np.stack([msar_expand(reps[n], conv) for n in range(N)])       # [N, 4, T, d]
    o = np.zeros((S, MSAR_STREAMS, T, d))
    lse = np.zeros((S, MSAR_STREAMS, T))
    for i in range(S):
        for r in range(MSAR_STREAMS):
            vals = streams[:, r]
            s = np.einsum("ntc,c->nt", rms_normalise(vals, eps), w[i, r])
            m = s.max(axis=0)
            e = np.exp(s - m)
            l = e.sum(axis=0)
            o[i, r] = np.einsum("nt,ntc->tc", e / l, vals)
            lse[i, r] = m + np.log(l)
    return _mixer(o[0], P1, eps), o[1:], lse[1:]


def block_msar_phase2(o_i, lse_i, partial, w_i, conv, P_i, eps: float = 1e-6):
    """Block MSAR, Phase 2 for sublayer i >= 2: the partial sum's streams are
    scored with the sublayer's queries and merged into Phase 1's per-stream
    states by online softmax (exact), then the mixer gives h_i.

    o_i [4, T, d]; lse_i [4, T]; partial [T, d]; w_i [4, d]; P_i [4 d, 4]."""
    o_i = _f64(o_i)
    lse_i = _f64(lse_i)
    xp = msar_expand(partial, conv)                                           # [4, T, d]
    Z = np.zeros_like(o_i)
    for r in range(MSAR_STREAMS):
        sp = rms_normalise(xp[r], eps) @ _f64(w_i)[r]
        m = np.maximum(lse_i[r], sp)
        a = np.exp(lse_i[r] - m)[:, None]
        b = np.exp(sp - m)[:, None]
        Z[r] = (a * o_i[r] + b * xp[r]) / (a + b)
    return _mixer(Z, P_i, eps)


def block_msar_direct(reps, partials, w, conv, P, eps: float = 1e-6):
    """Every sublayer of one block by the plain definition: sublayer i reads
    the reps and (i >= 2) the partial sum b_{i-1} as one more source."""
    reps = _f64(reps)
    S = _f64(w).shape[0]
    out = []
    for i in range(1, S + 1):
        src = reps if i == 1 else np.concatenate([reps, _f64(partials)[i - 2][None]])
        out.append(msar_fwd(src, _f64(w)[i - 1:i], conv, _f64(P)[i - 1:i], eps)[0])
    return np.stack(out)


__all__ = ["MSAR_STREAMS", "MSAR_KERNEL_SIZES", "MSAR_TAP_OFFSETS", "MSAR_TAPS", "msar_expand", "sigmoid",
           "msar_fwd", "block_msar_phase1", "block_msar_phase2", "block_msar_direct"]
