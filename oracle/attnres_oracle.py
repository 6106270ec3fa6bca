"""CPU oracle for the AttnRes depth-routing hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  The product path
(the HIP library and its Python binding) never calls it, and it imports
nothing from the product path.

Plain, slow, float64 numpy.  Every function computes the plain definition
written on the pages, with no blocking, fusion or reordering beyond what the
definition states.  Inputs are upcast to float64 exactly (bf16 inputs arrive
as bf16-exact float32).

Sources cited (page title and section):
  [B-LAB]  b-lab.team summary of "Attention Residuals": §1 Full Attention
           Residuals (h_l, alpha, phi, v_i), §2 Block Attention Residuals
           (b_n, value matrix per sublayer), §3 Infrastructure Design
           (two-phase inference).
  [REVIEW] dimensionstp.github.io "Attention Residuals Review": §3-2 Module
           breakdown -- (1) Full AttnRes, (2) Block AttnRes, (3) learned
           pseudo-query and zero init, (4) two-phase computation with an
           exact online-softmax merge.
  [EXPL]   ai-systems-engineering.com "Attention Residuals" explainer:
           weights example, learned-query example (RMSNorm for scores only,
           gain 1, eps omitted), Block grouping example.
  [MHAR]   chatpaper.ai "Multi-Head Attention Residuals" abstract: the routing
           query reshaped into H per-subspace heads, each with its own depth
           softmax; H = 1 is exactly AttnRes.

Readings where the pages are silent (each also listed in the design notes):
  * eps sits inside the root: x / sqrt(mean(x^2) + eps).  parity unpinned for
    eps > 0 (the worked example omits eps).
  * RMSNorm gain g is elementwise, one [d] vector per destination by default
    (or one shared vector); key k_i = g * RMSNorm(v_i).  Only the fold identity
    (w, g) == (w * g, 1) pins it.
  * MHAR normalises over the full width d, then splits keys, query and values
    into H contiguous chunks of d/H channels.  Heads beyond H = 1 are pinned
    only by the per-head worked example and the zero-query invariant.
  * Backward: the pages give no formula; block_bwd and full_bwd are the
    analytic gradients of sum_j <dh_j, h_j> derived from the forward
    definition, pinned by central finite differences (finite_difference_grads,
    full_finite_difference_grads) and closed-form identities.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _gain_row(gain, j: int, d: int) -> np.ndarray:
    """Gain used by destination j: per-destination [n_dst, d], shared [d], or ones."""
    if gain is None:
        return np.ones(d)
    g = _f64(gain)
    return g if g.ndim == 1 else g[j]


# ---------------------------------------------------------------------------
# Forward building blocks
# ---------------------------------------------------------------------------

def rms_normalise(v, eps: float) -> np.ndarray:
    """RMSNorm without gain over the last axis: v / sqrt(mean_k v_k^2 + eps).

    [EXPL] learned-query section: RMS is the root of the mean of squares, so
    RMS([2, 0, 0]) = 2/sqrt(3) and the normalised vector is [sqrt(3), 0, 0].
    """
    v = _f64(v)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def depth_read(sources, w, g, eps: float, H: int = 1):
    """One destination reading an explicit list of depth sources.

    sources: [n, T, d]  (the destination's value matrix, one row per source)
    w: [d] pseudo-query of the destination; g: [d] RMSNorm gain.

    Steps ([B-LAB] §1; [REVIEW] §3-2; [EXPL] learned-query section; [MHAR]):
      1. key k_i = g * RMSNorm(v_i)                (normalised for the score only)
      2. score s_i = w . k_i, per head h on channels [h*d/H, (h+1)*d/H)
         (no 1/sqrt(d) and no temperature: phi(q, k) = exp(q^T RMSNorm(k)))
      3. alpha_i = exp(s_i) / sum_j exp(s_j) over the destination's sources
         (evaluated as exp(s_i - max s) / sum exp(s_j - max s), exact in reals)
      4. h = sum_i alpha_i v_i with the UN-normalised v_i, head h's alpha on
         head h's channels.
    Returns (h [T, d], alpha [T, H, n], scores [T, H, n]).
    """
    V = _f64(sources)
    n, T, d = V.shape
    assert d % H == 0
    dh = d // H
    K = rms_normalise(V, eps) * _f64(g)[None, None, :]
    Kh = K.reshape(n, T, H, dh)
    Vh = V.reshape(n, T, H, dh)
    wh = _f64(w).reshape(H, dh)
    scores = np.einsum("nthk,hk->thn", Kh, wh)
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    alpha = e / e.sum(axis=-1, keepdims=True)
    h = np.einsum("thn,nthk->thk", alpha, Vh).reshape(T, d)
    return h, alpha, scores


def full_fwd(src, w, gain=None, eps: float = 1e-6, H: int = 1, n_dst: Optional[int] = None):
    """Full AttnRes ([B-LAB] §1, h_l = sum_{i<l} alpha_{i->l} v_i).

    src: [n_src, T, d] with v_0 the embedding and v_i the sublayer outputs.
    w: [n_dst, d].  Destination j (0-based) reads sources 0 .. n_src-n_dst+j, so
    with n_dst = n_src = L destination l = j+1 reads v_0..v_{l-1}.
    Returns out [n_dst, T, d].
    """
    src = _f64(src)
    n_src, T, d = src.shape
    n_dst = _f64(w).shape[0] if n_dst is None else n_dst
    assert 1 <= n_dst <= n_src
    out = np.empty((n_dst, T, d))
    for j in range(n_dst):
        n_j = n_src - n_dst + j + 1
        out[j] = depth_read(src[:n_j], _f64(w)[j], _gain_row(gain, j, d), eps, H)[0]
    return out


def block_sources(reps, partials, i: int) -> np.ndarray:
    """Value matrix of sublayer i (1-based) of the current block ([B-LAB] §2).

    i = 1 reads the cached reps [b_0 .. b_{N-1}] only: the still-empty partial
    sum is not a source ([EXPL] Block grouping example).  i >= 2 reads
    [b_0 .. b_{N-1}, b^{(n)}_{i-1}] where b^{(n)}_{i-1} = partials[i-2] is the
    sum of the block's outputs before sublayer i.
    """
    reps = _f64(reps)
    if i == 1:
        return reps
    return np.concatenate([reps, _f64(partials)[i - 2][None]], axis=0)


def block_direct(reps, partials, w, gain=None, eps: float = 1e-6, H: int = 1):
    """Block AttnRes for all S sublayers of one block, by the plain definition.

    reps [N, T, d]; partials [S-1, T, d]; w [S, d]; gain [S, d], [d] or None.
    Returns h [S, T, d].  With H > 1 this is MHAR ([MHAR]).
    """
    w = _f64(w)
    S = w.shape[0]
    T, d = _f64(reps).shape[1:]
    h = np.empty((S, T, d))
    for i in range(1, S + 1):
        h[i - 1] = depth_read(block_sources(reps, partials, i), w[i - 1],
                              _gain_row(gain, i - 1, d), eps, H)[0]
    return h


def mhar_fwd(reps, partials, w, gain=None, eps: float = 1e-6, H: int = 1):
    """Multi-head Block routing: the plain definition with H heads ([MHAR])."""
    return block_direct(reps, partials, w, gain, eps, H)


# ---------------------------------------------------------------------------
# Two-phase algorithm ([B-LAB] §3 Inference; [REVIEW] §3-2 (4)).  A separate
# check of the algebra: must equal block_direct exactly in real arithmetic.
# ---------------------------------------------------------------------------

def block_phase1(reps, w, gain=None, eps: float = 1e-6, H: int = 1):
    """Phase 1: all S pseudo-queries of the block against the N cached reps.

    Returns o [S, T, d] (softmax-normalised read over the reps only) and the
    softmax statistics lse [S, H, T] = log sum_i exp(s_i).
    """
    reps = _f64(reps)
    w = _f64(w)
    S = w.shape[0]
    N, T, d = reps.shape
    o = np.empty((S, T, d))
    lse = np.empty((S, H, T))
    for l in range(S):
        o[l], _, s = depth_read(reps, w[l], _gain_row(gain, l, d), eps, H)
        m = s.max(axis=-1)
        lse[l] = (m + np.log(np.exp(s - m[..., None]).sum(axis=-1))).T
    return o, lse


def block_phase2_merge(o_i, lse_i, partial, w_i, g_i, eps: float = 1e-6, H: int = 1):
    """Phase 2 for sublayer i >= 2: score the partial sum and merge it with
    Phase 1's (o_i, lse_i) by online softmax.

    o_i [T, d], lse_i [H, T], partial [T, d], w_i [d], g_i [d] or None.
    Per head: s_p = w_i . (g_i * RMSNorm(p)), m = max(lse, s_p),
    a = exp(lse - m), b = exp(s_p - m), h = (a * o_i + b * p) / (a + b).
    """
    p = _f64(partial)
    T, d = p.shape
    dh = d // H
    g = np.ones(d) if g_i is None else _f64(g_i)
    k = (rms_normalise(p, eps) * g).reshape(T, H, dh)
    s_p = np.einsum("thk,hk->th", k, _f64(w_i).reshape(H, dh))
    lse = _f64(lse_i).T
    m = np.maximum(lse, s_p)
    a = np.exp(lse - m)[..., None]
    b = np.exp(s_p - m)[..., None]
    oh = _f64(o_i).reshape(T, H, dh)
    return ((a * oh + b * p.reshape(T, H, dh)) / (a + b)).reshape(T, d)


def block_phase2_merge_update(o_i, lse_i, partial_prev, f_prev, w_i, g_i, eps: float = 1e-6, H: int = 1,
                              norm_eps: float = 1e-6):
    """Phase 2 fused with the intra-block partial-sum update and the next
    sublayer's PreNorm statistic ([B-LAB] §3 and [REVIEW] §3-2 (4): the merge is
    the fused step of two-phase inference; [B-LAB] §2: the partial sum
    b_i = b_{i-1} + f_i).

    partial_prev [T, d] (None for the block's first update, i.e. zero) and the
    previous sublayer's output f_prev [T, d] give partial = partial_prev + f_prev,
    the partial this sublayer reads; h_i = block_phase2_merge(o_i, lse_i, partial,
    ...); inv_rms = 1 / sqrt(mean(h_i^2) + norm_eps), the scale a PreNorm sublayer
    applies to h_i.  Returns (partial, h_i, inv_rms [T]).
    """
    f = _f64(f_prev)
    partial = f if partial_prev is None else _f64(partial_prev) + f
    h = block_phase2_merge(o_i, lse_i, partial, w_i, g_i, eps, H)
    inv_rms = 1.0 / np.sqrt(np.mean(h * h, axis=-1) + norm_eps)
    return partial, h, inv_rms


def block_two_phase(reps, partials, w, gain=None, eps: float = 1e-6, H: int = 1):
    """Phase 1 for all S sublayers, then S-1 sequential Phase-2 merges."""
    w = _f64(w)
    S = w.shape[0]
    d = w.shape[1]
    o, lse = block_phase1(reps, w, gain, eps, H)
    h = o.copy()
    for i in range(2, S + 1):
        h[i - 1] = block_phase2_merge(o[i - 1], lse[i - 1], _f64(partials)[i - 2], w[i - 1],
                                      _gain_row(gain, i - 1, d), eps, H)
    return h


# ---------------------------------------------------------------------------
# Backward of the Block routing (gradient of sum_j <dh_j, h_j>).
# ---------------------------------------------------------------------------

def block_bwd(reps, partials, w, gain=None, eps: float = 1e-6, H: int = 1, dh=None):
    """Analytic gradients of L = sum_j <dh_j, h_j> for h = block_direct(...).

    Derived from the forward definition (the pages give no backward).  With
    x_i = RMSNorm(v_i), r_i = 1/sqrt(mean v_i^2 + eps), q_j = w_j * g_j and
    s_{j,i,h} = q_{j,h} . x_{i,h}:
      a_{j,i,h} = dh_{j,h} . v_{i,h}
      c_{j,i,h} = alpha_{j,i,h} (a_{j,i,h} - sum_m alpha_{j,m,h} a_{j,m,h})      (dL/ds)
      dv_i[k]   = sum_j alpha_{j,i,h(k)} dh_j[k]
                  + r_i sum_j c_{j,i,h(k)} q_j[k]
                  - r_i x_i[k] sum_{j,h} c_{j,i,h} s_{j,i,h} / d
      Z_j[k]    = sum_{t,i} c_{j,i,h(k)} x_i[k];  dw_j = g_j * Z_j;  dg_j = w_j * Z_j
    where j runs over the destinations that read source i.  A shared gain
    gets dg = sum_j w_j * Z_j.  Returns (d_reps, d_partials, dw, dgain).
    """
    reps = _f64(reps)
    partials = _f64(partials)
    w = _f64(w)
    dh = _f64(dh)
    N, T, d = reps.shape
    S = w.shape[0]
    hd = d // H
    shared_gain = gain is not None and _f64(gain).ndim == 1

    d_reps = np.zeros_like(reps)
    d_partials = np.zeros_like(partials)
    Z = np.zeros((S, d))
    for j in range(S):
        i_sub = j + 1
        V = block_sources(reps, partials, i_sub)                  # [n, T, d]
        n = V.shape[0]
        g = _gain_row(gain, j, d)
        q = w[j] * g
        r = 1.0 / np.sqrt(np.mean(V * V, axis=-1) + eps)           # [n, T]
        X = V * r[..., None]                                      # normalised sources
        _, alpha, s = depth_read(V, w[j], g, eps, H)              # [T, H, n]
        a = np.einsum("thk,nthk->thn", dh[j].reshape(T, H, hd), V.reshape(n, T, H, hd))
        c = alpha * (a - np.sum(alpha * a, axis=-1, keepdims=True))
        cs = np.einsum("thn,thn->tn", c, s)                       # sum_h c*s, [T, n]
        alpha_full = np.repeat(alpha, hd, axis=1)                 # [T, d, n]
        c_full = np.repeat(c, hd, axis=1)                         # [T, d, n]
        grad = (np.einsum("tkn,tk->ntk", alpha_full, dh[j])
                + r[..., None] * np.einsum("tkn,k->ntk", c_full, q)
                - X * r[..., None] * cs.T[..., None] / d)
        d_reps += grad[:N]
        if n > N:
            d_partials[i_sub - 2] += grad[N]
        Z[j] = np.einsum("tkn,ntk->k", c_full, X)
    dw = np.empty((S, d))
    dg_rows = np.empty((S, d))
    for j in range(S):
        dw[j] = _gain_row(gain, j, d) * Z[j]
        dg_rows[j] = w[j] * Z[j]
    if gain is None:
        dgain = None
    elif shared_gain:
        dgain = dg_rows.sum(axis=0)
    else:
        dgain = dg_rows
    return d_reps, d_partials, dw, dgain


def block_loss(reps, partials, w, gain, eps: float, H: int, dh) -> float:
    """L = sum_j <dh_j, h_j> for h = block_direct(...)."""
    return float(np.sum(_f64(dh) * block_direct(reps, partials, w, gain, eps, H)))


def finite_difference_grads(reps, partials, w, gain, eps: float, H: int, dh, step: float = 1e-6):
    """Central finite differences of block_loss w.r.t. every input element.

    Independent of block_bwd: it calls only the forward definition.
    Returns (d_reps, d_partials, dw, dgain) with dgain None when gain is None.
    """
    reps = _f64(reps).copy()
    partials = _f64(partials).copy()
    w = _f64(w).copy()
    gain = None if gain is None else _f64(gain).copy()

    def grad_of(arr: np.ndarray) -> np.ndarray:
        out = np.empty_like(arr)
        flat = arr.reshape(-1)
        gflat = out.reshape(-1)
        for k in range(flat.size):
            old = flat[k]
            flat[k] = old + step
            lp = block_loss(reps, partials, w, gain, eps, H, dh)
            flat[k] = old - step
            lm = block_loss(reps, partials, w, gain, eps, H, dh)
            flat[k] = old
            gflat[k] = (lp - lm) / (2 * step)
        return out

    return (grad_of(reps), grad_of(partials), grad_of(w),
            None if gain is None else grad_of(gain))


def full_loss(src, w, gain, eps: float, H: int, dout) -> float:
    """L = sum_j <dout_j, out_j> for out = full_fwd(...)."""
    return float(np.sum(_f64(dout) * full_fwd(src, w, gain, eps, H)))


def full_bwd(src, w, gain=None, eps: float = 1e-6, H: int = 1, dout=None):
    """Analytic gradients of L = sum_j <dout_j, out_j> for out = full_fwd(...).

    The pages give no backward.  This is the chain rule through the forward
    definition ([B-LAB] §1; [EXPL] learned-query section; [MHAR] heads), with
    destination j reading the causal prefix of sources 0 .. n_src-n_dst+j.
    With x_i = RMSNorm(v_i), r_i = 1/sqrt(mean v_i^2 + eps), q_j = w_j * g_j and
    s_{j,i,h} = q_{j,h} . x_{i,h}:
      a_{j,i,h} = dout_{j,h} . v_{i,h}
      c_{j,i,h} = alpha_{j,i,h} (a_{j,i,h} - sum_m alpha_{j,m,h} a_{j,m,h})    (dL/ds)
      dv_i[k]   = sum_j alpha_{j,i,h(k)} dout_j[k]
                  + r_i sum_j c_{j,i,h(k)} q_j[k]
                  - r_i x_i[k] sum_{j,h} c_{j,i,h} s_{j,i,h} / d
      Z_j[k]    = sum_{t,i} c_{j,i,h(k)} x_i[k];  dw_j = g_j * Z_j;  dg_j = w_j * Z_j
    where j runs over the destinations whose prefix contains source i.  A
    shared gain gets dg = sum_j w_j * Z_j.  Returns (d_src, dw, dgain).
    """
    src = _f64(src)
    w = _f64(w)
    dout = _f64(dout)
    n_src, T, d = src.shape
    n_dst = w.shape[0]
    assert 1 <= n_dst <= n_src and dout.shape == (n_dst, T, d)
    hd = d // H
    shared_gain = gain is not None and _f64(gain).ndim == 1

    d_src = np.zeros_like(src)
    Z = np.zeros((n_dst, d))
    for j in range(n_dst):
        n = n_src - n_dst + j + 1
        V = src[:n]                                                # [n, T, d]
        g = _gain_row(gain, j, d)
        q = w[j] * g
        r = 1.0 / np.sqrt(np.mean(V * V, axis=-1) + eps)           # [n, T]
        X = V * r[..., None]
        _, alpha, sc = depth_read(V, w[j], g, eps, H)             # [T, H, n]
        a = np.einsum("thk,nthk->thn", dout[j].reshape(T, H, hd), V.reshape(n, T, H, hd))
        c = alpha * (a - np.sum(alpha * a, axis=-1, keepdims=True))
        cs = np.einsum("thn,thn->tn", c, sc)                      # sum_h c*s, [T, n]
        alpha_full = np.repeat(alpha, hd, axis=1)                 # [T, d, n]
        c_full = np.repeat(c, hd, axis=1)
        d_src[:n] += (np.einsum("tkn,tk->ntk", alpha_full, dout[j])
                      + r[..., None] * np.einsum("tkn,k->ntk", c_full, q)
                      - X * r[..., None] * cs.T[..., None] / d)
        Z[j] = np.einsum("tkn,ntk->k", c_full, X)
    dw = np.empty((n_dst, d))
    dg_rows = np.empty((n_dst, d))
    for j in range(n_dst):
        dw[j] = _gain_row(gain, j, d) * Z[j]
        dg_rows[j] = w[j] * Z[j]
    if gain is None:
        dgain = None
    elif shared_gain:
        dgain = dg_rows.sum(axis=0)
    else:
        dgain = dg_rows
    return d_src, dw, dgain


def full_finite_difference_grads(src, w, gain, eps: float, H: int, dout, step: float = 1e-6):
    """Central finite differences of full_loss w.r.t. every input element.

    Independent of full_bwd: it calls only the forward definition.
    Returns (d_src, dw, dgain) with dgain None when gain is None.
    """
    src = _f64(src).copy()
    w = _f64(w).copy()
    gain = None if gain is None else _f64(gain).copy()

    def grad_of(arr: np.ndarray) -> np.ndarray:
        out = np.empty_like(arr)
        flat = arr.reshape(-1)
        gflat = out.reshape(-1)
        for k in range(flat.size):
            old = flat[k]
            flat[k] = old + step
            lp = full_loss(src, w, gain, eps, H, dout)
            flat[k] = old - step
            lm = full_loss(src, w, gain, eps, H, dout)
            flat[k] = old
            gflat[k] = (lp - lm) / (2 * step)
        return out

    return grad_of(src), grad_of(w), None if gain is None else grad_of(gain)


def tolerance_error(y, y_ref) -> float:
    """max |y - y_ref| / sqrt(mean(y_ref^2)) for one output tensor."""
    y = _f64(y)
    y_ref = _f64(y_ref)
    rms = np.sqrt(np.mean(y_ref * y_ref))
    if rms == 0.0:
        return float(np.max(np.abs(y - y_ref))) if y.size else 0.0
    return float(np.max(np.abs(y - y_ref)) / rms) if y.size else 0.0


__all__: Sequence[str] = (
    "rms_normalise", "depth_read", "full_fwd", "block_sources", "block_direct", "mhar_fwd",
    "block_phase1", "block_phase2_merge", "block_phase2_merge_update", "block_two_phase", "block_bwd", "block_loss",
    "finite_difference_grads", "full_loss", "full_bwd", "full_finite_difference_grads", "tolerance_error",
)
