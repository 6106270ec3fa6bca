"""Pins for the MSAR oracle (onedev.kr MSAR summary, "How it differs").

Each pin raises AssertionError when the oracle is wrong.  They use a library
routine (numpy's convolution for the causal depthwise streams), reductions to
the pinned AttnRes oracle (one-tap streams), closed forms of the mixer and
invariants (the token window of the convolutions, magnitude invariance).
test_msar_oracle.py runs them and plants mistakes that some pin must catch.
"""

from __future__ import annotations

import numpy as np

from oracle import attnres_oracle as aro
from oracle import msar_oracle as mso

K_SIZES = (4, 8, 12)
OFFS = (0, 4, 12)


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, n_src=5, n_dst=3, T=17, d=8, taps="random"):
    r = _rng(seed)
    src = r.standard_normal((n_src, T, d)) * (1 + 0.3 * np.arange(n_src))[:, None, None]
    w = r.standard_normal((n_dst, 4, d)) / np.sqrt(d)
    if taps == "random":
        conv = r.standard_normal((24, d)) / 3
    else:  # one tap: every stream is the source itself
        conv = np.zeros((24, d))
        conv[[0, 4, 12], :] = 1.0
    P = r.standard_normal((n_dst, 4 * d, 4)) / np.sqrt(4 * d)
    return src, w, conv, P


def _np_causal_conv(x, taps):
    """Causal convolution of one channel: numpy's full convolution, first len(x) outputs."""
    return np.convolve(x, taps)[: len(x)]


def pin_msar_expand_is_causal_convolution():
    for T in (17, 3, 1):           # longer and shorter than the kernels
        r = _rng(T)
        v = r.standard_normal((T, 5))
        conv = r.standard_normal((24, 5))
        out = mso.msar_expand(v, conv)
        np.testing.assert_array_equal(out[0], v)
        for s in range(1, 4):
            K, off = K_SIZES[s - 1], OFFS[s - 1]
            for c in range(5):
                np.testing.assert_allclose(out[s, :, c], _np_causal_conv(v[:, c], conv[off:off + K, c]),
                                           rtol=1e-12, atol=1e-12)


def pin_msar_one_tap_streams_reduce_to_attnres():
    """With one-tap streams every stream is the source, so stream r is Full
    AttnRes with query w^(r); with P = 0 every mixer weight is 1/2."""
    src, w, conv, P = _case(1, taps="one")
    P[:] = 0.0
    h = mso.msar_fwd(src, w, conv, P, eps=1e-6)
    want = 0.5 * sum(aro.full_fwd(src, w[:, r], None, 1e-6) for r in range(4))
    np.testing.assert_allclose(h, want, rtol=1e-12, atol=1e-12)


def pin_msar_mixer_closed_form():
    """One-tap streams, and P non-zero only in column 0 over the first d rows:
    beta_0 = sigmoid(Z0 . p / RMS([Z0..Z3])), the other betas are 1/2."""
    src, w, conv, P = _case(2, taps="one")
    n_dst, d = w.shape[0], w.shape[2]
    p = _rng(3).standard_normal((n_dst, d))
    P[:] = 0.0
    P[:, :d, 0] = p
    eps = 1e-6
    h, Z, beta = mso.msar_fwd(src, w, conv, P, eps=eps, return_parts=True)
    for j in range(n_dst):
        Zr = [aro.full_fwd(src, w[:, r], None, eps)[j] for r in range(4)]     # [T, d] each
        rms_all = np.sqrt(sum((z * z).sum(-1) for z in Zr) / (4 * d) + eps)
        b0 = 1.0 / (1.0 + np.exp(-(Zr[0] @ p[j]) / rms_all))
        np.testing.assert_allclose(beta[j, :, 0], b0, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(beta[j, :, 1:], 0.5, rtol=0, atol=0)
        want = b0[:, None] * Zr[0] + 0.5 * (Zr[1] + Zr[2] + Zr[3])
        np.testing.assert_allclose(h[j], want, rtol=1e-12, atol=1e-12)


def pin_msar_identical_sources():
    """Identical sources: each stream's weights sum to 1, so Z^(r) is the
    stream itself whatever the scores."""
    r = _rng(4)
    T, d = 15, 6
    u = r.standard_normal((T, d))
    taps = r.standard_normal((24, d))
    src = np.stack([u] * 4)
    conv = taps
    w = r.standard_normal((2, 4, d))
    P = np.zeros((2, 4 * d, 4))
    h, Z, beta = mso.msar_fwd(src, w, conv, P, eps=1e-6, return_parts=True)
    streams = [u] + [np.stack([_np_causal_conv(u[:, c], taps[OFFS[s] : OFFS[s] + K_SIZES[s], c])
                                for c in range(d)], axis=-1) for s in range(3)]
    for j in range(2):
        for s in range(4):
            np.testing.assert_allclose(Z[j, s], streams[s], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(h[j], 0.5 * sum(streams), rtol=1e-12, atol=1e-12)


def pin_msar_token_window():
    """h at token t depends on tokens t-11 .. t of the sources only."""
    src, w, conv, P = _case(5, T=30)
    h = mso.msar_fwd(src, w, conv, P)
    t = 20
    far = src.copy()
    far[:, : t - 11] += 5.0          # older than the longest kernel
    far[:, t + 1 :] -= 3.0           # later tokens
    np.testing.assert_array_equal(mso.msar_fwd(far, w, conv, P)[:, t], h[:, t])
    near = src.copy()
    near[:, t - 11] += 5.0           # the oldest tap of the 12-tap stream
    assert np.max(np.abs(mso.msar_fwd(near, w, conv, P)[:, t] - h[:, t])) > 1e-3


def pin_msar_magnitude_invariance():
    """With eps = 0, scaling every source by c > 0 scales h by c: both RMSNorms
    remove the scale, so the weights and the mixer do not change."""
    src, w, conv, P = _case(6)
    h = mso.msar_fwd(src, w, conv, P, eps=0.0)
    np.testing.assert_allclose(mso.msar_fwd(src * 7.5, w, conv, P, eps=0.0), 7.5 * h, rtol=1e-11, atol=1e-12)


def pin_msar_prefix_sets():
    """Destination j of n_dst reads sources 0 .. n_src - n_dst + j: changing a
    later source leaves the earlier destinations unchanged."""
    src, w, conv, P = _case(7, n_src=5, n_dst=3)
    h = mso.msar_fwd(src, w, conv, P)
    moved = src.copy()
    moved[4] *= -2.0                  # read by the last destination only
    h2 = mso.msar_fwd(moved, w, conv, P)
    np.testing.assert_array_equal(h2[:2], h[:2])
    assert np.max(np.abs(h2[2] - h[2])) > 1e-3


def pin_block_msar_two_phase_equals_direct():
    """[MSAR] "How to use it": the two-phase computation carries over.  Phase 1
    over the reps plus the online-softmax merge of each partial equals the
    direct routing over reps + partial, for every sublayer of the block."""
    r = _rng(8)
    N, S, T, d = 5, 4, 20, 8
    reps = r.standard_normal((N, T, d)) * (1 + 0.3 * np.arange(N))[:, None, None]
    partials = np.cumsum(r.standard_normal((S - 1, T, d)), axis=0)
    w = r.standard_normal((S, 4, d)) / np.sqrt(d)
    conv = r.standard_normal((24, d)) / 3
    P = r.standard_normal((S, 4 * d, 4)) / np.sqrt(4 * d)
    direct = mso.block_msar_direct(reps, partials, w, conv, P)
    h1, o, lse = mso.block_msar_phase1(reps, w, conv, P[0])
    np.testing.assert_allclose(h1, direct[0], rtol=1e-12, atol=1e-12)
    for i in range(2, S + 1):
        hi = mso.block_msar_phase2(o[i - 2], lse[i - 2], partials[i - 2], w[i - 1], conv, P[i - 1])
        np.testing.assert_allclose(hi, direct[i - 1], rtol=1e-11, atol=1e-12)


def pin_block_msar_merge_with_dominant_partial():
    """A partial whose score dominates every rep's makes each stream's merged
    state the partial's own stream (the reps' weight underflows): with one-tap
    streams and P = 0, h = 4 * (1/2) * partial.  One token; the query is a
    large multiple of the partial's normalised key, so by Cauchy-Schwarz its
    score exceeds every rep's by a wide margin."""
    r = _rng(9)
    N, T, d = 3, 1, 8
    reps = r.standard_normal((N, T, d))
    part = r.standard_normal((T, d))
    conv = np.zeros((24, d))
    conv[[0, 4, 12], :] = 1.0                        # one-tap streams: every stream is the source
    kp = aro.rms_normalise(part, 1e-6)[0]
    w = np.zeros((2, 4, d))
    w[1] = 60.0 * kp
    s_rep = aro.rms_normalise(reps, 1e-6)[:, 0] @ w[1, 0]
    assert kp @ w[1, 0] - s_rep.max() > 100.0        # the construction holds
    _, o, lse = mso.block_msar_phase1(reps, w, conv, np.zeros((4 * d, 4)))
    h2 = mso.block_msar_phase2(o[0], lse[0], part, w[1], conv, np.zeros((4 * d, 4)))
    np.testing.assert_allclose(h2, 2.0 * part, rtol=1e-12, atol=1e-12)


ALL_MSAR_PINS = [
    pin_msar_expand_is_causal_convolution, pin_msar_one_tap_streams_reduce_to_attnres, pin_msar_mixer_closed_form,
    pin_msar_identical_sources, pin_msar_token_window, pin_msar_magnitude_invariance, pin_msar_prefix_sets,
    pin_block_msar_two_phase_equals_direct, pin_block_msar_merge_with_dominant_partial,
]
