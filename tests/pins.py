"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each pin is a plain function that raises AssertionError when the oracle is
wrong.  test_oracle_pins.py runs them; test_oracle_mutations.py plants
plausible mistakes into the oracle and checks that some pin catches each one.
The pins never retype the oracle's formulas: they use printed values, closed
forms, invariants and finite differences.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import attnres_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "explainer_worked_example.json")


def _num(x) -> float:
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"sqrt": math.sqrt, "ln": math.log}))  # fixture arithmetic only


def golden():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    src = g["sources"]
    e, f1, f2 = (np.array(src[k], dtype=np.float64) for k in ("e", "f1", "f2"))
    return g, e, f1, f2


def _one_token(*vecs) -> np.ndarray:
    return np.stack([np.asarray(v, np.float64)[None, :] for v in vecs])  # [n, T=1, d]


# --- worked example (explainer: weights table, learned-query section) -------------------

def pin_rms_of_example():
    g, e, f1, f2 = golden()
    for name, v in (("e", e), ("f1", f1), ("f2", f2)):
        want = np.array([_num(x) for x in g["normalised"][name]])
        got = orc.rms_normalise(v[None, :], 0.0)[0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
        # the printed RMS is the ratio of the source to its normalised form
        k = int(np.argmax(np.abs(v)))
        assert abs(v[k] / got[k] - _num(g["rms"][name])) < 1e-15


def pin_learned_query_example():
    g, e, f1, f2 = golden()
    lq = g["learned_query"]
    w = np.array([_num(x) for x in lq["w"]])
    h, alpha, s = orc.depth_read(_one_token(e, f1, f2), w, np.ones(3), 0.0, 1)
    np.testing.assert_allclose(s[0, 0], [_num(x) for x in lq["scores"]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(np.exp(s[0, 0]), lq["exp_scores"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(alpha[0, 0], lq["alpha"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(h[0], lq["h"], rtol=0, atol=1e-15)


def pin_alternate_weights_example():
    g, e, f1, f2 = golden()
    alt = g["alternate_weights"]
    w = np.array([_num(x) for x in alt["w_alt"]])
    h, alpha, _ = orc.depth_read(_one_token(e, f1, f2), w, np.ones(3), 0.0, 1)
    np.testing.assert_allclose(alpha[0, 0], alt["alpha"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(h[0], alt["h"], rtol=0, atol=1e-15)


def pin_uniform_is_mean_not_sum():
    g, e, f1, f2 = golden()
    h, alpha, _ = orc.depth_read(_one_token(e, f1, f2), np.zeros(3), np.ones(3), 0.0, 1)
    np.testing.assert_allclose(h[0], [_num(x) for x in g["uniform_weights_mean"]], rtol=0, atol=1e-15)
    assert not np.allclose(h[0], g["plain_residual_sum"])
    # Zero query on random data: the output is the mean of the sources.
    rng = np.random.default_rng(5)
    V = rng.standard_normal((5, 7, 12)) * np.arange(1, 6)[:, None, None]
    for H in (1, 2, 3):
        h, _, _ = orc.depth_read(V, np.zeros(12), rng.standard_normal(12), 1e-6, H)
        np.testing.assert_allclose(h, V.mean(axis=0), rtol=0, atol=1e-14)


def pin_full_prefix_sets_example():
    """Full AttnRes destination l reads v_0..v_{l-1}: with the example sources and
    n_dst = n_src = 3, destination 1 returns e, destination 3 is the worked example."""
    g, e, f1, f2 = golden()
    lq = g["learned_query"]
    w3 = np.array([_num(x) for x in lq["w"]])
    W = np.stack([np.zeros(3), np.zeros(3), w3])
    out = orc.full_fwd(_one_token(e, f1, f2), W, None, 0.0, 1)
    np.testing.assert_allclose(out[0, 0], e, rtol=0, atol=0)               # single source
    np.testing.assert_allclose(out[1, 0], (e + f1) / 2, rtol=0, atol=1e-15)  # uniform over 2
    np.testing.assert_allclose(out[2, 0], lq["h"], rtol=0, atol=1e-15)
    # n_dst = 1 is the last destination only.
    out1 = orc.full_fwd(_one_token(e, f1, f2), w3[None, :], None, 0.0, 1)
    np.testing.assert_allclose(out1[0, 0], lq["h"], rtol=0, atol=1e-15)


# --- invariants -------------------------------------------------------------------------

def pin_magnitude_invariance():
    """With eps = 0 the score ignores a positive rescaling of a source
    (explainer learned-query section: normalisation removes pure magnitude)."""
    rng = np.random.default_rng(1)
    V = rng.standard_normal((4, 6, 16))
    w = rng.standard_normal(16) * 0.3
    gn = 1 + 0.1 * rng.standard_normal(16)
    _, a0, s0 = orc.depth_read(V, w, gn, 0.0, 1)
    V2 = V.copy()
    V2[2] *= 7.5
    _, a1, s1 = orc.depth_read(V2, w, gn, 0.0, 1)
    np.testing.assert_allclose(s1, s0, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(a1, a0, rtol=1e-13, atol=1e-13)


def pin_softmax_simplex_and_permutation():
    rng = np.random.default_rng(2)
    V = rng.standard_normal((6, 5, 24)) * 3
    w = rng.standard_normal(24)
    for H in (1, 2, 4):
        h, alpha, _ = orc.depth_read(V, w, np.ones(24), 1e-6, H)
        assert np.all(alpha > 0)
        np.testing.assert_allclose(alpha.sum(axis=-1), 1.0, rtol=0, atol=1e-14)
        perm = np.array([3, 0, 5, 1, 4, 2])
        hp, _, _ = orc.depth_read(V[perm], w, np.ones(24), 1e-6, H)
        np.testing.assert_allclose(hp, h, rtol=0, atol=1e-13)
        # the output stays inside the per-channel hull of the sources
        assert np.all(h <= V.max(axis=0) + 1e-12) and np.all(h >= V.min(axis=0) - 1e-12)


def pin_single_source_identity():
    rng = np.random.default_rng(3)
    V = rng.standard_normal((1, 9, 10))
    h, alpha, _ = orc.depth_read(V, rng.standard_normal(10), np.ones(10), 1e-6, 2)
    np.testing.assert_array_equal(alpha, 1.0)
    np.testing.assert_array_equal(h, V[0])


def pin_gain_fold_identity():
    """Forward depends on (w, g) only through w * g."""
    rng = np.random.default_rng(4)
    V = rng.standard_normal((5, 4, 32))
    w = rng.standard_normal(32) / 5
    gn = 1 + 0.2 * rng.standard_normal(32)
    h1, _, s1 = orc.depth_read(V, w, gn, 1e-6, 2)
    h2, _, s2 = orc.depth_read(V, w * gn, np.ones(32), 1e-6, 2)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h1, h2, rtol=1e-13, atol=1e-13)


# --- Block source sets (b-lab §2; explainer Block grouping section) ---------------------

def pin_block_grouping_example():
    g, e, f1, f2 = golden()
    f3 = np.array([1.0, -2.0, 0.5])  # not printed on the page; any value works
    rng = np.random.default_rng(6)
    w = rng.standard_normal((2, 3))
    reps = _one_token(e, f1 + f2)        # b_0 = e, b_1 = f1 + f2 (completed block)
    partials = _one_token(f3)            # b^(2)_1 = f3
    h = orc.block_direct(reps, partials, w, None, 0.0, 1)
    # first sublayer of block 2 (forms h3): reads [e, f1+f2] only, never an empty partial
    h3_want = orc.depth_read(_one_token(e, f1 + f2), w[0], np.ones(3), 0.0, 1)[0]
    np.testing.assert_allclose(h[0], h3_want, rtol=0, atol=1e-15)
    # second sublayer (forms h4): reads exactly [e, f1+f2, f3]
    h4_want = orc.depth_read(_one_token(e, f1 + f2, f3), w[1], np.ones(3), 0.0, 1)[0]
    np.testing.assert_allclose(h[1], h4_want, rtol=0, atol=1e-15)
    # a zero vector in place of the empty partial would change h3 (it would get weight e^0)
    h3_zero = orc.depth_read(_one_token(e, f1 + f2, np.zeros(3)), w[0], np.ones(3), 1e-6, 1)[0]
    assert not np.allclose(h3_zero, h[0])


def pin_block_s1_is_full():
    """Block size S = 1 is Full AttnRes (review: block-size sweep, S = 1 is Full)."""
    rng = np.random.default_rng(7)
    L, T, d = 6, 5, 16
    src = rng.standard_normal((L, T, d)) * (1 + 0.3 * np.arange(L))[:, None, None]
    W = rng.standard_normal((L, d)) / 4
    G = 1 + 0.1 * rng.standard_normal((L, d))
    full = orc.full_fwd(src, W, G, 1e-6, 1)
    for l in range(1, L + 1):
        # with S = 1 the block before destination l holds the l individual outputs
        hb = orc.block_direct(src[:l], np.zeros((0, T, d)), W[l - 1:l], G[l - 1:l], 1e-6, 1)
        np.testing.assert_allclose(hb[0], full[l - 1], rtol=0, atol=1e-14)


def pin_later_sources_do_not_leak():
    rng = np.random.default_rng(8)
    src = rng.standard_normal((5, 3, 8))
    W = rng.standard_normal((5, 8))
    out = orc.full_fwd(src, W, None, 1e-6, 2)
    src2 = src.copy()
    src2[3:] += 10.0
    out2 = orc.full_fwd(src2, W, None, 1e-6, 2)
    np.testing.assert_array_equal(out2[:3], out[:3])
    assert not np.allclose(out2[3], out[3])


# --- two-phase (review §3-2 (4): the merge is exact) ------------------------------------

def _block_case(seed, T=6, d=16, N=5, S=4, gain="per"):
    rng = np.random.default_rng(seed)
    reps = rng.standard_normal((N, T, d)) * (1 + 0.3 * np.arange(N))[:, None, None]
    partials = np.cumsum(rng.standard_normal((S - 1, T, d)), axis=0)
    w = rng.standard_normal((S, d)) / math.sqrt(d) * 3
    g = {"per": 1 + 0.1 * rng.standard_normal((S, d)), "shared": 1 + 0.1 * rng.standard_normal(d),
         None: None}[gain]
    return reps, partials, w, g


def pin_two_phase_equals_direct():
    for H in (1, 2, 4):
        for gain in ("per", "shared", None):
            reps, partials, w, g = _block_case(10 + H, gain=gain)
            direct = orc.block_direct(reps, partials, w, g, 1e-6, H)
            two = orc.block_two_phase(reps, partials, w, g, 1e-6, H)
            np.testing.assert_allclose(two, direct, rtol=1e-12, atol=1e-12)


def pin_fused_update_chain_equals_direct():
    """Running the fused merge-and-update through a block from a zero partial
    (b_1 = f_1, b_i = b_{i-1} + f_i) reproduces the plain definition, whose
    sublayer i reads the reps and the sum of f_1 .. f_{i-1} ([B-LAB] §2)."""
    for H, gain in ((1, "per"), (2, "shared"), (4, None)):
        rng = np.random.default_rng(60 + H)
        T, d, N, S = 5, 16, 4, 4
        reps = rng.standard_normal((N, T, d)) * (1 + 0.3 * np.arange(N))[:, None, None]
        f = rng.standard_normal((S - 1, T, d))
        w = rng.standard_normal((S, d)) / math.sqrt(d) * 3
        g = {"per": 1 + 0.1 * rng.standard_normal((S, d)), "shared": 1 + 0.1 * rng.standard_normal(d),
             None: None}[gain]
        direct = orc.block_direct(reps, np.cumsum(f, axis=0), w, g, 1e-6, H)
        o, lse = orc.block_phase1(reps, w, g, 1e-6, H)
        b = None
        for i in range(2, S + 1):
            gi = None if g is None else (g if g.ndim == 1 else g[i - 1])
            b, h, inv = orc.block_phase2_merge_update(o[i - 1], lse[i - 1], b, f[i - 2], w[i - 1], gi, 1e-6, H)
            np.testing.assert_allclose(b, f[:i - 1].sum(axis=0), rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(h, direct[i - 1], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(inv, 1 / np.sqrt(np.mean(direct[i - 1] ** 2, axis=-1) + 1e-6), rtol=1e-12)


def pin_fused_update_rms_example():
    """With o_i equal to the partial the merge is a convex combination of two
    equal vectors, so h = partial exactly; for e = [2, 0, 0] the PreNorm
    statistic is the explainer's RMS([2, 0, 0]) = 2 / sqrt(3) (learned-query
    section), i.e. inv_rms = sqrt(3) / 2 with eps 0."""
    e = np.array([[2.0, 0.0, 0.0]])
    for w in ([0.0, 0.0, 0.0], [0.3, -1.0, 2.0]):
        b, h, inv = orc.block_phase2_merge_update(e, np.array([[0.7]]), None, e, np.array(w), None, 0.0, 1, 0.0)
        np.testing.assert_array_equal(b, e)
        np.testing.assert_allclose(h, e, rtol=0, atol=1e-15)
        np.testing.assert_allclose(inv, [math.sqrt(3) / 2], rtol=1e-15)


# --- MHAR (H heads; H = 1 is AttnRes exactly) -------------------------------------------

def pin_mhar_h1_is_attnres():
    reps, partials, w, g = _block_case(20)
    a = orc.mhar_fwd(reps, partials, w, g, 1e-6, 1)
    S = w.shape[0]
    for i in range(1, S + 1):
        V = reps if i == 1 else np.concatenate([reps, partials[i - 2][None]])
        h, _, _ = orc.depth_read(V, w[i - 1], g[i - 1], 1e-6, 1)
        np.testing.assert_allclose(a[i - 1], h, rtol=0, atol=1e-15)


def pin_mhar_per_head_worked_example():
    """Two heads, each a copy of the worked example's sources: head 0 uses the
    learned-query w, head 1 the alternate-weights w, so the output chunks are
    the two printed results.  The tiling keeps the full-width RMS equal to the
    3-wide one, so the example's scores carry over unchanged."""
    g, e, f1, f2 = golden()
    w0 = np.array([_num(x) for x in g["learned_query"]["w"]])
    w1 = np.array([_num(x) for x in g["alternate_weights"]["w_alt"]])
    V = _one_token(np.tile(e, 2), np.tile(f1, 2), np.tile(f2, 2))
    h, alpha, _ = orc.depth_read(V, np.concatenate([w0, w1]), np.ones(6), 0.0, 2)
    np.testing.assert_allclose(alpha[0, 0], g["learned_query"]["alpha"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(alpha[0, 1], g["alternate_weights"]["alpha"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(h[0, :3], g["learned_query"]["h"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(h[0, 3:], g["alternate_weights"]["h"], rtol=0, atol=1e-15)


def pin_mhar_zero_query_heads_are_means():
    rng = np.random.default_rng(21)
    H, d = 4, 16
    V = rng.standard_normal((5, 3, d)) * 2
    w = np.zeros(d)
    w[4:8] = rng.standard_normal(4)      # only head 1 has a non-zero query
    h, alpha, _ = orc.depth_read(V, w, np.ones(d), 1e-6, H)
    mean = V.mean(axis=0)
    for hh in (0, 2, 3):
        np.testing.assert_allclose(h[:, hh * 4:(hh + 1) * 4], mean[:, hh * 4:(hh + 1) * 4], rtol=0, atol=1e-14)
        np.testing.assert_allclose(alpha[:, hh], 0.2, rtol=0, atol=1e-15)
    assert not np.allclose(h[:, 4:8], mean[:, 4:8])


# --- backward -----------------------------------------------------------------------------

def _bwd_case(seed, H, gain):
    T, d, N, S = 4, 16, 8, 4
    reps, partials, w, g = _block_case(seed, T=T, d=d, N=N, S=S, gain=gain)
    dh = np.random.default_rng(seed + 100).standard_normal((S, T, d))
    return reps, partials, w, g, dh


def pin_bwd_finite_differences(H=1, gain="per", eps=1e-6):
    reps, partials, w, g, dh = _bwd_case(30 + H, H, gain)
    an = orc.block_bwd(reps, partials, w, g, eps, H, dh)
    fd = orc.finite_difference_grads(reps, partials, w, g, eps, H, dh, step=1e-6)
    for name, a, f in zip(("d_reps", "d_partials", "dw", "dgain"), an, fd):
        if f is None:
            assert a is None, name
            continue
        scale = max(1.0, float(np.max(np.abs(f))))
        err = float(np.max(np.abs(a - f))) / scale
        assert err < 1e-6, f"{name}: {err}"


def pin_bwd_closed_forms():
    """Identities of the derived gradient:
    (1) sum_i c_{j,i,h} = 0 for every destination and head;
    (2) v_i . dv_i = sum_j sum_k alpha_{j,i,h(k)} dh_j[k] v_i[k] + eps r_i^2 sum_{j,h} c s
        (the normalisation path is orthogonal to v_i up to the eps term);
    (3) dw_j * w_j == dg_j * g_j for a per-destination gain."""
    H, eps = 2, 1e-3
    reps, partials, w, g, dh = _bwd_case(40, H, "per")
    d_reps, d_partials, dw, dg = orc.block_bwd(reps, partials, w, g, eps, H, dh)
    np.testing.assert_allclose(dw * w, dg * g, rtol=1e-12, atol=1e-14)
    S, T, d = dh.shape
    N = reps.shape[0]
    hd = d // H
    rhs_reps = np.zeros((N, T))
    for j in range(S):
        V = orc.block_sources(reps, partials, j + 1)
        n = V.shape[0]
        _, alpha, s = orc.depth_read(V, w[j], g[j], eps, H)
        a = np.einsum("thk,nthk->thn", dh[j].reshape(T, H, hd), V.reshape(n, T, H, hd))
        c = alpha * (a - np.sum(alpha * a, axis=-1, keepdims=True))
        np.testing.assert_allclose(c.sum(axis=-1), 0.0, rtol=0, atol=1e-13)
        r2 = 1.0 / (np.mean(V * V, axis=-1) + eps)            # r_i^2, [n, T]
        # sum_k alpha_{j,i,h(k)} dh_j[k] v_i[k] = sum_h alpha_{j,i,h} a_{j,i,h}
        rhs = np.einsum("thn,thn->nt", alpha, a) + eps * r2 * np.einsum("thn,thn->nt", c, s)
        rhs_reps += rhs[:N]
        if n > N:
            lhs_p = np.sum(partials[j - 1] * d_partials[j - 1], axis=-1)
            np.testing.assert_allclose(lhs_p, rhs[N], rtol=1e-11, atol=1e-11)
    lhs_reps = np.sum(reps * d_reps, axis=-1)
    np.testing.assert_allclose(lhs_reps, rhs_reps, rtol=1e-11, atol=1e-11)


def _full_bwd_case(seed, H, gain, n_src=5, n_dst=5, T=3, d=8):
    rng = np.random.default_rng(seed)
    src = rng.standard_normal((n_src, T, d)) * (1.0 + 0.3 * np.arange(n_src))[:, None, None]
    w = rng.standard_normal((n_dst, d)) * 0.7
    if gain == "per":
        g = 1.0 + 0.1 * rng.standard_normal((n_dst, d))
    elif gain == "shared":
        g = 1.0 + 0.1 * rng.standard_normal(d)
    else:
        g = None
    dout = rng.standard_normal((n_dst, T, d))
    return src, w, g, dout


def pin_full_bwd_finite_differences(H=1, gain="per", n_dst=5, eps=1e-6):
    """full_bwd against central differences of full_loss (forward only)."""
    src, w, g, dout = _full_bwd_case(50 + H + n_dst, H, gain, n_dst=n_dst)
    an = orc.full_bwd(src, w, g, eps, H, dout)
    fd = orc.full_finite_difference_grads(src, w, g, eps, H, dout, step=1e-6)
    for name, a, f in zip(("d_src", "dw", "dgain"), an, fd):
        if f is None:
            assert a is None, name
            continue
        scale = max(1.0, float(np.max(np.abs(f))))
        err = float(np.max(np.abs(a - f))) / scale
        assert err < 1e-6, f"{name}: {err}"


def pin_full_bwd_single_source():
    """One source, one destination: alpha = 1 whatever the score, so the
    gradient is dout itself and nothing reaches the query or the gain."""
    src, w, g, dout = _full_bwd_case(61, 1, "per", n_src=1, n_dst=1, T=4, d=8)
    d_src, dw, dg = orc.full_bwd(src, w, g, 1e-6, 1, dout)
    np.testing.assert_array_equal(d_src, dout)
    np.testing.assert_array_equal(dw, 0.0)
    np.testing.assert_array_equal(dg, 0.0)


def pin_full_bwd_block_s1_identity():
    """A Block with S = 1 reads exactly its N reps, which is Full with one
    destination over N sources ([REVIEW] §5 block-size sweep: S = 1 is Full),
    so the two derived backwards agree; dw * w == dg * g per destination."""
    src, w, g, dout = _full_bwd_case(62, 2, "per", n_src=6, n_dst=1, T=3, d=8)
    d_src, dw, dg = orc.full_bwd(src, w, g, 1e-6, 2, dout)
    d_reps, d_parts, dw_b, dg_b = orc.block_bwd(src, np.zeros((0, 3, 8)), w, g, 1e-6, 2, dout)
    np.testing.assert_allclose(d_src, d_reps, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, dw_b, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dg, dg_b, rtol=1e-12, atol=1e-13)
    src, w, g, dout = _full_bwd_case(63, 1, "per")
    _, dw, dg = orc.full_bwd(src, w, g, 1e-3, 1, dout)
    np.testing.assert_allclose(dw * w, dg * g, rtol=1e-12, atol=1e-14)


def pin_tolerance_error():
    y_ref = np.array([3.0, -4.0, 0.0, 0.0])      # RMS = 2.5
    y = y_ref + np.array([0.0, 0.05, 0.0, -0.01])
    assert abs(orc.tolerance_error(y, y_ref) - 0.02) < 1e-15


ALL_FORWARD_PINS = [
    pin_rms_of_example, pin_learned_query_example, pin_alternate_weights_example,
    pin_uniform_is_mean_not_sum, pin_full_prefix_sets_example, pin_magnitude_invariance,
    pin_softmax_simplex_and_permutation, pin_single_source_identity, pin_gain_fold_identity,
    pin_block_grouping_example, pin_block_s1_is_full, pin_later_sources_do_not_leak,
    pin_two_phase_equals_direct, pin_mhar_h1_is_attnres, pin_mhar_per_head_worked_example,
    pin_mhar_zero_query_heads_are_means, pin_fused_update_chain_equals_direct, pin_fused_update_rms_example,
]
ALL_BACKWARD_PINS = [
    lambda: pin_bwd_finite_differences(1, "per"),
    lambda: pin_bwd_finite_differences(2, "shared"),
    pin_bwd_closed_forms,
]
ALL_FULL_BACKWARD_PINS = [
    lambda: pin_full_bwd_finite_differences(1, "per", 5),
    lambda: pin_full_bwd_finite_differences(2, "shared", 3),
    pin_full_bwd_single_source,
    pin_full_bwd_block_s1_identity,
]
