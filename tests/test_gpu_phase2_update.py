"""Parity of the fused Phase 2 update (attnres_block_phase2_merge_update) with
the oracle on MI355X.

Inputs are one block's synthetic reps and sublayer outputs f; the HIP side runs
Phase 1 and then the fused update, the oracle runs its own Phase 1 and
block_phase2_merge_update on the same numbers.  Tolerances:
  partial_out, h_i : the output bars (bf16: excess over half an ulp <= 2e-2 of
                     the RMS; fp32: max-abs <= 1e-5 of the RMS);
  h_inv_rms        : taken over the stored h_i.  Rounding h_i to bf16 moves
                     each element by at most 2^-8 relative, so the statistic
                     moves by at most about 2^-8 relative: rtol 4e-3 for bf16
                     (1e-5 for fp32) against the oracle, and rtol 2e-5 against
                     the fp64 statistic of the stored h_i itself (fp32
                     accumulation over d <= 4096 terms).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import depth_wise_attention_amd as ar  # noqa: E402
from metrics import check  # noqa: E402
from oracle import attnres_oracle as orc  # noqa: E402
from workloads import synth  # noqa: E402

DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
NORM_EPS = 1e-5


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, dtype="f32"):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t if dtype == "f32" else t.to(TDT[dtype])


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@pytest.fixture(params=[0, 1], ids=["auto", "general"])
def policy(request):
    prev = ar.attnres_set_kernel_policy(request.param)
    yield request.param
    ar.attnres_set_kernel_policy(prev)


def _gain(wl, kind, rng):
    if kind == "none":
        return None
    if kind == "shared":
        return (1 + 0.1 * rng.standard_normal(wl.d)).astype(np.float32)
    return wl.gain


def _row(g, i):
    """Gain row of sublayer i (1-based) for a [S, d], [d] or absent gain."""
    if g is None:
        return None
    return g if g.ndim == 1 else g[i - 1]


def _check_rms(got, h_stored, ref_rms, dtype):
    got = host(got)
    own = 1.0 / np.sqrt(np.mean(h_stored * h_stored, axis=-1) + NORM_EPS)
    np.testing.assert_allclose(got, own, rtol=2e-5, atol=0)
    np.testing.assert_allclose(got, ref_rms, rtol=4e-3 if dtype == "bf16" else 1e-5, atol=0)


UPDATE_CASES = [
    # T, d, H, dtype, state, with_prev, gain, rms
    (1, 64, 1, "bf16", "f16", True, "per", True),
    (37, 64, 1, "f32", "f32", True, "per", True),
    (100, 512, 1, "bf16", "f16", True, "per", True),
    (130, 4096, 1, "bf16", "f16", True, "per", True),
    (130, 4096, 1, "bf16", "f16", False, "per", True),
    (67, 2048, 2, "bf16", "f32", True, "shared", True),
    (65, 4096, 8, "bf16", "f16", True, "none", False),
    (300, 2048, 4, "bf16", "f32", False, "per", True),
    (40, 4096, 16, "bf16", "f16", False, "per", True),
    (12, 96, 3, "f32", "f32", False, "per", False),
    (257, 4096, 1, "bf16", "f32", True, "per", True),
]


@pytest.mark.parametrize("T,d,H,dtype,state,with_prev,gain,rms", UPDATE_CASES)
def test_update_shapes(T, d, H, dtype, state, with_prev, gain, rms, policy):
    say(f"phase2 update T={T} d={d} H={H} {dtype} state={state} prev={with_prev} gain={gain} "
        f"rms={rms} policy={policy}")
    wl = synth.block_workload(T=T, d=d, N=8, S=4, H=H, rep_std_step=0.3, dtype=dtype, seed=21, with_f=True)
    g = _gain(wl, gain, np.random.default_rng(4))
    i = 3 if with_prev else 2                    # the sublayer whose input is merged
    prev = wl.partials[i - 3] if with_prev else None
    f = wl.f[i - 2]
    o_ref, lse_ref = orc.block_phase1(wl.reps, wl.w, g, wl.eps, H)
    p_ref, h_ref, rms_ref = orc.block_phase2_merge_update(o_ref[i - 1], lse_ref[i - 1], prev, f, wl.w[i - 1],
                                                          _row(g, i), wl.eps, H, NORM_EPS)

    reps, w, gg = dev(wl.reps, dtype), dev(wl.w), dev(g)
    _, o_state, lse, o_scale = ar.attnres_block_phase1(reps, w, gg, wl.eps, H, o_dtype=TDT[state])
    g_i = None if gg is None else (gg if gg.dim() == 1 else gg[i - 1])
    prev_d = dev(prev, dtype)
    p_out, h, r = ar.attnres_block_phase2_merge_update(
        o_state[i - 2], lse[i - 1], prev_d, dev(f, dtype), w[i - 1], g_i, wl.eps, H, norm_eps=NORM_EPS,
        h_inv_rms=None if rms else False, o_scale=o_scale)
    check(host(p_out), p_ref, dtype, "partial_out")
    check(host(h), h_ref, dtype, "h_i")
    if rms:
        _check_rms(r, host(h), rms_ref, dtype)
    else:
        assert r is None
    # The merge reads the stored partial: identical to the plain merge of it.
    plain = ar.attnres_block_phase2_merge(o_state[i - 2], lse[i - 1], p_out, w[i - 1], g_i, wl.eps, H,
                                          o_scale=o_scale)
    assert torch.equal(plain, h), "fused merge differs from the plain merge of the stored partial"
    if prev_d is not None:
        assert torch.equal(prev_d, dev(prev, dtype)), "partial_prev was written"


@pytest.mark.parametrize("state", ["f32", "f16"])
def test_update_in_place(state, policy):
    """partial_out == partial_prev, and h_i == o_i for the scaled fp16 state (the
    I/O element size): same bits as out of place."""
    wl = synth.block_workload(T=300, d=4096, N=8, S=4, H=2, rep_std_step=0.3, dtype="bf16", seed=22, with_f=True)
    say(f"phase2 update in place state={state} T={wl.T} policy={policy}")
    reps, w, g = dev(wl.reps, "bf16"), dev(wl.w), dev(wl.gain)
    _, o, lse, sc = ar.attnres_block_phase1(reps, w, g, wl.eps, 2, o_dtype=TDT[state])
    prev, f = dev(wl.partials[0], "bf16"), dev(wl.f[1], "bf16")
    p_ref, h_ref, r_ref = ar.attnres_block_phase2_merge_update(o[1], lse[2], prev, f, w[2], g[2], wl.eps, 2,
                                                               norm_eps=NORM_EPS, o_scale=sc)
    p = prev.clone()
    h_out = o[1] if state == "f16" else None
    _, h, r = ar.attnres_block_phase2_merge_update(o[1], lse[2], p, f, w[2], g[2], wl.eps, 2, partial_out=p,
                                                   h_i=h_out, norm_eps=NORM_EPS, o_scale=sc)
    if state == "f16":
        h = h.view(torch.bfloat16)
        assert h.data_ptr() == o[1].data_ptr()
    assert torch.equal(p, p_ref)
    assert torch.equal(h, h_ref)
    assert torch.equal(r, r_ref)


@pytest.mark.parametrize("d,H", [(4096, 1), (2048, 4), (192, 3)])
def test_update_chain(d, H, policy):
    """A whole block as the model runs it: b_1 = f_1, b_i = b_{i-1} + f_i, kept in
    one bf16 buffer updated in place, each sublayer's input from the fused call.

    The running partial is stored in the I/O dtype after every update, so the
    oracle chain is fed its own partial rounded to bf16 (the storage format)
    before the next call; each call is then held to the per-call bar, and the
    stored partials must match bit for bit (the sum of two bf16 numbers is
    rounded once on both sides)."""
    S = 5
    wl = synth.block_workload(T=129, d=d, N=6, S=S, H=H, rep_std_step=0.3, dtype="bf16", seed=23, with_f=True)
    say(f"phase2 update chain d={d} H={H} S={S} policy={policy}")
    o_ref, lse_ref = orc.block_phase1(wl.reps, wl.w, wl.gain, wl.eps, H)
    reps, w, g = dev(wl.reps, "bf16"), dev(wl.w), dev(wl.gain)
    _, o, lse, sc = ar.attnres_block_phase1(reps, w, g, wl.eps, H, o_dtype=torch.float16)
    p_dev = torch.empty((wl.T, d), dtype=torch.bfloat16, device=DEV)
    p_ref = None
    for i in range(2, S + 1):
        p_ref, h_ref, r_ref = orc.block_phase2_merge_update(o_ref[i - 1], lse_ref[i - 1], p_ref, wl.f[i - 2],
                                                            wl.w[i - 1], wl.gain[i - 1], wl.eps, H, NORM_EPS)
        _, h, r = ar.attnres_block_phase2_merge_update(o[i - 2], lse[i - 1], None if i == 2 else p_dev,
                                                       dev(wl.f[i - 2], "bf16"), w[i - 1], g[i - 1], wl.eps, H,
                                                       partial_out=p_dev, norm_eps=NORM_EPS, o_scale=sc)
        p_ref = synth.bf16_round(p_ref.astype(np.float32))
        np.testing.assert_array_equal(host(p_dev), p_ref, err_msg=f"b_{i - 1}")
        check(host(h), h_ref, "bf16", f"h_{i}")
        _check_rms(r, host(h), r_ref, "bf16")


def test_update_empty():
    say("phase2 update T=0")
    z = torch.empty((0, 4096), dtype=torch.bfloat16, device=DEV)
    o = torch.empty((0, 4096), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, 0), dtype=torch.float32, device=DEV)
    w = torch.zeros(4096, dtype=torch.float32, device=DEV)
    p, h, r = ar.attnres_block_phase2_merge_update(o, lse, z, z, w)
    assert p.shape == (0, 4096) and h.shape == (0, 4096) and r.shape == (0,)


def test_update_config_sampled():
    """Block two-phase bf16 at full size (T=16384, d=4096, N=8, S=4): the fused
    update of sublayer 3 over every token, checked on sampled tokens."""
    wl = synth.block_workload(T=16384, d=4096, N=8, S=4, H=1, rep_std_step=0.3, dtype="bf16", seed=0,
                              with_f=True)
    say(f"phase2 update full size T={wl.T} d={wl.d} (sampled tokens)")
    reps, w, g = dev(wl.reps, "bf16"), dev(wl.w), dev(wl.gain)
    _, o, lse, sc = ar.attnres_block_phase1(reps, w, g, wl.eps, 1, o_dtype=torch.float16)
    prev, f = dev(wl.partials[0], "bf16"), dev(wl.f[1], "bf16")
    p, h, r = ar.attnres_block_phase2_merge_update(o[1], lse[2], prev, f, w[2], g[2], wl.eps, 1,
                                                   norm_eps=NORM_EPS, o_scale=sc)
    p2, h2, r2 = ar.attnres_block_phase2_merge_update(o[1], lse[2], prev, f, w[2], g[2], wl.eps, 1,
                                                      norm_eps=NORM_EPS, o_scale=sc)
    assert torch.equal(h, h2) and torch.equal(p, p2) and torch.equal(r, r2), "not deterministic"
    idx = synth.sample_tokens(wl.T, 96)
    o_ref, lse_ref = orc.block_phase1(synth.take_tokens(wl.reps, idx), wl.w, wl.gain, wl.eps, 1)
    p_ref, h_ref, r_ref = orc.block_phase2_merge_update(o_ref[2], lse_ref[2], wl.partials[0][idx], wl.f[1][idx],
                                                        wl.w[2], wl.gain[2], wl.eps, 1, NORM_EPS)
    it = torch.from_numpy(idx).to(DEV)
    check(host(p[it]), p_ref, "bf16", "partial_out (sampled)")
    check(host(h[it]), h_ref, "bf16", "h_3 (sampled)")
    _check_rms(r[it], host(h[it]), r_ref, "bf16")
