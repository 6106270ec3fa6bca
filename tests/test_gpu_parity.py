"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Small shapes are compared element by element over every output; the five
benchmark workloads run at full size and are compared on sampled tokens
(tokens are independent in every forward op and in the per-token gradients),
with token reductions (dw, dgain) checked through properties that hold at any
size plus exact parity at a smaller T.  Every case prints its name and shape
before touching the GPU.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import depth_wise_attention_amd as ar  # noqa: E402
from metrics import check, bf16_excess_over_rms, max_abs_over_rms  # noqa: E402
from oracle import attnres_oracle as orc  # noqa: E402
from workloads import synth  # noqa: E402

DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


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


def _gain_arg(wl_gain, kind, rows, d, rng):
    if kind == "none":
        return None
    if kind == "shared":
        return (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return wl_gain if wl_gain is not None else (1 + 0.1 * rng.standard_normal((rows, d))).astype(np.float32)


# ----------------------------------------------------------------- worked example
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hand_example(dtype, policy):
    """ai-systems-engineering explainer: e, f1, f2 with w = [0, ln2/sqrt3, 0] -> [0.5, 2, 1.5];
    w = [ln2/sqrt3, 0, 0] -> [1, 1, 1.5]; gain 1, eps 0."""
    say(f"hand example dtype={dtype} policy={policy}")
    src = np.array([[[2, 0, 0]], [[0, 4, 0]], [[0, 0, 6]]], dtype=np.float32)
    c = math.log(2) / math.sqrt(3)
    for w, want in (([0, c, 0], [0.5, 2, 1.5]), ([c, 0, 0], [1, 1, 1.5])):
        out = ar.attnres_full_fwd(dev(src, dtype), dev(np.array([w], np.float32)), eps=0.0)
        np.testing.assert_allclose(host(out)[0, 0], want, rtol=0, atol=1e-6)
    # all three prefixes: destination 1 reads e only (alpha = 1, exact)
    W = np.array([[0, 0, 0], [0, 0, 0], [0, c, 0]], np.float32)
    out = host(ar.attnres_full_fwd(dev(src, dtype), dev(W), eps=0.0))
    np.testing.assert_array_equal(out[0, 0], [2, 0, 0])
    np.testing.assert_allclose(out[1, 0], [1, 2, 0], rtol=0, atol=1e-6)
    np.testing.assert_allclose(out[2, 0], [0.5, 2, 1.5], rtol=0, atol=1e-6)


# ----------------------------------------------------------------- Full AttnRes
def test_full_fp32_config(policy):
    """Full AttnRes fp32, T=64, d=64, L=8, gain 1, eps 1e-6."""
    wl = synth.config_full_fp32_small()
    say(f"full fp32 T={wl.T} d={wl.d} L=8 policy={policy}")
    ref = orc.full_fwd(wl.src, wl.w, wl.gain, wl.eps, wl.H)
    out = ar.attnres_full_fwd(dev(wl.src), dev(wl.w), None, wl.eps, wl.H)
    check(host(out), ref, "f32", "full fp32")


@pytest.mark.parametrize("T,d,L,n_dst,H,dtype,gain", [
    (37, 64, 5, 5, 1, "bf16", "per"),
    (70, 128, 9, 3, 2, "bf16", "shared"),
    (5, 24, 4, 1, 3, "f32", "per"),
    (130, 2048, 6, 6, 1, "bf16", "per"),
    (9, 2048, 32, 32, 4, "bf16", "none"),
    (1, 16, 64, 2, 1, "f32", "none"),
    (33, 1000, 3, 3, 5, "bf16", "per"),
    # single-head bf16 with n_src <= 32 and d % 512 == 0: the matrix-core kernel under "auto"
    (67, 512, 32, 32, 1, "bf16", "per"),
    (300, 1024, 32, 1, 1, "bf16", "shared"),
    (45, 4096, 17, 9, 1, "bf16", "none"),
    (3, 1536, 1, 1, 1, "bf16", "per"),
    (513, 2560, 32, 32, 1, "bf16", "per"),
    (20, 512, 33, 33, 1, "bf16", "per"),
    (11, 768, 32, 32, 1, "bf16", "per"),
])
def test_full_shapes(T, d, L, n_dst, H, dtype, gain, policy):
    say(f"full T={T} d={d} L={L} n_dst={n_dst} H={H} {dtype} gain={gain} policy={policy}")
    wl = synth.full_workload(T=T, d=d, L=L, std_step=0.2, dtype=dtype, seed=3, gain_variance=0.02,
                             n_dst=n_dst)
    g = _gain_arg(wl.gain, gain, n_dst, d, np.random.default_rng(1))
    ref = orc.full_fwd(wl.src, wl.w, g, wl.eps, H)
    out = ar.attnres_full_fwd(dev(wl.src, dtype), dev(wl.w), dev(g), wl.eps, H)
    check(host(out), ref, dtype, "full")


def test_full_workspace_reuse(policy):
    """One caller-owned workspace across calls with different queries and destination counts."""
    say(f"full workspace reuse T=96 d=1024 L=24 policy={policy}")
    ws = torch.empty(ar.attnres_full_fwd_workspace_size(24, 24, 1024, 1, ar.BF16), dtype=torch.uint8,
                     device=DEV)
    assert ws.numel() == 2 * 32 * 1024 * 2
    for seed, n_dst in ((5, 24), (6, 7)):
        wl = synth.full_workload(T=96, d=1024, L=24, std_step=0.2, dtype="bf16", seed=seed,
                                 gain_variance=0.02, n_dst=n_dst)
        ref = orc.full_fwd(wl.src, wl.w, wl.gain, wl.eps, 1)
        out = ar.attnres_full_fwd(dev(wl.src, "bf16"), dev(wl.w), dev(wl.gain), wl.eps, 1, ws=ws)
        check(host(out), ref, "bf16", f"full ws reuse n_dst={n_dst}")


def test_full_bf16_config_sampled():
    """Full AttnRes bf16 at full size: T=4096, d=2048, L=32, every destination."""
    wl = synth.config_full_bf16()
    say(f"full bf16 T={wl.T} d={wl.d} L=32 (sampled tokens)")
    out = host(ar.attnres_full_fwd(dev(wl.src, "bf16"), dev(wl.w), dev(wl.gain), wl.eps, 1))
    idx = synth.sample_tokens(wl.T, 96)
    ref = orc.full_fwd(synth.take_tokens(wl.src, idx), wl.w, wl.gain, wl.eps, 1)
    err = check(out[:, idx], ref, "bf16", "full bf16 config")
    print(f"  full bf16: excess/RMS {err:.2e}, raw max-abs/RMS {max_abs_over_rms(out[:, idx], ref):.2e}")


# ----------------------------------------------------------------- Block two-phase / MHAR
def _block_on_gpu(wl, dtype, gain):
    return (dev(wl.reps, dtype), dev(wl.partials, dtype) if wl.S > 1 else None, dev(wl.w), dev(gain))


@pytest.mark.parametrize("T,d,N,S,H,dtype,gain", [
    (1, 64, 8, 4, 1, "bf16", "per"),
    (37, 64, 3, 2, 1, "f32", "per"),
    (100, 512, 8, 4, 1, "bf16", "per"),
    (67, 512, 8, 4, 2, "bf16", "shared"),
    (130, 4096, 8, 4, 1, "bf16", "per"),
    (130, 4096, 8, 4, 8, "bf16", "per"),
    (65, 2048, 9, 6, 4, "bf16", "none"),
    (20, 4096, 1, 3, 1, "bf16", "per"),
    (12, 96, 5, 1, 3, "f32", "per"),
    (40, 4096, 8, 4, 16, "bf16", "per"),
    (9, 16, 8, 4, 16, "f32", "shared"),
])
def test_block_shapes(T, d, N, S, H, dtype, gain, policy):
    say(f"block T={T} d={d} N={N} S={S} H={H} {dtype} gain={gain} policy={policy}")
    wl = synth.block_workload(T=T, d=d, N=N, S=S, H=H, rep_std_step=0.3, dtype=dtype, seed=5)
    g = _gain_arg(wl.gain, gain, S, d, np.random.default_rng(2))
    ref = orc.block_direct(wl.reps, wl.partials, wl.w, g, wl.eps, H)
    reps, parts, w, gg = _block_on_gpu(wl, dtype, g)
    h = ar.mhar_fwd(reps, parts, w, gg, wl.eps, H)
    check(host(h), ref, dtype, "mhar_fwd")
    # The public two-phase calls are exactly mhar_fwd's launches: bit-identical.
    state_dt = torch.float16 if dtype == "bf16" else torch.float32
    h_first, o_state, lse, o_scale = ar.attnres_block_phase1(reps, w, gg, wl.eps, H, o_dtype=state_dt)
    assert torch.equal(h_first, h[0]), "phase 1 h_first differs from mhar_fwd"
    for i in range(2, S + 1):
        hi = ar.attnres_block_phase2_merge(o_state[i - 2], lse[i - 1], parts[i - 2], w[i - 1],
                                           None if gg is None else (gg if gg.dim() == 1 else gg[i - 1]),
                                           wl.eps, H, o_scale=o_scale)
        assert torch.equal(hi, h[i - 1]), f"phase 2 of sublayer {i} differs from mhar_fwd"
    # Phase 1 state (fp32) and statistics against the oracle's two-phase check function.
    _, o32, lse32, _ = ar.attnres_block_phase1(reps, w, gg, wl.eps, H, o_dtype=torch.float32)
    o_ref, lse_ref = orc.block_phase1(wl.reps, wl.w, g, wl.eps, H)
    check(host(o32), o_ref[1:], "f32" if dtype == "f32" else "f32_from_bf16", "phase1 state")
    np.testing.assert_allclose(host(lse32), lse_ref, rtol=0, atol=1e-4 if dtype == "bf16" else 2e-5)
    if dtype == "bf16" and S > 1:
        # scaled fp16 state: stored * scale is the fp32 state rounded to fp16, i.e.
        # within half an fp16 ulp (2^-11 relative) plus fp32 arithmetic slack
        back = host(o_state) * host(o_scale)[None, :, None]
        bound = 2.0 ** -11 * np.abs(o_ref[1:]) * (1 + 1e-3) + 1e-5 * np.sqrt(np.mean(o_ref[1:] ** 2))
        assert np.all(np.abs(back - o_ref[1:]) <= bound)


@pytest.mark.parametrize("state", ["f32", "f16"])
def test_two_phase_state_formats(state, policy):
    """Every state format through the public calls, against the plain definition."""
    wl = synth.block_workload(T=257, d=4096, N=8, S=4, H=1, rep_std_step=0.3, dtype="bf16", seed=12)
    say(f"state format {state} T={wl.T} policy={policy}")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    sdt = {"f32": torch.float32, "f16": torch.float16}[state]
    h_first, o_state, lse, o_scale = ar.attnres_block_phase1(reps, w, g, wl.eps, 1, o_dtype=sdt)
    ref = orc.block_direct(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, 1)
    check(host(h_first), ref[0], "bf16", "h1")
    errs = []
    for i in range(2, 5):
        hi = ar.attnres_block_phase2_merge(o_state[i - 2], lse[i - 1], parts[i - 2], w[i - 1], g[i - 1], wl.eps, 1,
                                           o_scale=o_scale)
        errs.append(bf16_excess_over_rms(host(hi), ref[i - 1]))
    print(f"  state {state}: excess/RMS " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= 2e-2
    if state == "f32":
        assert max(errs) < 1e-3


def test_bf16_state_is_refused():
    """A bf16 Phase-1 state would miss the bf16 bar at full size: refused before any launch."""
    wl = synth.block_workload(T=8, d=512, N=8, S=4, H=1, rep_std_step=0.3, dtype="bf16", seed=12)
    say("bf16 state refused")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    with pytest.raises(ar.AttnResError) as e:
        ar.attnres_block_phase1(reps, w, g, wl.eps, 1, o_dtype=torch.bfloat16)
    assert e.value.code == -2
    o = torch.zeros((8, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((1, 8), device=DEV)
    with pytest.raises(ar.AttnResError) as e:
        ar.attnres_block_phase2_merge(o, lse, parts[0], w[1], g[1], wl.eps, 1)
    assert e.value.code == -2


@pytest.mark.parametrize("magnitude", [1e-7, 1.0, 3e4, 1e12])
def test_scaled_state_range(magnitude, policy):
    """The per-token scale keeps the fp16 state finite and accurate for tiny and
    huge activations (fp16 alone would flush 1e-7 to zero and overflow past 65504)."""
    wl = synth.block_workload(T=64, d=2048, N=8, S=4, H=2, rep_std_step=0.3, dtype="bf16", seed=13)
    say(f"scaled state magnitude={magnitude} policy={policy}")
    reps_h = synth.bf16_round((wl.reps * np.float32(magnitude)).astype(np.float32))
    parts_h = synth.bf16_round((wl.partials * np.float32(magnitude)).astype(np.float32))
    ref = orc.block_direct(reps_h, parts_h, wl.w, wl.gain, wl.eps, 2)
    h = host(ar.mhar_fwd(dev(reps_h, "bf16"), dev(parts_h, "bf16"), dev(wl.w), dev(wl.gain), wl.eps, 2))
    assert np.all(np.isfinite(h))
    for i in range(4):
        check(h[i], ref[i], "bf16", f"h{i + 1} at magnitude {magnitude}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_phase2_in_place(dtype, policy):
    """In-place merge (h_i == o_i) with a state of the I/O element size (the
    scaled fp16 state under bf16 I/O, fp32 under fp32 I/O) gives the bits of
    the out-of-place merge."""
    wl = synth.block_workload(T=300, d=4096 if dtype == "bf16" else 256, N=8, S=4, H=2, rep_std_step=0.3,
                              dtype=dtype, seed=9)
    say(f"phase2 in place {dtype} T={wl.T} policy={policy}")
    reps, parts, w, g = _block_on_gpu(wl, dtype, wl.gain)
    sdt = torch.float16 if dtype == "bf16" else torch.float32
    _, o, lse, sc = ar.attnres_block_phase1(reps, w, g, wl.eps, 2, o_dtype=sdt)
    out_of_place = ar.attnres_block_phase2_merge(o[0], lse[1], parts[0], w[1], g[1], wl.eps, 2, o_scale=sc)
    view = o[0].view(TDT[dtype])
    ar.attnres_block_phase2_merge(o[0], lse[1], parts[0], w[1], g[1], wl.eps, 2, h_i=o[0], o_scale=sc)
    assert torch.equal(view, out_of_place)
    ref = orc.block_direct(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, 2)
    check(host(view), ref[1], dtype, "in-place merge")


def test_block_two_phase_config_sampled():
    """Block two-phase bf16 at full size: T=16384, d=4096, N=8, S=4, H=1."""
    wl = synth.config_block_two_phase()
    say(f"block two-phase T={wl.T} d={wl.d} N=8 S=4 (sampled tokens)")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    h = ar.mhar_fwd(reps, parts, w, g, wl.eps, 1)
    h_again = ar.mhar_fwd(reps, parts, w, g, wl.eps, 1)
    assert torch.equal(h, h_again), "not deterministic"
    idx = synth.sample_tokens(wl.T, 384)
    ref = orc.block_direct(synth.take_tokens(wl.reps, idx), synth.take_tokens(wl.partials, idx), wl.w,
                           wl.gain, wl.eps, 1)
    hh = host(h[:, idx])
    for i in range(4):
        err = check(hh[i], ref[i], "bf16", f"h{i + 1}")
        print(f"  h{i + 1}: excess/RMS {err:.2e}, raw max-abs/RMS {max_abs_over_rms(hh[i], ref[i]):.2e}")


def test_mhar_config_sampled():
    """MHAR bf16 at full size: T=32768, d=4096, H=8 heads of 512, N=8, S=4."""
    wl = synth.config_mhar()
    say(f"mhar T={wl.T} d={wl.d} H=8 (sampled tokens)")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    h = ar.mhar_fwd(reps, parts, w, g, wl.eps, 8)
    idx = synth.sample_tokens(wl.T, 384)
    ref = orc.mhar_fwd(synth.take_tokens(wl.reps, idx), synth.take_tokens(wl.partials, idx), wl.w,
                       wl.gain, wl.eps, 8)
    hh = host(h[:, idx])
    for i in range(4):
        check(hh[i], ref[i], "bf16", f"mhar h{i + 1}")


def test_mhar_h1_reduces_to_attnres():
    """H = 1 MHAR equals Block AttnRes (oracle with one head), at the MHAR distributions."""
    wl = synth.config_mhar(T=2048, H=1)
    say(f"mhar H=1 T={wl.T}")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    h = host(ar.mhar_fwd(reps, parts, w, g, wl.eps, 1))
    ref = orc.block_direct(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, 1)
    for i in range(4):
        check(h[i], ref[i], "bf16", f"H=1 h{i + 1}")


def test_single_rep_is_identity_for_first_sublayer(policy):
    """N = 1: the first sublayer reads one source, so alpha = 1 and h_1 = b_0 exactly."""
    wl = synth.block_workload(T=50, d=4096, N=1, S=2, H=1, rep_std_step=0.3, dtype="bf16", seed=4)
    say(f"single rep T={wl.T} policy={policy}")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    h = ar.mhar_fwd(reps, parts, w, g, wl.eps, 1)
    assert torch.equal(h[0], reps[0])


def test_empty_tokens_no_op():
    say("T = 0")
    reps = torch.empty((8, 0, 64), device=DEV, dtype=torch.bfloat16)
    w = torch.zeros((4, 64), device=DEV)
    h = ar.mhar_fwd(reps, torch.empty((3, 0, 64), device=DEV, dtype=torch.bfloat16), w)
    assert h.shape == (4, 0, 64)
    dw = torch.full((4, 64), 7.0, device=DEV)
    ar.attnres_bwd(reps, torch.empty((3, 0, 64), device=DEV, dtype=torch.bfloat16), w,
                   torch.empty((4, 0, 64), device=DEV, dtype=torch.bfloat16), dw=dw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0


# ----------------------------------------------------------------- chunked prefill
@pytest.mark.parametrize("T,d,H,dtype,chunks", [
    (37, 512, 1, "bf16", (1, 5, 36, 37, 100)),
    (300, 4096, 1, "bf16", (64, 128, 299)),
    (200, 4096, 8, "bf16", (3, 77)),
    (20, 96, 3, "f32", (7, 19)),
])
def test_mhar_chunked_matches_whole(T, d, H, dtype, chunks, policy):
    """Chunked prefill: every chunk size gives the bits of the whole-sequence call
    (tokens never interact), from a workspace sized for one chunk."""
    say(f"mhar chunked T={T} d={d} H={H} {dtype} chunks={chunks} policy={policy}")
    wl = synth.block_workload(T=T, d=d, N=8, S=4, H=H, rep_std_step=0.3, dtype=dtype, seed=31)
    reps, parts, w, g = _block_on_gpu(wl, dtype, wl.gain)
    whole = ar.mhar_fwd(reps, parts, w, g, wl.eps, H)
    for c in chunks:
        h = ar.mhar_fwd_chunked(reps, parts, w, c, g, wl.eps, H)
        assert torch.equal(h, whole), f"chunk_T={c} differs from the whole-sequence call"
    ref = orc.block_direct(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, H)
    check(host(whole), ref, dtype, "mhar_fwd")


def test_mhar_chunked_workspace_reuse():
    """One chunk-sized workspace serves several calls and sequence lengths."""
    wl = synth.block_workload(T=513, d=2048, N=8, S=4, H=2, rep_std_step=0.3, dtype="bf16", seed=32)
    say(f"mhar chunked workspace reuse T={wl.T}")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    ws = torch.empty(ar.mhar_fwd_workspace_size(8, 4, 128, 2048, 2), dtype=torch.uint8, device=DEV)
    whole = ar.mhar_fwd(reps, parts, w, g, wl.eps, 2)
    for T in (513, 128, 1, 200):
        h = ar.mhar_fwd_chunked(reps[:, :T].contiguous(), parts[:, :T].contiguous(), w, 128, g, wl.eps, 2, ws=ws)
        assert torch.equal(h, whole[:, :T]), f"T={T}"


# ----------------------------------------------------------------- backward
@pytest.mark.parametrize("T,d,N,S,H,dtype,gain", [
    (4, 16, 8, 4, 1, "f32", "per"),
    (4, 16, 8, 4, 2, "f32", "shared"),
    (3, 16, 8, 4, 1, "f32", "none"),
    (37, 512, 8, 4, 1, "bf16", "per"),
    (21, 4096, 8, 4, 1, "bf16", "per"),
    (21, 4096, 8, 4, 8, "bf16", "shared"),
    # heads of whole waves on the fast kernel: 512 channels per wave
    (33, 4096, 8, 4, 2, "bf16", "per"),
    (37, 2048, 8, 4, 4, "bf16", "per"),
    (19, 1024, 8, 4, 2, "bf16", "none"),
    (10, 96, 3, 2, 3, "bf16", "per"),
    (6, 64, 5, 1, 1, "f32", "per"),
])
def test_bwd_shapes(T, d, N, S, H, dtype, gain, policy):
    say(f"bwd T={T} d={d} N={N} S={S} H={H} {dtype} gain={gain} policy={policy}")
    wl = synth.block_workload(T=T, d=d, N=N, S=S, H=H, rep_std_step=0.3, dtype=dtype, seed=7, with_dh=True)
    g = _gain_arg(wl.gain, gain, S, d, np.random.default_rng(3))
    ref = orc.block_bwd(wl.reps, wl.partials, wl.w, g, wl.eps, H, wl.dh)
    reps, parts, w, gg = _block_on_gpu(wl, dtype, g)
    got = ar.attnres_bwd(reps, parts, w, dev(wl.dh, dtype), gg, wl.eps, H)
    check(host(got[0]), ref[0], dtype, "d_reps")
    if S > 1:
        check(host(got[1]), ref[1], dtype, "d_partials")
    pdt = "f32" if dtype == "f32" else "f32_from_bf16"
    check(host(got[2]), ref[2], pdt, "dw")
    if g is not None:
        check(host(got[3]), ref[3], pdt, "dgain")


def test_bwd_accumulate(policy):
    wl = synth.block_workload(T=33, d=512, N=8, S=4, H=1, rep_std_step=0.3, dtype="f32", seed=8, with_dh=True)
    say(f"bwd accumulate policy={policy}")
    reps, parts, w, g = _block_on_gpu(wl, "f32", wl.gain)
    dh = dev(wl.dh)
    base = [torch.randn_like(x) for x in (reps, parts, w, g)]
    outs = [b.clone() for b in base]
    ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, 1, d_reps=outs[0], d_partials=outs[1], dw=outs[2],
                   dgain=outs[3], accumulate=True)
    fresh = ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, 1)
    for b, o, f in zip(base, outs, fresh):
        np.testing.assert_allclose(host(o), host(b) + host(f), rtol=1e-6, atol=1e-6)


def test_bwd_full_d_against_oracle():
    """Block backward at the full width (d=4096, N=8, S=4) over every token of a
    T=512 batch, so dw and dgain (sums over tokens) are compared exactly."""
    wl = synth.config_block_fwd_bwd(T=512)
    say(f"bwd full-d T={wl.T}")
    ref = orc.block_bwd(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, 1, wl.dh)
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    got = ar.attnres_bwd(reps, parts, w, dev(wl.dh, "bf16"), g, wl.eps, 1)
    for name, y, r, kind in zip(("d_reps", "d_partials", "dw", "dgain"), got, ref,
                                ("bf16", "bf16", "f32_from_bf16", "f32_from_bf16")):
        err = check(host(y), r, kind, name)
        print(f"  {name}: {err:.2e}")


def _param_grad_golden(H):
    """The oracle's dw and dgain summed over every token of the full-size
    backward workload (written by tests/golden/make_bwd_param_grads.py)."""
    import os
    z = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bwd_param_grads.npz"))
    return z[f"dw_H{H}"], z[f"dgain_H{H}"]


def test_bwd_config_sampled():
    """Block fwd+bwd bf16 at full size: T=8192, d=4096, N=8, S=4.

    Per-token gradients on sampled tokens against the oracle; dw/dgain through
    properties: dw_j * w_j == dg_j * g_j, and additivity over two token halves."""
    wl = synth.config_block_fwd_bwd()
    say(f"bwd config T={wl.T} (sampled tokens + properties)")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    dh = dev(wl.dh, "bf16")
    h = ar.mhar_fwd(reps, parts, w, g, wl.eps, 1)
    d_reps, d_parts, dw, dg = ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, 1)
    idx = synth.sample_tokens(wl.T, 48)
    ref = orc.block_bwd(synth.take_tokens(wl.reps, idx), synth.take_tokens(wl.partials, idx), wl.w,
                        wl.gain, wl.eps, 1, synth.take_tokens(wl.dh, idx))
    check(host(d_reps[:, idx]), ref[0], "bf16", "d_reps (sampled)")
    check(host(d_parts[:, idx]), ref[1], "bf16", "d_partials (sampled)")
    href = orc.block_direct(synth.take_tokens(wl.reps, idx), synth.take_tokens(wl.partials, idx), wl.w,
                            wl.gain, wl.eps, 1)
    check(host(h[:, idx]), href, "bf16", "forward h (sampled)")
    # closed form: dw * w == dgain * g (both equal w * g * Z)
    lhs, rhs = host(dw) * wl.w, host(dg) * wl.gain
    assert max_abs_over_rms(lhs, rhs) < 1e-5
    # additivity over tokens
    half = wl.T // 2
    a = ar.attnres_bwd(reps[:, :half].contiguous(), parts[:, :half].contiguous(), w,
                       dh[:, :half].contiguous(), g, wl.eps, 1)
    b = ar.attnres_bwd(reps[:, half:].contiguous(), parts[:, half:].contiguous(), w,
                       dh[:, half:].contiguous(), g, wl.eps, 1)
    assert max_abs_over_rms(host(a[2]) + host(b[2]), host(dw)) < 1e-4
    assert max_abs_over_rms(host(a[3]) + host(b[3]), host(dg)) < 1e-4
    # determinism
    again = ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, 1)
    assert all(torch.equal(x, y) for x, y in zip(again, (d_reps, d_parts, dw, dg)))
    # dw and dgain over all 8192 tokens against the oracle's token sums
    gold = _param_grad_golden(1)
    print(f"  dw {check(host(dw), gold[0], 'f32_from_bf16', 'dw (all tokens)'):.2e}, "
          f"dgain {check(host(dg), gold[1], 'f32_from_bf16', 'dgain (all tokens)'):.2e}")


def test_mhar_bwd_config_sampled():
    """MHAR Block backward bf16 at full size: T=8192, d=4096, H=8 heads of 512,
    N=8, S=4.  Sampled tokens against the oracle; dw and dgain through the
    closed form dw * w == dg * g and against the general kernel's sums."""
    wl = synth.config_mhar_fwd_bwd()
    say(f"mhar bwd config T={wl.T} H=8 (sampled tokens + properties)")
    reps, parts, w, g = _block_on_gpu(wl, "bf16", wl.gain)
    dh = dev(wl.dh, "bf16")
    d_reps, d_parts, dw, dg = ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, 8)
    idx = synth.sample_tokens(wl.T, 48)
    ref = orc.block_bwd(synth.take_tokens(wl.reps, idx), synth.take_tokens(wl.partials, idx), wl.w,
                        wl.gain, wl.eps, 8, synth.take_tokens(wl.dh, idx))
    check(host(d_reps[:, idx]), ref[0], "bf16", "d_reps (sampled)")
    check(host(d_parts[:, idx]), ref[1], "bf16", "d_partials (sampled)")
    lhs, rhs = host(dw) * wl.w, host(dg) * wl.gain
    assert max_abs_over_rms(lhs, rhs) < 1e-5
    again = ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, 8)
    assert all(torch.equal(x, y) for x, y in zip(again, (d_reps, d_parts, dw, dg)))
    prev = ar.attnres_set_kernel_policy(1)
    try:
        gen = ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, 8)
    finally:
        ar.attnres_set_kernel_policy(prev)
    for name, x, y in (("dw", dw, gen[2]), ("dgain", dg, gen[3])):   # sums over all 8192 tokens
        err = max_abs_over_rms(host(x), host(y))
        print(f"  fast vs general {name}: {err:.2e}")
        assert err < 1e-4, name
    gold = _param_grad_golden(8)
    check(host(dw), gold[0], "f32_from_bf16", "dw (all tokens)")
    check(host(dg), gold[1], "f32_from_bf16", "dgain (all tokens)")


# ----------------------------------------------------------------- Full backward
@pytest.mark.parametrize("T,d,L,n_dst,H,dtype,gain", [
    (5, 16, 4, 4, 1, "f32", "per"),
    (9, 64, 6, 3, 2, "bf16", "shared"),
    (3, 24, 3, 1, 3, "f32", "none"),
    (41, 256, 8, 8, 1, "bf16", "per"),
    (6, 2048, 32, 32, 1, "bf16", "per"),
    (2, 8, 64, 16, 1, "f32", "none"),      # 16 x 64 = 1024 table entries, the limit
    # bf16, one head, n_src <= 32, d % 512 == 0: the matrix-core kernels under "auto"
    (37, 512, 32, 32, 1, "bf16", "per"),
    (19, 1024, 7, 3, 1, "bf16", "shared"),
    (70, 1536, 32, 1, 1, "bf16", "none"),
    (3, 4096, 17, 17, 1, "bf16", "per"),
])
def test_full_bwd_shapes(T, d, L, n_dst, H, dtype, gain, policy):
    say(f"full bwd T={T} d={d} L={L} n_dst={n_dst} H={H} {dtype} gain={gain} policy={policy}")
    wl = synth.full_workload(T=T, d=d, L=L, std_step=0.2, dtype=dtype, seed=9, gain_variance=0.02,
                             n_dst=n_dst, with_dout=True)
    g = _gain_arg(wl.gain, gain, n_dst, d, np.random.default_rng(4))
    ref = orc.full_bwd(wl.src, wl.w, g, wl.eps, H, wl.dh)
    got = ar.attnres_full_bwd(dev(wl.src, dtype), dev(wl.w), dev(wl.dh, dtype), dev(g), wl.eps, H)
    check(host(got[0]), ref[0], dtype, "d_src")
    pdt = "f32" if dtype == "f32" else "f32_from_bf16"
    check(host(got[1]), ref[1], pdt, "dw")
    if g is not None:
        check(host(got[2]), ref[2], pdt, "dgain")


def test_full_bwd_accumulate():
    wl = synth.full_workload(T=21, d=128, L=6, std_step=0.2, dtype="f32", seed=10, gain_variance=0.02,
                             with_dout=True)
    say("full bwd accumulate")
    src, w, g, dout = dev(wl.src), dev(wl.w), dev(wl.gain), dev(wl.dh)
    base = [torch.randn_like(x) for x in (src, w, g)]
    outs = [b.clone() for b in base]
    ar.attnres_full_bwd(src, w, dout, g, wl.eps, 1, d_src=outs[0], dw=outs[1], dgain=outs[2], accumulate=True)
    fresh = ar.attnres_full_bwd(src, w, dout, g, wl.eps, 1)
    for b, o, f in zip(base, outs, fresh):
        np.testing.assert_allclose(host(o), host(b) + host(f), rtol=1e-6, atol=1e-6)


def test_full_bwd_accumulate_bf16(policy):
    """accumulate = 1 adds the gradient in fp32 to the bf16 d_src before one rounding."""
    wl = synth.full_workload(T=45, d=512, L=12, std_step=0.2, dtype="bf16", seed=11, gain_variance=0.02,
                             with_dout=True)
    say(f"full bwd accumulate bf16 policy={policy}")
    ref = orc.full_bwd(wl.src, wl.w, wl.gain, wl.eps, 1, wl.dh)
    src, w, g, dout = dev(wl.src, "bf16"), dev(wl.w), dev(wl.gain), dev(wl.dh, "bf16")
    rng = np.random.default_rng(12)
    base = [rng.standard_normal(x.shape).astype(np.float32) for x in (wl.src, wl.w, wl.gain)]
    base[0] = synth.bf16_round(base[0])
    outs = [dev(base[0], "bf16"), dev(base[1]), dev(base[2])]
    ar.attnres_full_bwd(src, w, dout, g, wl.eps, 1, d_src=outs[0], dw=outs[1], dgain=outs[2], accumulate=True)
    check(host(outs[0]), base[0] + ref[0], "bf16", "d_src accumulated")
    check(host(outs[1]), base[1] + ref[1], "f32_from_bf16", "dw accumulated")
    check(host(outs[2]), base[2] + ref[2], "f32_from_bf16", "dgain accumulated")


def test_full_bwd_no_tokens_zeroes_parameter_grads():
    say("full bwd T=0")
    w = dev(np.ones((3, 64), np.float32))
    g = dev(np.ones(64, np.float32))
    src = torch.empty((4, 0, 64), dtype=torch.bfloat16, device=DEV)
    dout = torch.empty((3, 0, 64), dtype=torch.bfloat16, device=DEV)
    dw = torch.full((3, 64), 7.0, device=DEV)
    dg = torch.full((64,), 7.0, device=DEV)
    ar.attnres_full_bwd(src, w, dout, g, 1e-6, 1, dw=dw, dgain=dg)
    assert torch.count_nonzero(dw).item() == 0 and torch.count_nonzero(dg).item() == 0


def test_full_bwd_full_width_against_oracle():
    """Full backward at the full width (d=2048, L=32) over every token of a
    T=128 batch, so dw and dgain (sums over tokens) are compared exactly."""
    wl = synth.config_full_fwd_bwd(T=128)
    say(f"full bwd full-width T={wl.T}")
    ref = orc.full_bwd(wl.src, wl.w, wl.gain, wl.eps, 1, wl.dh)
    got = ar.attnres_full_bwd(dev(wl.src, "bf16"), dev(wl.w), dev(wl.dh, "bf16"), dev(wl.gain), wl.eps, 1)
    for name, y, r, kind in zip(("d_src", "dw", "dgain"), got, ref, ("bf16", "f32_from_bf16", "f32_from_bf16")):
        err = check(host(y), r, kind, name)
        print(f"  {name}: {err:.2e}")


def test_full_bwd_config_sampled():
    """Full fwd+bwd bf16 at full size: T=4096, d=2048, L=32.

    Per-token gradients on sampled tokens against the oracle; dw/dgain through
    properties: dw_j * w_j == dg_j * g_j, additivity over two token halves,
    and bit-identical repeats."""
    wl = synth.config_full_fwd_bwd()
    say(f"full bwd config T={wl.T} (sampled tokens + properties)")
    src, w, g, dout = dev(wl.src, "bf16"), dev(wl.w), dev(wl.gain), dev(wl.dh, "bf16")
    d_src, dw, dg = ar.attnres_full_bwd(src, w, dout, g, wl.eps, 1)
    idx = synth.sample_tokens(wl.T, 24)
    ref = orc.full_bwd(synth.take_tokens(wl.src, idx), wl.w, wl.gain, wl.eps, 1, synth.take_tokens(wl.dh, idx))
    check(host(d_src[:, idx]), ref[0], "bf16", "d_src (sampled)")
    lhs, rhs = host(dw) * wl.w, host(dg) * wl.gain
    assert max_abs_over_rms(lhs, rhs) < 1e-5
    half = wl.T // 2
    a = ar.attnres_full_bwd(src[:, :half].contiguous(), w, dout[:, :half].contiguous(), g, wl.eps, 1)
    b = ar.attnres_full_bwd(src[:, half:].contiguous(), w, dout[:, half:].contiguous(), g, wl.eps, 1)
    assert max_abs_over_rms(host(a[1]) + host(b[1]), host(dw)) < 1e-4
    assert max_abs_over_rms(host(a[2]) + host(b[2]), host(dg)) < 1e-4
    again = ar.attnres_full_bwd(src, w, dout, g, wl.eps, 1)
    for x, y in zip((d_src, dw, dg), again):
        assert torch.equal(x, y)
