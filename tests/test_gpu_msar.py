"""Parity of the MSAR forward (attnres_msar_fwd) with the MSAR oracle on MI355X,
through both the specialised and the general kernels (the policy fixture).

Element by element over every output at small sizes (ragged d, sequences
shorter than the longest kernel, Full-style prefix sets and Block-style single
destinations); at the Block MSAR sublayer size (T=16384, d=4096, 8 reps and
the partial) on sampled tokens, each with the 11 tokens before it that its
streams read.  Bars: bf16 I/O, excess over half an ulp <= 2e-2 of the RMS;
fp32 I/O, max-abs <= 1e-5 of the RMS.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import depth_wise_attention_amd as ar  # noqa: E402
from metrics import check  # noqa: E402
from oracle import msar_oracle as mso  # noqa: E402
from workloads import synth  # noqa: E402

DEV = "cuda"


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@pytest.fixture(params=[0, 1], ids=["auto", "general"])
def policy(request):
    prev = ar.attnres_set_kernel_policy(request.param)
    yield request.param
    ar.attnres_set_kernel_policy(prev)


def _run(wl):
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    return ar.attnres_msar_fwd(dev(wl.src, tdt), dev(wl.w), dev(wl.meta["conv"]), dev(wl.meta["mix"]), wl.eps)


@pytest.mark.parametrize("T,d,n_src,n_dst,dtype", [
    (1, 64, 1, 1, "f32"),
    (5, 64, 3, 2, "f32"),       # shorter than the 12-tap stream
    (17, 96, 5, 3, "f32"),
    (30, 130, 4, 2, "f32"),     # ragged channel count
    (40, 512, 9, 1, "bf16"),    # a Block MSAR sublayer: 8 reps + the partial
    (13, 256, 32, 32, "bf16"),  # Full-style prefix sets
    (64, 2048, 9, 1, "bf16"),
    (24, 4096, 9, 1, "bf16"),
    (9, 1024, 64, 4, "bf16"),   # the most sources
    # the specialised path (bf16, one destination, <= 12 sources, d % 512 == 0):
    (5, 512, 3, 1, "bf16"),     # shorter than the history
    (300, 1024, 12, 1, "bf16"), # several token ranges and a ragged last one
    (257, 512, 1, 1, "bf16"),
    (130, 1536, 6, 1, "bf16"),
])
def test_msar_shapes(T, d, n_src, n_dst, dtype, policy):
    say(f"msar T={T} d={d} n_src={n_src} n_dst={n_dst} {dtype} policy={policy}")
    wl = synth.msar_workload(T=T, d=d, n_src=n_src, n_dst=n_dst, dtype=dtype, seed=60)
    ref = mso.msar_fwd(wl.src, wl.w, wl.meta["conv"], wl.meta["mix"], wl.eps)
    out = _run(wl)
    check(host(out), ref, dtype, "msar out")
    again = _run(wl)
    assert torch.equal(out, again), "not deterministic"


def test_msar_empty():
    say("msar T=0")
    src = torch.empty((3, 0, 64), dtype=torch.bfloat16, device=DEV)
    out = ar.attnres_msar_fwd(src, torch.zeros((2, 4, 64), device=DEV), torch.zeros((24, 64), device=DEV),
                              torch.zeros((2, 256, 4), device=DEV))
    assert out.shape == (2, 0, 64)


def test_msar_block_sublayer_sampled():
    """Block MSAR sublayer at full size: T=16384, d=4096, 8 reps + the partial."""
    wl = synth.msar_workload(T=16384, d=4096, n_src=9, n_dst=1, dtype="bf16", seed=0)
    say(f"msar block sublayer T={wl.T} d={wl.d} n_src=9 (sampled tokens)")
    out = _run(wl)
    idx = np.concatenate([[0, 1, 11, 12], synth.sample_tokens(wl.T, 60)])
    for t in idx:
        lo = max(0, int(t) - 11)      # the window its streams read
        ref = mso.msar_fwd(wl.src[:, lo:t + 1], wl.w, wl.meta["conv"], wl.meta["mix"], wl.eps)[:, -1]
        check(host(out[:, t]), ref, "bf16", f"msar token {t}")


# ----------------------------------------------------------------- Block MSAR, two-phase
def _bm_run(wl, N, S):
    reps = dev(wl.reps, torch.bfloat16)
    parts = dev(wl.partials, torch.bfloat16) if S > 1 else None
    w, conv, mix = dev(wl.w), dev(wl.meta["conv"]), dev(wl.meta["mix"])
    h1, o, sc, lse = ar.attnres_block_msar_phase1(reps, w, conv, mix[0], wl.eps)
    hs = [h1]
    for i in range(2, S + 1):
        hs.append(ar.attnres_block_msar_phase2(o[i - 2], sc, lse[i - 2], parts[i - 2], w[i - 1], conv, mix[i - 1],
                                               wl.eps))
    return torch.stack(hs), o, sc, lse


@pytest.mark.parametrize("T,d,N,S", [
    (5, 512, 1, 1),
    (20, 512, 3, 4),
    (130, 1024, 8, 4),
    (257, 512, 12, 2),
    (300, 1536, 5, 3),
    (64, 4096, 8, 4),
])
def test_block_msar_two_phase(T, d, N, S):
    say(f"block msar two-phase T={T} d={d} N={N} S={S}")
    wl = synth.block_msar_workload(T=T, d=d, N=N, S=S, seed=70)
    ref = mso.block_msar_direct(wl.reps, wl.partials, wl.w, wl.meta["conv"], wl.meta["mix"], wl.eps)
    h, o, sc, lse = _bm_run(wl, N, S)
    for i in range(S):
        check(host(h[i]), ref[i], "bf16", f"h_{i + 1}")
    if S > 1:
        _, o_ref, lse_ref = mso.block_msar_phase1(wl.reps, wl.w, wl.meta["conv"], wl.meta["mix"][0], wl.eps)
        back = host(o) * host(sc)[None, None, :, None]
        # the fp16 state: within half an fp16 ulp of the value (2^-11 relative)
        # plus the fp32 arithmetic's slack; the scale bounds every value
        bound = 2.0 ** -11 * np.abs(o_ref) * (1 + 1e-3) + 1e-4 * np.sqrt(np.mean(o_ref ** 2))
        assert np.all(np.abs(back - o_ref) <= bound), float(np.max(np.abs(back - o_ref) - bound))
        assert np.all(np.isfinite(host(o)))
        np.testing.assert_allclose(host(lse), lse_ref, rtol=0, atol=1e-4)
    h2, _, _, _ = _bm_run(wl, N, S)
    assert torch.equal(h, h2), "not deterministic"


def test_block_msar_sampled():
    """Block MSAR at the Block size: T=16384, d=4096, N=8 reps, S=4, on sampled
    tokens (each with the 11 tokens its streams read)."""
    wl = synth.block_msar_workload(T=16384, d=4096, N=8, S=4, seed=0)
    say(f"block msar two-phase T={wl.T} d={wl.d} N=8 S=4 (sampled tokens)")
    h, _, _, _ = _bm_run(wl, 8, 4)
    for t in np.concatenate([[0, 11, 12], synth.sample_tokens(wl.T, 40)]):
        lo = max(0, int(t) - 11)
        ref = mso.block_msar_direct(wl.reps[:, lo:t + 1], wl.partials[:, lo:t + 1], wl.w, wl.meta["conv"],
                                    wl.meta["mix"], wl.eps)[:, -1]
        check(host(h[:, t]), ref, "bf16", f"block msar token {t}")
