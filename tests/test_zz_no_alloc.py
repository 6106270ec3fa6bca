"""mhar_fwd_noalloc: mhar_fwd with its workspace in the library's static
per-device scratch, for callers that cannot allocate.  Through the C ABI it
must give the bits of mhar_fwd (the same kernels), and the oracle's result
within the bf16 bar, on consecutive calls that reuse the scratch -- the second
with a smaller input -- and refuse a request beyond the scratch."""

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


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


@pytest.mark.parametrize("H", [1, 8])
def test_noalloc_matches_mhar_fwd_on_consecutive_calls(H):
    for T, seed in ((3000, 5), (517, 6)):   # the second call is smaller and reuses the scratch
        say(f"mhar_fwd_noalloc T={T} H={H}")
        wl = synth.block_workload(T=T, d=4096, N=8, S=4, H=H, rep_std_step=0.3, dtype="bf16", seed=seed)
        reps, parts, w, g = dev(wl.reps, True), dev(wl.partials, True), dev(wl.w), dev(wl.gain)
        h = torch.empty((4, T, 4096), dtype=torch.bfloat16, device=DEV)
        ar.mhar_fwd_noalloc(reps, parts, w, h, g, wl.eps, H)
        want = ar.mhar_fwd(reps, parts, w, g, wl.eps, H)
        torch.cuda.synchronize()
        assert torch.equal(h, want), "mhar_fwd_noalloc differs from mhar_fwd"
        ref = orc.block_direct(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, H)
        check(h.float().cpu().numpy().astype(np.float64), ref, "bf16", "mhar_fwd_noalloc")


def test_noalloc_general_kernels_and_fp32():
    """fp32 I/O (general kernels, fp32 state) through the same scratch."""
    say("mhar_fwd_noalloc fp32")
    wl = synth.block_workload(T=40, d=96, N=5, S=3, H=3, rep_std_step=0.3, dtype="f32", seed=7)
    reps, parts, w, g = dev(wl.reps), dev(wl.partials), dev(wl.w), dev(wl.gain)
    h = torch.empty((3, 40, 96), device=DEV)
    ar.mhar_fwd_noalloc(reps, parts, w, h, g, wl.eps, 3)
    assert torch.equal(h, ar.mhar_fwd(reps, parts, w, g, wl.eps, 3))
    ref = orc.block_direct(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, 3)
    check(h.cpu().numpy().astype(np.float64), ref, "f32", "mhar_fwd_noalloc fp32")


def test_noalloc_refuses_requests_beyond_the_scratch():
    """S = 4, H = 8 needs 132 bytes of scratch per token: 70000 tokens exceed 8 MiB."""
    T, d = 70000, 512
    say(f"mhar_fwd_noalloc oversize T={T}")
    reps = torch.zeros((1, T, d), dtype=torch.bfloat16, device=DEV)
    parts = torch.zeros((3, T, d), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((4, d), device=DEV)
    h = torch.empty((4, T, d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ar.AttnResError) as e:
        ar.mhar_fwd_noalloc(reps, parts, w, h, None, 1e-6, 8)
    assert e.value.code == -2 and "scratch" in e.value.message
    torch.cuda.synchronize()
