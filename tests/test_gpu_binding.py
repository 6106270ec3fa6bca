"""The binding's checks that need GPU tensors, and its use of the caller's stream.

Shapes, parameter dtypes and state formats are refused with ValueError or
TypeError before any call into the library.  A call on a side stream
allocates its outputs and workspace on that stream: while it still runs, the
caching allocator cannot hand that memory to work on the current stream, so
the result equals a current-stream run bit for bit even with such work
racing it.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import depth_wise_attention_amd as ar  # noqa: E402
from workloads import synth  # noqa: E402

DEV = "cuda"


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def _block(T=64, d=512, N=8, S=4, H=1, with_dh=False):
    wl = synth.block_workload(T=T, d=d, N=N, S=S, H=H, rep_std_step=0.3, dtype="bf16", seed=3, with_dh=with_dh)
    out = [dev(wl.reps, True), dev(wl.partials, True), dev(wl.w), dev(wl.gain)]
    if with_dh:
        out.append(dev(wl.dh, True))
    return out


def test_shapes_and_parameter_dtypes_are_checked():
    say("binding shape and dtype checks")
    reps, parts, w, g, dh = _block(with_dh=True)
    with pytest.raises(ValueError, match="partials"):
        ar.mhar_fwd(reps, parts[:2], w, g)
    with pytest.raises(ValueError, match="w must have shape"):
        ar.mhar_fwd(reps, parts, w[:, :256].contiguous(), g)
    with pytest.raises(TypeError, match="w must be"):
        ar.mhar_fwd(reps, parts, w.to(torch.bfloat16), g)
    with pytest.raises(ValueError, match="gain"):
        ar.mhar_fwd(reps, parts, w, g[:3].contiguous())
    with pytest.raises(TypeError, match="gain"):
        ar.mhar_fwd(reps, parts, w, g.to(torch.bfloat16))
    with pytest.raises(ValueError, match="h must have shape"):
        ar.mhar_fwd(reps, parts, w, g, h=torch.empty((3, 64, 512), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(TypeError, match="partials"):
        ar.mhar_fwd(reps, parts.float(), w, g)
    with pytest.raises(ValueError, match="lse"):
        ar.attnres_block_phase1(reps, w, g, lse=torch.empty((4, 2, 64), device=DEV))
    with pytest.raises(ValueError, match="o_state"):
        ar.attnres_block_phase1(reps, w, g, o_state=torch.empty((4, 64, 512), device=DEV))
    with pytest.raises(ValueError, match="dh"):
        ar.attnres_bwd(reps, parts, w, dh[:, :32].contiguous(), g)
    with pytest.raises(TypeError, match="dw"):
        ar.attnres_bwd(reps, parts, w, dh, g, dw=torch.empty((4, 512), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="contiguous"):
        ar.attnres_full_fwd(reps.transpose(1, 2), w)
    with pytest.raises(ValueError, match="o_scale"):
        ar.attnres_block_phase2_merge(torch.zeros((64, 512), dtype=torch.float16, device=DEV),
                                      torch.zeros((1, 64), device=DEV), parts[0], w[1], g[1])
    torch.cuda.synchronize()


@pytest.mark.parametrize("op", ["mhar_fwd", "attnres_bwd", "attnres_full_fwd"])
def test_side_stream_allocations(op):
    """Outputs and workspace allocated by the binding belong to the call's stream."""
    say(f"side stream {op}")
    reps, parts, w, g, dh = _block(T=2048, d=4096, with_dh=True)
    call = {
        "mhar_fwd": lambda st: (ar.mhar_fwd(reps, parts, w, g, stream=st),),
        "attnres_bwd": lambda st: ar.attnres_bwd(reps, parts, w, dh, g, stream=st)[:3],
        "attnres_full_fwd": lambda st: (ar.attnres_full_fwd(reps, w, stream=st),),
    }[op]
    want = [t.clone() for t in call(None)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        got = call(side)
        # Work on the current stream while the side stream may still run: with
        # the binding's buffers owned by the current stream, these writes could
        # land in the call's workspace.
        junk = [torch.full((1 << 22,), float(k), device=DEV) for k in range(8)]
        del junk
        torch.cuda.current_stream().wait_stream(side)
        for a, b in zip(got, want):
            assert torch.equal(a, b)
        del got
    torch.cuda.synchronize()
