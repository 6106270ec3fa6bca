"""Decode-size calls on MI355X: a few tokens per call, launched eagerly and from
a captured HIP graph.

A decode step of one Block AttnRes block is Phase 1 (once per block) and, per
sublayer i >= 2, the fused update of the running partial with the previous
sublayer's output.  The step is captured once and replayed with new inputs
copied into the captured buffers between replays; every replay must give the
bits of the same calls made eagerly, and the eager calls match the oracle.
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


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class BlockStep:
    """Buffers and calls of one block's decode step (bf16 I/O, scaled fp16 state)."""

    def __init__(self, T, d, N, S, H):
        self.S, self.H = S, H
        z = dict(device=DEV)
        self.reps = torch.empty((N, T, d), dtype=torch.bfloat16, **z)
        self.f = torch.empty((S - 1, T, d), dtype=torch.bfloat16, **z)
        self.w = torch.empty((S, d), **z)
        self.g = torch.empty((S, d), **z)
        self.h = torch.empty((S, T, d), dtype=torch.bfloat16, **z)
        self.state = torch.empty((S - 1, T, d), dtype=torch.float16, **z)
        self.lse = torch.empty((S, H, T), **z)
        self.scale = torch.empty((T,), **z)
        self.part = torch.empty((T, d), dtype=torch.bfloat16, **z)
        self.rms = torch.empty((S - 1, T), **z)

    def load(self, wl):
        self.reps.copy_(dev(wl.reps, torch.bfloat16))
        self.f.copy_(dev(wl.f, torch.bfloat16))
        self.w.copy_(dev(wl.w))
        self.g.copy_(dev(wl.gain))

    def run(self):
        ar.attnres_block_phase1(self.reps, self.w, self.g, 1e-6, self.H, h_first=self.h[0], o_state=self.state,
                                lse=self.lse, o_scale=self.scale)
        for i in range(2, self.S + 1):
            ar.attnres_block_phase2_merge_update(
                self.state[i - 2], self.lse[i - 1], None if i == 2 else self.part, self.f[i - 2], self.w[i - 1],
                self.g[i - 1], 1e-6, self.H, partial_out=self.part, h_i=self.h[i - 1], norm_eps=1e-6,
                h_inv_rms=self.rms[i - 2], o_scale=self.scale)

    def outputs(self):
        return [self.h.clone(), self.part.clone(), self.rms.clone()]


@pytest.mark.parametrize("T,H", [(1, 1), (3, 1), (64, 8), (5, 4)])
def test_block_decode_graph_replays(T, H):
    d, N, S = 4096, 8, 4
    say(f"block decode graph T={T} H={H}")
    step = BlockStep(T, d, N, S, H)
    wls = [synth.block_workload(T=T, d=d, N=N, S=S, H=H, rep_std_step=0.3, dtype="bf16", seed=40 + k,
                                with_f=True) for k in range(3)]
    # eager results per input set
    eager = []
    for wl in wls:
        step.load(wl)
        step.run()
        eager.append(step.outputs())
    # the oracle on the first input set: h, the final partial and every statistic
    wl = wls[0]
    o_ref, lse_ref = orc.block_phase1(wl.reps, wl.w, wl.gain, wl.eps, H)
    check(host(eager[0][0][0]), o_ref[0], "bf16", "h_1")
    p_ref = None
    for i in range(2, S + 1):
        p_ref, h_ref, r_ref = orc.block_phase2_merge_update(o_ref[i - 1], lse_ref[i - 1], p_ref, wl.f[i - 2],
                                                            wl.w[i - 1], wl.gain[i - 1], wl.eps, H, 1e-6)
        check(host(eager[0][0][i - 1]), h_ref, "bf16", f"h_{i}")
        np.testing.assert_allclose(host(eager[0][2][i - 2]), r_ref, rtol=4e-3)
        p_ref = synth.bf16_round(p_ref.astype(np.float32))   # the partial is stored in bf16
    np.testing.assert_array_equal(host(eager[0][1]), p_ref)

    # capture one step on a side stream, then replay with each input set
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    for rnd in range(2):
        for k, wl in enumerate(wls):
            step.load(wl)          # eager copies between replays
            graph.replay()
            got = step.outputs()
            torch.cuda.synchronize()
            for name, a, b in zip(("h", "partial", "inv_rms"), got, eager[k]):
                assert torch.equal(a, b), f"replay {rnd}/{k}: {name} differs from the eager step"


@pytest.mark.parametrize("T,n_src", [(1, 32), (4, 7), (2, 1)])
def test_full_decode_graph_replays(T, n_src):
    """One Full AttnRes sublayer at decode: a single destination over its n_src sources."""
    d = 2048
    say(f"full decode graph T={T} n_src={n_src}")
    wls = [synth.full_workload(T=T, d=d, L=n_src, std_step=0.1, dtype="bf16", seed=50 + k, n_dst=1,
                               gain_variance=0.02) for k in range(2)]
    src = torch.empty((n_src, T, d), dtype=torch.bfloat16, device=DEV)
    w = torch.empty((1, d), device=DEV)
    g = torch.empty((1, d), device=DEV)
    out = torch.empty((1, T, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(1, ar.attnres_full_fwd_workspace_size(n_src, 1, d, 1, ar.BF16)), dtype=torch.uint8,
                     device=DEV)

    def load(wl):
        src.copy_(dev(wl.src, torch.bfloat16))
        w.copy_(dev(wl.w))
        g.copy_(dev(wl.gain))

    def run():
        ar.attnres_full_fwd(src, w, g, 1e-6, 1, out=out, ws=ws)

    eager = []
    for wl in wls:
        load(wl)
        run()
        eager.append(out.clone())
        ref = orc.full_fwd(wl.src, wl.w, wl.gain, wl.eps, 1)
        check(host(eager[-1]), ref, "bf16", "full decode")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rnd in range(2):
        for k, wl in enumerate(wls):
            load(wl)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager[k]), f"replay {rnd}/{k} differs from the eager call"
