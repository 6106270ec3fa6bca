"""Benchmark of the AttnRes Block two-phase routing on one MI355X.

One step = one pass of the Block hot path over a batch of T tokens: Phase 1
(all S pseudo-queries against the N cached reps, one launch) followed by the
S-1 Phase-2 online-softmax merges (one launch each) -- exactly the launches of
mhar_fwd, issued through the public C-ABI calls so HIP events can bracket each
kernel inside the timed region.  Inputs are seeded synthetic tensors, resident
in HBM before timing starts.

Prints ONE JSON line on stdout.  Everything else goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--no-extra] [--workload block|mhar|full|full_h8|full_wide|full_one|f32|bwd|full_bwd|full_bwd_h8|block_update|decode|msar|block_msar]
                  [--copy-calibration]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD's published peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # 50 untimed steps (about 27 ms of the headline step): the device takes
    # some 25 ms of sustained streaming to settle its clocks; timed from 5
    # warm-up steps, Phase 1 measured 314-323 us, from 50 or 200, 298-300 us.
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="block", choices=["block", "mhar", "full", "full_h8", "full_wide", "bwd", "mhar_bwd", "full_bwd", "full_bwd_h8", "block_update",
                                                                "decode", "msar", "block_msar", "depth_sweep", "full_one", "f32"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    p.add_argument("--ceilings", action="store_true",
                   help="measure the streaming ceilings of the kernels' read/write patterns and exit")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


# ------------------------------------------------------------------ byte accounting
def block_bytes(T, d, N, S, H, es=2, state_es=2):
    """Algorithmic bytes of one Phase-1 launch, one Phase-2 launch, and one step.

    Phase 1 reads N reps, writes h_first, the S-1 state rows (scaled fp16: 2 B per
    value), S*H lse values and one fp32 scale per token.  Phase 2 reads a state
    row, H lse values, the scale and the partial, and writes h_i."""
    p1 = T * (N * d * es + d * es + (S - 1) * d * state_es + S * H * 4 + 4)
    p2 = T * (d * state_es + H * 4 + 4 + d * es + d * es)
    return p1, p2, p1 + (S - 1) * p2


def full_bytes(T, d, L, es=2):
    return T * (L * d * es + L * d * es)


def bwd_bytes(T, d, N, S, es=2):
    # read reps, partials, dh; write d_reps, d_partials (the dw/dgain slabs are small)
    return T * d * es * ((N + (S - 1) + S) + (N + (S - 1)))


# ------------------------------------------------------------------ helpers
def to_dev(x, dtype):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return t.to(dtype)


def time_loop(fn, steps, warmup):
    """Run fn() warmup times, then time `steps` calls bracketed by synchronisation."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3, wall


def kernel_source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "depth_wise_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_for(kernel_key, src_hash):
    """Per-launch HBM bytes measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE, scaled
    by the copy-kernel factor), if recorded for this exact kernel source."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------ workloads
def bench_block(args, H=1, T=16384, name=None, with_events=True, cold_steps=0):
    import torch
    import depth_wise_attention_amd as ar
    from workloads import synth

    wl = synth.config_block_two_phase(T=T) if H == 1 else synth.config_mhar(T=T, H=H)
    N, S, d = wl.N, wl.S, wl.d
    log(f"[bench] {wl.name}: generating done, uploading")
    reps = to_dev(wl.reps, torch.bfloat16)
    parts = to_dev(wl.partials, torch.bfloat16)
    w = to_dev(wl.w, torch.float32)
    g = to_dev(wl.gain, torch.float32)
    del wl
    h = torch.empty((S, T, d), dtype=torch.bfloat16, device="cuda")
    state = torch.empty((S - 1, T, d), dtype=torch.float16, device="cuda")  # scaled fp16 state
    lse = torch.empty((S, H, T), dtype=torch.float32, device="cuda")
    oscale = torch.empty((T,), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(S + 1)] for _ in range(args.steps)]
    k = {"i": -1}

    # record: None, "p1" (events around Phase 1 only) or "all" (also after each merge).
    def step(record=None):
        e = ev[k["i"]] if record else None
        if e:
            e[0].record(stream)
        ar.attnres_block_phase1(reps, w, g, 1e-6, H, h_first=h[0], o_state=state, lse=lse, o_scale=oscale,
                                stream=stream)
        if e:
            e[1].record(stream)
        for i in range(2, S + 1):
            ar.attnres_block_phase2_merge(state[i - 2], lse[i - 1], parts[i - 2], w[i - 1], g[i - 1], 1e-6,
                                          H, h_i=h[i - 1], o_scale=oscale, stream=stream)
            if e and record == "all":
                e[i].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(args.steps):
        k["i"] = s
        step(record="p1" if with_events else None)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = start.elapsed_time(end) / 1e3
    p1_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)]
    # The merges' own durations come from a second pass with an event after each
    # launch, outside the timed region: every recorded event adds a gap to the
    # step, so the timed steps carry only the two events around Phase 1.
    for s in range(args.steps):
        k["i"] = s
        step(record="all" if with_events else None)
    torch.cuda.synchronize()
    p2_ms = [ev[s][i - 1].elapsed_time(ev[s][i]) for s in range(args.steps) for i in range(2, S + 1)]
    p1_b, p2_b, step_b = block_bytes(T, d, N, S, H)
    p1_avg = sum(p1_ms) / len(p1_ms) / 1e3
    p2_avg = sum(p2_ms) / len(p2_ms) / 1e3
    res = dict(
        name=name or f"block_two_phase_bf16_T{T}_d{d}_N{N}_S{S}_H{H}",
        T=T, d=d, N=N, S=S, H=H, seconds=total, wall=wall,
        tokens_per_s=T * args.steps / total, ms_per_step=total / args.steps * 1e3,
        step_bytes=step_b, step_gbs=step_b * args.steps / total / 1e9,
        phase1=dict(bytes_per_launch=p1_b, avg_us=p1_avg * 1e6, gbs=p1_b / p1_avg / 1e9),
        phase2=dict(bytes_per_launch=p2_b, avg_us=p2_avg * 1e6, gbs=p2_b / p2_avg / 1e9),
    )
    if cold_steps:
        # Cold-cache steps: before each, 1 GiB is written to a scratch buffer
        # (four times the 256 MiB last-level cache), outside the timed events.
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        ms = []
        for _ in range(cold_steps):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        del flush
        ms.sort()
        q = lambda f: ms[min(len(ms) - 1, int(f * len(ms)))]
        res["cold"] = dict(steps=cold_steps, ms_median=q(0.5), ms_p10=q(0.1), ms_p90=q(0.9),
                           tokens_per_s_median=T / (q(0.5) / 1e3))
    return res


def update_bytes(T, d, H, first, es=2, state_es=2):
    """Algorithmic bytes of one fused Phase-2 update: reads the state row, H lse
    values, the scale, the previous partial (absent for the block's first
    update) and f; writes the updated partial, h_i and one fp32 inverse RMS."""
    return T * (d * state_es + H * 4 + 4 + (0 if first else d * es) + d * es + 2 * d * es + 4)


def bench_update(args, T=16384):
    """Block two-phase as a model runs it: Phase 1, then per sublayer i >= 2 the
    fused update b_{i-1} = b_{i-2} + f_{i-1} (in place), merge and inverse RMS."""
    import torch
    import depth_wise_attention_amd as ar
    from workloads import synth

    wl = synth.block_workload(T=T, d=4096, N=8, S=4, H=1, rep_std_step=0.3, dtype="bf16", seed=0, with_f=True)
    N, S, d, H = wl.N, wl.S, wl.d, 1
    reps = to_dev(wl.reps, torch.bfloat16)
    f = to_dev(wl.f, torch.bfloat16)
    w = to_dev(wl.w, torch.float32)
    g = to_dev(wl.gain, torch.float32)
    del wl
    h = torch.empty((S, T, d), dtype=torch.bfloat16, device="cuda")
    state = torch.empty((S - 1, T, d), dtype=torch.float16, device="cuda")
    lse = torch.empty((S, H, T), dtype=torch.float32, device="cuda")
    oscale = torch.empty((T,), dtype=torch.float32, device="cuda")
    part = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    rms = torch.empty((S - 1, T), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(S + 1)] for _ in range(args.steps)]

    def step(e=None):
        if e:
            e[0].record(stream)
        ar.attnres_block_phase1(reps, w, g, 1e-6, H, h_first=h[0], o_state=state, lse=lse, o_scale=oscale,
                                stream=stream)
        if e:
            e[1].record(stream)
        for i in range(2, S + 1):
            ar.attnres_block_phase2_merge_update(state[i - 2], lse[i - 1], None if i == 2 else part, f[i - 2],
                                                 w[i - 1], g[i - 1], 1e-6, H, partial_out=part, h_i=h[i - 1],
                                                 norm_eps=1e-6, h_inv_rms=rms[i - 2], o_scale=oscale,
                                                 stream=stream)
            if e:
                e[i].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(args.steps):
        step(ev[s])
    end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end) / 1e3
    p1_b, _, _ = block_bytes(T, d, N, S, H)
    first_b, next_b = update_bytes(T, d, H, True), update_bytes(T, d, H, False)
    first_us = sum(ev[s][1].elapsed_time(ev[s][2]) for s in range(args.steps)) / args.steps * 1e3
    next_us = sum(ev[s][i - 1].elapsed_time(ev[s][i]) for s in range(args.steps)
                  for i in range(3, S + 1)) / (args.steps * (S - 2)) * 1e3
    step_b = p1_b + first_b + (S - 2) * next_b
    return dict(
        name=f"block_fused_update_bf16_T{T}_d{d}_N{N}_S{S}_H{H}", T=T, d=d, N=N, S=S, H=H, seconds=total,
        tokens_per_s=T * args.steps / total, ms_per_step=total / args.steps * 1e3,
        step_bytes=step_b, step_gbs=step_b * args.steps / total / 1e9,
        update_first=dict(bytes_per_launch=first_b, avg_us=first_us, gbs=first_b / first_us / 1e3),
        update=dict(bytes_per_launch=next_b, avg_us=next_us, gbs=next_b / next_us / 1e3),
    )


def bench_decode(args, Ts=(1, 16, 64, 256), iters=200):
    """Decode-size latency: one block step (Phase 1 + S-1 fused updates, d=4096,
    N=8, S=4) and one Full AttnRes sublayer (one destination over 32 sources,
    d=2048), per call, launched eagerly, replayed from a captured HIP graph of
    one call, and per call inside a graph of 8."""
    import torch
    import depth_wise_attention_amd as ar

    def timed(fn):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters

    def graphed(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return timed(g.replay)

    out = {}
    gen = torch.Generator(device="cuda").manual_seed(0)
    for T in Ts:
        N, S, d = 8, 4, 4096
        reps = torch.randn((N, T, d), device="cuda", generator=gen).to(torch.bfloat16)
        f = torch.randn((S - 1, T, d), device="cuda", generator=gen).to(torch.bfloat16)
        w = torch.randn((S, d), device="cuda", generator=gen) / d ** 0.5
        g = 1 + 0.1 * torch.randn((S, d), device="cuda", generator=gen)
        h = torch.empty((S, T, d), dtype=torch.bfloat16, device="cuda")
        st = torch.empty((S - 1, T, d), dtype=torch.float16, device="cuda")
        lse = torch.empty((S, 1, T), device="cuda")
        sc = torch.empty((T,), device="cuda")
        part = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        rms = torch.empty((S - 1, T), device="cuda")

        def block_step():
            ar.attnres_block_phase1(reps, w, g, 1e-6, 1, h_first=h[0], o_state=st, lse=lse, o_scale=sc)
            for i in range(2, S + 1):
                ar.attnres_block_phase2_merge_update(st[i - 2], lse[i - 1], None if i == 2 else part, f[i - 2],
                                                     w[i - 1], g[i - 1], 1e-6, 1, partial_out=part, h_i=h[i - 1],
                                                     norm_eps=1e-6, h_inv_rms=rms[i - 2], o_scale=sc)

        L, dF = 32, 2048
        src = torch.randn((L, T, dF), device="cuda", generator=gen).to(torch.bfloat16)
        wF = torch.randn((1, dF), device="cuda", generator=gen) / dF ** 0.5
        outF = torch.empty((1, T, dF), dtype=torch.bfloat16, device="cuda")
        wsF = torch.empty(max(1, ar.attnres_full_fwd_workspace_size(L, 1, dF, 1, ar.BF16)), dtype=torch.uint8,
                          device="cuda")

        def full_sublayer():
            ar.attnres_full_fwd(src, wF, None, 1e-6, 1, out=outF, ws=wsF)

        def block_steps8():
            for _ in range(8):
                block_step()

        def full_sublayers8():
            for _ in range(8):
                full_sublayer()

        # Each graph replay carries a fixed launch cost; a model captures many
        # steps in one graph, so the per-step cost inside an 8-step graph is
        # reported beside the one-step graph.
        out[f"T{T}"] = dict(block_step_eager_us=timed(block_step), block_step_graph_us=graphed(block_step),
                            block_step_in_graph_of_8_us=graphed(block_steps8) / 8,
                            full_sublayer_eager_us=timed(full_sublayer), full_sublayer_graph_us=graphed(full_sublayer),
                            full_sublayer_in_graph_of_8_us=graphed(full_sublayers8) / 8)
    return dict(name="decode_latency_block_d4096_N8_S4_full_d2048_L32", **out)


def msar_flops(T, d, n):
    """Algorithmic flops of one MSAR call with one destination over n sources:
    per token and channel, 24 taps per source for the three convolved streams,
    a square and a query product per source and stream for the scores, a
    weighted sum per source and stream, and the mixer's squares (4), projections
    (16) and output sum (4); two flops per multiply-add."""
    return 2 * T * d * (n * (24 + 8 + 4) + 24)


def bench_msar(args, T=16384, d=4096, n=9):
    """A Block MSAR sublayer: one destination over 8 block reps and the partial."""
    import torch
    import depth_wise_attention_amd as ar
    from workloads import synth

    wl = synth.msar_workload(T=T, d=d, n_src=n, n_dst=1, dtype="bf16", seed=0)
    src = to_dev(wl.src, torch.bfloat16)
    w = to_dev(wl.w, torch.float32)
    conv = to_dev(wl.meta["conv"], torch.float32)
    mix = to_dev(wl.meta["mix"], torch.float32)
    del wl
    out = torch.empty((1, T, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, ar.attnres_msar_fwd_workspace_size(n, 1, T, d, ar.BF16)), dtype=torch.uint8,
                     device="cuda")
    fn = lambda: ar.attnres_msar_fwd(src, w, conv, mix, 1e-6, out=out, ws=ws)
    total, wall = time_loop(fn, args.steps, args.warmup)
    per = total / args.steps
    flops = msar_flops(T, d, n)
    nbytes = T * (n + 1) * d * 2
    return dict(name=f"msar_block_sublayer_bf16_T{T}_d{d}_sources{n}", T=T, d=d, seconds=total,
                tokens_per_s=T * args.steps / total, ms_per_call=per * 1e3, flops_per_call=flops,
                tflops=flops / per / 1e12, bytes_per_call=nbytes, gbs=nbytes / per / 1e9)


def bench_block_msar(args, T=16384, d=4096, N=8, S=4):
    """One Block MSAR block, two-phase: Phase 1 over the 8 reps for the 4
    sublayers, then 3 Phase-2 merges (the reps' streams are expanded once per
    block instead of once per sublayer)."""
    import torch
    import depth_wise_attention_amd as ar
    from workloads import synth

    wl = synth.block_msar_workload(T=T, d=d, N=N, S=S, seed=0)
    reps = to_dev(wl.reps, torch.bfloat16)
    parts = to_dev(wl.partials, torch.bfloat16)
    w = to_dev(wl.w, torch.float32)
    conv = to_dev(wl.meta["conv"], torch.float32)
    mix = to_dev(wl.meta["mix"], torch.float32)
    del wl
    h = torch.empty((S, T, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((S - 1, 4, T, d), dtype=torch.float16, device="cuda")
    osc = torch.empty((T,), dtype=torch.float32, device="cuda")
    lse = torch.empty((S - 1, 4, T), dtype=torch.float32, device="cuda")
    ws1 = torch.empty(ar.attnres_block_msar_phase1_workspace_size(N, S, T, d), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(ar.attnres_block_msar_phase2_workspace_size(T, d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(S + 1)] for _ in range(args.steps)]

    def step(e=None):
        if e:
            e[0].record(stream)
        ar.attnres_block_msar_phase1(reps, w, conv, mix[0], 1e-6, h1=h[0], o_state=o, o_scale=osc, lse=lse, ws=ws1,
                                     stream=stream)
        if e:
            e[1].record(stream)
        for i in range(2, S + 1):
            ar.attnres_block_msar_phase2(o[i - 2], osc, lse[i - 2], parts[i - 2], w[i - 1], conv, mix[i - 1], 1e-6,
                                         h_i=h[i - 1], ws=ws2, stream=stream)
            if e:
                e[i].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s_ in range(args.steps):
        step(ev[s_])
    end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end) / 1e3
    p1 = sum(ev[k][0].elapsed_time(ev[k][1]) for k in range(args.steps)) / args.steps
    p2 = sum(ev[k][i - 1].elapsed_time(ev[k][i]) for k in range(args.steps) for i in range(2, S + 1)) / (
        args.steps * (S - 1))
    return dict(name=f"block_msar_two_phase_bf16_T{T}_d{d}_N{N}_S{S}", T=T, d=d, N=N, S=S, seconds=total,
                tokens_per_s=T * args.steps / total, ms_per_step=total / args.steps * 1e3, phase1_ms=p1,
                phase2_ms=p2)


def bench_full(args, T=4096, H=1):
    """Full AttnRes forward at the C2 shape (T=4096, d=2048, L=32), one head or
    H heads of d/H channels (each with its own depth softmax)."""
    import torch
    import depth_wise_attention_amd as ar
    from workloads import synth

    wl = synth.config_full_bf16(T=T)
    src = to_dev(wl.src, torch.bfloat16)
    w = to_dev(wl.w, torch.float32)
    g = to_dev(wl.gain, torch.float32)
    L, d = wl.src.shape[0], wl.d
    del wl
    out = torch.empty((L, T, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, ar.attnres_full_fwd_workspace_size(L, L, d, H, ar.BF16)), dtype=torch.uint8,
                     device="cuda")
    sec, wall = time_loop(lambda: ar.attnres_full_fwd(src, w, g, 1e-6, H, out=out, ws=ws),
                          max(3, args.steps // 4), 2)
    n = max(3, args.steps // 4)
    b = full_bytes(T, d, L)
    tag = "" if H == 1 else f"_H{H}"
    return dict(name=f"full_bf16_T{T}_d{d}_L{L}{tag}", tokens_per_s=T * n / sec, ms_per_step=sec / n * 1e3,
                step_bytes=b, step_gbs=b * n / sec / 1e9,
                kernel=ar.attnres_kernel_variant(ar.OP_FULL_FWD, L, L, T, d, H))


def bench_full_wide(args, T=4096, d=2048, L=55):
    """Full AttnRes with more sources than one 32-source tile: the deepest
    sublayer of a 54-sublayer model reads L = 55 sources.  The forward with one
    destination (the per-sublayer call) and with 54 (every destination at once),
    and the backward with one and with 32 destinations, each timed with HIP
    events around its launches.  Sources are seeded normal draws made on the
    device, source i with standard deviation 1 + 0.2 i (the residual stream
    grows with depth), w ~ N(0, 1/d), gain ~ 1 + N(0, 0.01)."""
    import torch
    import depth_wise_attention_amd as ar

    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    stream = torch.cuda.current_stream()
    src = torch.randn((L, T, d), generator=gen, device="cuda")
    src *= (1 + 0.2 * torch.arange(L, device="cuda", dtype=torch.float32))[:, None, None]
    src = src.to(torch.bfloat16)

    def timed(fn, n):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    n = max(3, args.steps // 2)
    cases = {}
    for nd in (1, L - 1):
        w = torch.randn((nd, d), generator=gen, device="cuda") / d ** 0.5
        g = 1 + 0.1 * torch.randn((nd, d), generator=gen, device="cuda")
        out = torch.empty((nd, T, d), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(1, ar.attnres_full_fwd_workspace_size(L, nd, d, 1, ar.BF16)), dtype=torch.uint8,
                         device="cuda")
        us = timed(lambda: ar.attnres_full_fwd(src, w, g, 1e-6, 1, out=out, ws=ws), n)
        b = T * d * 2 * (L + nd)
        cases[f"fwd_n_dst{nd}"] = dict(us=us, bytes=b, gbs=b / us / 1e3,
                                       kernel=ar.attnres_kernel_variant(ar.OP_FULL_FWD, L, nd, T, d, 1))
        del out, ws
    for nd in (1, 32):
        w = torch.randn((nd, d), generator=gen, device="cuda") / d ** 0.5
        g = 1 + 0.1 * torch.randn((nd, d), generator=gen, device="cuda")
        dout = torch.randn((nd, T, d), generator=gen, device="cuda").to(torch.bfloat16)
        d_src = torch.empty_like(src)
        dw, dg = torch.empty_like(w), torch.empty_like(g)
        ws = torch.empty(ar.attnres_full_bwd_workspace_size(L, nd, T, d, 1), dtype=torch.uint8, device="cuda")
        us = timed(lambda: ar.attnres_full_bwd(src, w, dout, g, 1e-6, 1, d_src=d_src, dw=dw, dgain=dg, ws=ws), n)
        b = T * d * 2 * (2 * L + nd)  # read src and dout, write d_src
        cases[f"bwd_n_dst{nd}"] = dict(us=us, bytes=b, gbs=b / us / 1e3,
                                       kernel=ar.attnres_kernel_variant(ar.OP_FULL_BWD, L, nd, T, d, 1))
        del dout, d_src, ws
    return dict(name=f"full_wide_bf16_T{T}_d{d}_L{L}", **cases)


def bench_full_one(args, T=4096, d=2048, Ls=(9, 32, 55)):
    """The per-sublayer Full AttnRes calls of a model: one destination over the
    L sources before it, forward and backward (the backward accumulating into
    d_src, as every later sublayer adds to a source's gradient), for a shallow,
    a 32-source and a 55-source sublayer.  Each is timed with HIP events around
    its launches.  Sources are seeded normal draws made on the device, source i
    with standard deviation 1 + 0.2 i, w ~ N(0, 1/d), gain ~ 1 + N(0, 0.01)."""
    import torch
    import depth_wise_attention_amd as ar

    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    n = max(3, args.steps // 2)
    cases = {}
    for L in Ls:
        src = torch.randn((L, T, d), generator=gen, device="cuda")
        src *= (1 + 0.2 * torch.arange(L, device="cuda", dtype=torch.float32))[:, None, None]
        src = src.to(torch.bfloat16)
        w = torch.randn((1, d), generator=gen, device="cuda") / d ** 0.5
        g = 1 + 0.1 * torch.randn((1, d), generator=gen, device="cuda")
        out = torch.empty((1, T, d), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(1, ar.attnres_full_fwd_workspace_size(L, 1, d, 1, ar.BF16)), dtype=torch.uint8,
                         device="cuda")
        us = timed(lambda: ar.attnres_full_fwd(src, w, g, 1e-6, 1, out=out, ws=ws), n)
        b = T * d * 2 * (L + 1)
        cases[f"fwd_L{L}"] = dict(us=us, bytes=b, gbs=b / us / 1e3,
                                  kernel=ar.attnres_kernel_variant(ar.OP_FULL_FWD, L, 1, T, d, 1))
        dout = torch.randn((1, T, d), generator=gen, device="cuda").to(torch.bfloat16)
        d_src = torch.zeros_like(src)
        dw, dg = torch.zeros_like(w), torch.zeros_like(g)
        wsb = torch.empty(ar.attnres_full_bwd_workspace_size(L, 1, T, d, 1), dtype=torch.uint8, device="cuda")
        us = timed(lambda: ar.attnres_full_bwd(src, w, dout, g, 1e-6, 1, d_src=d_src, dw=dw, dgain=dg, ws=wsb,
                                               accumulate=True), n)
        b = T * d * 2 * (3 * L + 1)  # read src, dout and the old d_src, write d_src
        cases[f"bwd_acc_L{L}"] = dict(us=us, bytes=b, gbs=b / us / 1e3,
                                      kernel=ar.attnres_kernel_variant(ar.OP_FULL_BWD, L, 1, T, d, 1))
        del src, out, ws, dout, d_src, wsb
    return dict(name=f"full_one_bf16_T{T}_d{d}", **cases)


def bench_f32(args):
    """fp32 I/O, which runs the general kernels at every shape: the headline
    block step (mhar_fwd, T=16384, d=4096, N=8, S=4), the Full forward over 32
    sources and destinations (T=4096, d=2048) and the one-destination Full
    call over 32 sources, each timed with HIP events over 3 calls after one
    warm-up call, on seeded normal inputs made on the device."""
    import torch
    import depth_wise_attention_amd as ar

    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    stream = torch.cuda.current_stream()

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    out = {}
    T, d, N, S = 16384, 4096, 8, 4
    reps = torch.randn((N, T, d), generator=gen, device="cuda")
    parts = torch.randn((S - 1, T, d), generator=gen, device="cuda")
    w = torch.randn((S, d), generator=gen, device="cuda") / d ** 0.5
    g = 1 + 0.1 * torch.randn((S, d), generator=gen, device="cuda")
    out["block_T16384_d4096_N8_S4_ms"] = timed(lambda: ar.mhar_fwd(reps, parts, w, g, 1e-6, 1))
    out["block_kernel"] = ar.attnres_kernel_variant(ar.OP_PHASE1, N, S, T, d, 1, dtype=ar.F32, o_dtype=ar.F32)
    del reps, parts
    Tf, df, L = 4096, 2048, 32
    src = torch.randn((L, Tf, df), generator=gen, device="cuda")
    wf = torch.randn((L, df), generator=gen, device="cuda") / df ** 0.5
    out["full_T4096_d2048_L32_ms"] = timed(lambda: ar.attnres_full_fwd(src, wf, None, 1e-6, 1))
    w1 = wf[:1].contiguous()
    out["full_one_destination_T4096_d2048_L32_ms"] = timed(lambda: ar.attnres_full_fwd(src, w1, None, 1e-6, 1))
    out["full_kernel"] = ar.attnres_kernel_variant(ar.OP_FULL_FWD, L, L, Tf, df, 1, dtype=ar.F32)
    return dict(name="f32_io_general_kernels", **out)


def bench_bwd(args, T=8192, H=1):
    import torch
    import depth_wise_attention_amd as ar
    from workloads import synth

    wl = synth.config_block_fwd_bwd(T=T) if H == 1 else synth.config_mhar_fwd_bwd(T=T, H=H)
    reps, parts, dh = (to_dev(x, torch.bfloat16) for x in (wl.reps, wl.partials, wl.dh))
    w, g = to_dev(wl.w, torch.float32), to_dev(wl.gain, torch.float32)
    N, S, d = wl.N, wl.S, wl.d
    del wl
    h = torch.empty((S, T, d), dtype=torch.bfloat16, device="cuda")
    ws_f = torch.empty(ar.mhar_fwd_workspace_size(N, S, T, d, H), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(ar.attnres_bwd_workspace_size(N, S, T, d, H), dtype=torch.uint8, device="cuda")
    d_reps, d_parts = torch.empty_like(reps), torch.empty_like(parts)
    dw, dg = torch.empty_like(w), torch.empty_like(g)

    def step():
        ar.mhar_fwd(reps, parts, w, g, 1e-6, H, h=h, ws=ws_f)
        ar.attnres_bwd(reps, parts, w, dh, g, 1e-6, H, d_reps=d_reps, d_partials=d_parts, dw=dw, dgain=dg,
                       ws=ws_b)

    n = max(3, args.steps // 4)
    sec, wall = time_loop(step, n, 2)
    fwd_b = block_bytes(T, d, N, S, H)[2]
    b = fwd_b + bwd_bytes(T, d, N, S)
    kind = "block" if H == 1 else f"mhar_H{H}"
    return dict(name=f"{kind}_fwd_bwd_bf16_T{T}_d{d}_N{N}_S{S}", tokens_per_s=T * n / sec,
                ms_per_step=sec / n * 1e3, step_bytes=b, step_gbs=b * n / sec / 1e9)


def bench_depth_sweep(args, T=16384, Tb=8192, d=4096):
    """Phase 1 at every block depth (block n of a model reads N = n reps), S = 4,
    plus the 6-sublayer block of the 54-sublayer model (N = 9, S = 6), and the
    Block backward at N = 1..12, S = 4, and at (9, 6) and (8, 8), which run as two
    destination chunks.  Inputs are seeded normal draws made on
    the device (rep n with std 1 + 0.3 n); each case's kernel is timed with HIP
    events around its launches on the stream they run on."""
    import torch
    import depth_wise_attention_amd as ar

    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    stream = torch.cuda.current_stream()

    def reps_of(N, TT):
        r = torch.randn((N, TT, d), generator=gen, device="cuda")
        r *= (1 + 0.3 * torch.arange(N, device="cuda", dtype=torch.float32))[:, None, None]
        return r.to(torch.bfloat16)

    def timed(fn, n):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    n = max(5, args.steps // 2)
    phase1, bwd = [], []
    for N, S in [(k, 4) for k in range(1, 13)] + [(9, 6)]:
        reps = reps_of(N, T)
        w = torch.randn((S, d), generator=gen, device="cuda") / 64
        g = 1 + 0.1414 * torch.randn((S, d), generator=gen, device="cuda")
        h0 = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        st = torch.empty((S - 1, T, d), dtype=torch.float16, device="cuda")
        lse = torch.empty((S, 1, T), device="cuda")
        sc = torch.empty((T,), device="cuda")
        sec = timed(lambda: ar.attnres_block_phase1(reps, w, g, 1e-6, 1, h_first=h0, o_state=st, lse=lse,
                                                    o_scale=sc, stream=stream), n)
        b = block_bytes(T, d, N, S, 1)[0]
        phase1.append(dict(N=N, S=S, kernel=ar.attnres_kernel_variant(ar.OP_PHASE1, N, S, T, d, 1),
                           us=sec * 1e6, gbs=b / sec / 1e9, frac_of_peak=b / sec / 1e9 / PEAK_HBM_GBS))
        log(f"[bench] depth sweep phase1 {json.dumps(phase1[-1])}")
        del reps, h0, st
        torch.cuda.empty_cache()
    for N, S in [(k, 4) for k in range(1, 13)] + [(9, 6), (8, 8)]:
        reps = reps_of(N, Tb)
        parts = torch.randn((S - 1, Tb, d), generator=gen, device="cuda").to(torch.bfloat16)
        dh = torch.randn((S, Tb, d), generator=gen, device="cuda").to(torch.bfloat16)
        w = torch.randn((S, d), generator=gen, device="cuda") / 64
        g = 1 + 0.1414 * torch.randn((S, d), generator=gen, device="cuda")
        outs = (torch.empty_like(reps), torch.empty_like(parts), torch.empty_like(w), torch.empty_like(g))
        ws = torch.empty(ar.attnres_bwd_workspace_size(N, S, Tb, d, 1), dtype=torch.uint8, device="cuda")
        sec = timed(lambda: ar.attnres_bwd(reps, parts, w, dh, g, 1e-6, 1, d_reps=outs[0], d_partials=outs[1],
                                           dw=outs[2], dgain=outs[3], ws=ws, stream=stream), n)
        b = bwd_bytes(Tb, d, N, S)
        bwd.append(dict(N=N, S=S, kernel=ar.attnres_kernel_variant(ar.OP_BWD, N, S, Tb, d, 1), us=sec * 1e6,
                        gbs=b / sec / 1e9, frac_of_peak=b / sec / 1e9 / PEAK_HBM_GBS))
        log(f"[bench] depth sweep bwd {json.dumps(bwd[-1])}")
        del reps, parts, dh, outs, ws
        torch.cuda.empty_cache()
    return dict(name=f"depth_sweep_d{d}", T_phase1=T, T_bwd=Tb, phase1=phase1, bwd=bwd)


def full_bwd_bytes(T, d, L, es=2):
    # read src and dout, write d_src (the dw/dgain slabs are small)
    return T * d * es * (L + L + L)


def bench_full_bwd(args, T=4096, H=1):
    import torch
    import depth_wise_attention_amd as ar
    from workloads import synth

    wl = synth.config_full_fwd_bwd(T=T)
    src, dout = to_dev(wl.src, torch.bfloat16), to_dev(wl.dh, torch.bfloat16)
    w, g = to_dev(wl.w, torch.float32), to_dev(wl.gain, torch.float32)
    L, d = wl.src.shape[0], wl.d
    del wl
    out = torch.empty((L, T, d), dtype=torch.bfloat16, device="cuda")
    ws_f = torch.empty(max(1, ar.attnres_full_fwd_workspace_size(L, L, d, H, ar.BF16)), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(ar.attnres_full_bwd_workspace_size(L, L, T, d, H), dtype=torch.uint8, device="cuda")
    d_src, dw, dg = torch.empty_like(src), torch.empty_like(w), torch.empty_like(g)

    def step():
        ar.attnres_full_fwd(src, w, g, 1e-6, H, out=out, ws=ws_f)
        ar.attnres_full_bwd(src, w, dout, g, 1e-6, H, d_src=d_src, dw=dw, dgain=dg, ws=ws_b)

    n = max(3, args.steps // 4)
    sec, wall = time_loop(step, n, 2)
    b = full_bytes(T, d, L) + full_bwd_bytes(T, d, L)
    tag = "" if H == 1 else f"_H{H}"
    return dict(name=f"full_fwd_bwd_bf16_T{T}_d{d}_L{L}{tag}", tokens_per_s=T * n / sec,
                ms_per_step=sec / n * 1e3, step_bytes=b, step_gbs=b * n / sec / 1e9,
                kernels=[ar.attnres_kernel_variant(ar.OP_FULL_FWD, L, L, T, d, H),
                         ar.attnres_kernel_variant(ar.OP_FULL_BWD, L, L, T, d, H)])


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_chunk(args):
    """One token chunk of the headline workload through the oracle (a worker
    process of the P-core baseline, BLAS at one thread)."""
    reps, parts, w, gain, eps = args
    from threadpoolctl import threadpool_limits
    from oracle import attnres_oracle as orc
    with threadpool_limits(1):
        t0 = time.perf_counter()
        orc.block_direct(reps, parts, w, gain, eps, 1)
        return time.perf_counter() - t0


def cpu_baseline(T=16384, chunk=256, sample=16384):
    """The float64 oracle (as it stands) on the headline block workload, on the
    host's cores: (1) one process with BLAS pinned to one thread over a bounded
    sample of `sample` tokens, and (2) a pool of P worker processes (P = the
    cores this process may run on, at most 16), each with BLAS at one thread,
    over the same sample split into token chunks.  Tokens are independent, so
    chunking changes nothing but peak memory; tokens/s scales to the full T."""
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits
    from oracle import attnres_oracle as orc
    from workloads import synth

    wl = synth.config_block_two_phase(T=T)
    n = min(sample, T)
    tasks = [(np.ascontiguousarray(wl.reps[:, lo:lo + chunk]), np.ascontiguousarray(wl.partials[:, lo:lo + chunk]),
              wl.w, wl.gain, wl.eps) for lo in range(0, n, chunk)]
    del wl
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for reps, parts, w, gain, eps in tasks:
            orc.block_direct(reps, parts, w, gain, eps, 1)
        one = time.perf_counter() - t0
    P = max(1, min(16, len(os.sched_getaffinity(0)))) if hasattr(os, "sched_getaffinity") else 1
    with ProcessPoolExecutor(P, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_chunk, tasks[:P]))  # start the workers and import the oracle
        t0 = time.perf_counter()
        list(ex.map(_oracle_chunk, tasks))
        many = time.perf_counter() - t0
    model = _cpu_model()
    return dict(value=n / one, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{n} of the {T} tokens of the d=4096 N=8 S=4 H=1 block workload in chunks of {chunk}, "
                       f"float64 numpy oracle (plain definition), BLAS at one thread, {one:.1f} s",
                cpu_model=model,
                p_cores=dict(value=n / many, unit="tokens/s", cores=P, kind="oracle",
                             sample=f"the same {n} tokens over {P} worker processes (one BLAS thread each), "
                                    f"{many:.1f} s"))


def copy_calibration(n=1 << 31, reps=10):
    """A plain device-to-device copy of n bytes: the counter-calibration kernel
    and the measured streaming ceiling (read n + write n bytes per copy)."""
    import torch
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        b.copy_(a)
    end.record()
    torch.cuda.synchronize()
    sec = start.elapsed_time(end) / 1e3 / reps
    res = dict(copy_bytes=n, read_plus_write_gbs=2 * n / sec / 1e9, us=sec * 1e6)
    log(f"[bench] copy: {json.dumps(res)}")
    return res


# Streaming-pattern ceilings: each routing kernel's per-token read/write mix
# with no arithmetic (libattnres_probe.so), for the roofline discussion.
# Every pattern moves at least 1 GiB per pass, four times the 256 MiB
# last-level cache, so repeated passes are not served from it.
CEILING_PATTERNS = [
    # name, rows read, rows written, T, d
    ("read_only", 8, 0, 16384, 4096),
    ("write_only", 0, 4, 32768, 4096),
    ("copy_1_to_1", 1, 1, 65536, 4096),
    ("block_phase1", 8, 4, 16384, 4096),
    ("block_phase2", 2, 1, 65536, 4096),
    ("block_backward", 15, 11, 8192, 4096),
    ("full_forward", 32, 32, 4096, 2048),
]


# Flavours of the probe's memory operations (its `mode` argument).
PROBE_MODES = {0: "nt loads, nt stores, 16 B per lane", 1: "plain loads, nt stores, 16 B per lane",
               2: "nt loads, plain stores, 16 B per lane", 3: "plain loads, plain stores, 16 B per lane",
               4: "nt loads, nt stores, 32 B per lane", 5: "plain loads, nt stores, 32 B per lane",
               6: "nt loads, plain stores, 32 B per lane", 7: "plain loads, plain stores, 32 B per lane"}


def pattern_ceilings(reps=10, only=None, blocks=(2, 4, 8, 16, 32), modes=(0,)):
    """Best rate of each pattern over the given workgroups per CU and probe modes."""
    import ctypes
    import torch
    from depth_wise_attention_amd import build as b

    if not os.path.exists(b.PROBE_LIB):
        raise RuntimeError(f"{b.PROBE_LIB} is missing: run __graft_entry__.build() first")
    probe = ctypes.CDLL(b.PROBE_LIB)
    probe.attnres_probe_stream.restype = ctypes.c_int
    probe.attnres_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = []
    for name, nr, nw, T, d in CEILING_PATTERNS:
        if only is not None and name not in only:
            continue
        src = torch.randint(-2**15, 2**15, (max(nr, 1), T, d), dtype=torch.int16, device="cuda")
        dst = torch.empty((max(nw, 1), T, d), dtype=torch.int16, device="cuda")
        best = None
        per_mode = {}
        by_blocks = {}  # the kernels' flavour (mode 0) at each occupancy
        for mode in modes:
            for per_cu in blocks:
                nblk = cus * per_cu
                run = lambda: probe.attnres_probe_stream(ctypes.c_void_p(src.data_ptr()), nr,
                                                         ctypes.c_void_p(dst.data_ptr()), nw, T, d,
                                                         ctypes.c_void_p(sink.data_ptr()), nblk, mode,
                                                         ctypes.c_void_p(stream.cuda_stream))
                for _ in range(2):
                    if run() != 0:
                        raise RuntimeError(f"probe launch failed for {name}")
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    run()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                gbs = (nr + nw) * T * d * 2 / (us * 1e-6) / 1e9
                if mode not in per_mode or gbs > per_mode[mode]["gbs"]:
                    per_mode[mode] = dict(gbs=gbs, us=us, blocks_per_cu=per_cu)
                if mode == 0:
                    by_blocks[per_cu] = dict(gbs=gbs, us=us)
                if best is None or gbs > best["gbs"]:
                    best = dict(pattern=name, rows_read=nr, rows_written=nw, T=T, d=d, bytes=(nr + nw) * T * d * 2,
                                us=us, gbs=gbs, blocks_per_cu=per_cu, mode=PROBE_MODES[mode])
        if len(modes) > 1:
            best["by_mode"] = {PROBE_MODES[m]: v for m, v in per_mode.items()}
        if by_blocks:
            best["mode0_by_blocks_per_cu"] = by_blocks
        log(f"[bench] ceiling {json.dumps(best)}")
        out.append(best)
        del src, dst
        torch.cuda.empty_cache()
    return {"pattern_ceilings": out}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the routing shards along "
              f"tokens with no exchange, so multi-GPU throughput is N times the one-GPU figure and is not "
              f"measured here.", file=sys.stderr)
        sys.exit(2)
    import torch
    import depth_wise_attention_amd as ar

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    ar.lib()  # fail loudly if the HIP library is missing
    if args.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return
    if args.ceilings:
        print(json.dumps(pattern_ceilings(modes=tuple(range(8)))), flush=True)
        return

    if args.workload != "block":
        fn = {"mhar": lambda: bench_block(args, H=8, T=32768), "full": lambda: bench_full(args),
              "full_h8": lambda: bench_full(args, H=8), "full_bwd_h8": lambda: bench_full_bwd(args, H=8),
              "bwd": lambda: bench_bwd(args), "mhar_bwd": lambda: bench_bwd(args, H=8), "full_bwd": lambda: bench_full_bwd(args),
              "block_update": lambda: bench_update(args), "decode": lambda: bench_decode(args),
              "msar": lambda: bench_msar(args), "block_msar": lambda: bench_block_msar(args),
              "depth_sweep": lambda: bench_depth_sweep(args), "full_wide": lambda: bench_full_wide(args),
              "full_one": lambda: bench_full_one(args), "f32": lambda: bench_f32(args)}[args.workload]
        log(json.dumps(fn()))
        return

    head = bench_block(args, cold_steps=10)
    log(f"[bench] headline: {json.dumps(head)}")
    src_hash = kernel_source_hash("p1_kernel.hpp", "p1_fast.hip", "xlane.hpp", "common.hpp")
    traffic = counters_for("phase1_block_T16384_d4096_N8_S4_H1", src_hash)
    p1 = head["phase1"]
    extra = {}
    if not args.no_extra:
        torch.cuda.empty_cache()
        for fn in (lambda: bench_block(args, H=8, T=32768, with_events=True), lambda: bench_full(args),
                   lambda: bench_bwd(args), lambda: bench_bwd(args, H=8), lambda: bench_full_bwd(args), lambda: bench_update(args),
                   lambda: bench_decode(args), lambda: bench_msar(args), lambda: bench_block_msar(args),
                   lambda: bench_full_wide(args), lambda: bench_full_one(args)):
            r = fn()
            extra[r.pop("name")] = {k: v for k, v in r.items() if k not in ("T", "d", "N", "S", "H")}
            torch.cuda.empty_cache()
    line = {
        "metric": "Block AttnRes routing tokens/s + achieved HBM GB/s (% peak), d=4096 N=8 S=4",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": head["name"], "T": head["T"], "d": head["d"], "N": head["N"], "S": head["S"],
            "H": head["H"], "io_dtype": "bf16", "state_dtype": "f16 scaled per token by a power of two",
            "step": "phase1 + 3 phase2 merges (the launches of mhar_fwd)",
            "step_bytes_per_token": head["step_bytes"] // head["T"],
            "step_gbs": head["step_gbs"], "step_frac_of_peak": head["step_gbs"] / PEAK_HBM_GBS,
            "phase2_gbs": head["phase2"]["gbs"], "phase2_avg_us": head["phase2"]["avg_us"],
            "cold_cache_steps": head.get("cold"),
        },
        "roofline": {
            "kernel": "k_p1<8,4,2,false> (Block Phase 1)",
            "bound": "hbm",
            "achieved": p1["gbs"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": p1["gbs"] / PEAK_HBM_GBS,
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "avg_us": p1["avg_us"],
            "algorithmic_bytes_per_launch": p1["bytes_per_launch"],
        },
        "extra_workloads": extra,
    }
    # The same box's streaming ceiling for Phase 1's read/write pattern (no
    # arithmetic), so that frac can be read against what the pattern reaches.
    try:
        ceil = pattern_ceilings(only=("block_phase1",), blocks=(8, 16), modes=(0, 2))["pattern_ceilings"][0]
        line["roofline"]["pattern_ceiling_gbs"] = ceil["gbs"]
        line["roofline"]["frac_of_pattern_ceiling"] = p1["gbs"] / ceil["gbs"]
    except (RuntimeError, OSError) as e:
        log(f"[bench] pattern ceiling not measured: {e}")
        line["roofline"]["pattern_ceiling_gbs"] = None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
