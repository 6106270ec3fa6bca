"""Every specialised kernel variant the dispatcher can select, against the oracle.

tests/test_dispatch.py fixes which kernel each shape runs (host logic, no
GPU).  Here every one of those variants runs on the GPU through the C ABI and
is compared with the oracle on the same seeded inputs:

  * Block Phase 1 for every block depth N = 1..12 and S = 1..8 at d = 4096,
    every width class (d = 512 .. 8192, one or two chunks per thread), and
    heads of whole 512-channel segments;
  * the Block backward for N = 1..12, S = 1..4, widths and heads;
  * the Full forward's matrix-core kernel with heads (H = 2, 4, 8; d = 512 ..
    2048), with one token per workgroup (query operands formed in the
    kernel) and with several;
  * the Full forward over 33 .. 64 sources (two source tiles, one or two
    destination tiles) and the backward over 33 .. 64 sources and up to 32
    destinations;
  * the Full backward's register-resident kernel (d = 1024 .. 2048, one head
    or H = 2, 4, 8 heads of whole waves) and the staged one, over source /
    destination counts, gains and accumulation;
  * a sharply peaked depth softmax (scores in the hundreds), where the
    merge's exp(lse - m) underflows to zero.

Each case first asserts that the dispatcher picks the specialised kernel, so a
shape that silently fell to the general kernel would fail here.  Cases with
T above the number of resident workgroups give each workgroup several tokens
and a ragged tail.
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


def dev(x, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


# (N, S, d, H, T)
PHASE1_CASES = (
    [(N, S, 4096, 1, 19) for N in range(1, 13) for S in range(1, 9)]
    + [(8, 4, d, 1, 1100) for d in (512, 1024, 1536, 2048, 3072, 8192)]
    + [(4, 4, d, 1, 700) for d in (1024, 2048, 4096, 8192)]
    + [(9, 6, 2048, 1, 600), (12, 8, 512, 1, 900), (5, 3, 4096, 1, 1300), (1, 1, 4096, 1, 800)]
    + [(8, 4, 4096, H, 700) for H in (2, 4, 8)]
    + [(4, 4, 8192, 16, 300), (8, 4, 2048, 4, 500), (4, 4, 1024, 2, 600), (9, 4, 4096, 8, 400),
       (12, 6, 4096, 8, 300), (3, 7, 2048, 2, 500), (8, 4, 8192, 8, 300)]
)


@pytest.mark.parametrize("N,S,d,H,T", PHASE1_CASES)
def test_phase1_variant(N, S, d, H, T):
    name = ar.attnres_kernel_variant(ar.OP_PHASE1, N, S, T, d, H)
    say(f"phase1 N={N} S={S} d={d} H={H} T={T}: {name}")
    assert name.startswith("phase1_fast"), name
    wl = synth.block_workload(T=T, d=d, N=N, S=S, H=H, rep_std_step=0.3, dtype="bf16", seed=40 + N + 13 * S)
    reps, w, g = dev(wl.reps, True), dev(wl.w), dev(wl.gain)
    parts = dev(wl.partials, True) if S > 1 else None
    # The block forward (Phase 1 with the scaled fp16 state kept in h, then the
    # in-place merges) against the plain definition.
    h = ar.mhar_fwd(reps, parts, w, g, wl.eps, H)
    ref = orc.block_direct(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, H)
    check(host(h), ref, "bf16", "mhar_fwd")
    # Phase 1 alone with the fp32 state: state and statistics against the oracle's Phase 1.
    h_first, o32, lse, _ = ar.attnres_block_phase1(reps, w, g, wl.eps, H, o_dtype=torch.float32)
    o_ref, lse_ref = orc.block_phase1(wl.reps, wl.w, wl.gain, wl.eps, H)
    assert torch.equal(h_first, h[0])
    if S > 1:
        check(host(o32), o_ref[1:], "f32_from_bf16", "phase1 fp32 state")
    np.testing.assert_allclose(host(lse), lse_ref, rtol=0, atol=2e-4)
    if S > 1:
        # the scaled fp16 state: within half an fp16 ulp of the exact state
        _, o16, _, sc = ar.attnres_block_phase1(reps, w, g, wl.eps, H, o_dtype=torch.float16)
        back = host(o16) * host(sc)[None, :, None]
        bound = 2.0 ** -11 * np.abs(o_ref[1:]) * (1 + 1e-3) + 1e-5 * np.sqrt(np.mean(o_ref[1:] ** 2))
        assert np.all(np.abs(back - o_ref[1:]) <= bound)


# (N, S, d, H, T)
BWD_CASES = (
    [(N, S, 4096, 1, 7) for N in range(1, 13) for S in range(1, 5)]
    + [(8, 4, d, 1, 600) for d in (512, 1024, 1536, 2048)]
    + [(8, 4, 4096, H, 300) for H in (2, 4, 8)]
    + [(12, 4, 4096, 8, 200), (3, 2, 2048, 4, 300), (9, 3, 1024, 2, 400), (5, 1, 4096, 1, 700)]
    # more than 4 destinations: two destination chunks
    + [(N, S, 4096, 1, 7) for N in range(1, 13) for S in range(5, 9)]
    + [(9, 6, d, 1, 300) for d in (512, 1024, 2048)] + [(9, 6, 4096, H, 200) for H in (2, 8)]
    + [(4, 8, 1024, 2, 500), (12, 8, 2048, 4, 130), (9, 5, 4096, 1, 1100), (11, 7, 4096, 8, 90),
       (9, 6, 4096, 1, 1), (3, 5, 512, 1, 1)]
)


@pytest.mark.parametrize("N,S,d,H,T", BWD_CASES)
def test_bwd_variant(N, S, d, H, T):
    name = ar.attnres_kernel_variant(ar.OP_BWD, N, S, T, d, H)
    say(f"bwd N={N} S={S} d={d} H={H} T={T}: {name}")
    assert name.startswith("bwd_fast"), name
    wl = synth.block_workload(T=T, d=d, N=N, S=S, H=H, rep_std_step=0.3, dtype="bf16", seed=60 + N + 13 * S,
                              with_dh=True)
    reps, w, g, dh = dev(wl.reps, True), dev(wl.w), dev(wl.gain), dev(wl.dh, True)
    parts = dev(wl.partials, True) if S > 1 else None
    got = ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, H)
    ref = orc.block_bwd(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, H, wl.dh)
    check(host(got[0]), ref[0], "bf16", "d_reps")
    if S > 1:
        check(host(got[1]), ref[1], "bf16", "d_partials")
    check(host(got[2]), ref[2], "f32_from_bf16", "dw")
    check(host(got[3]), ref[3], "f32_from_bf16", "dgain")
    # shared gain: the dgain reduction over destinations
    g1 = (1 + 0.1 * np.random.default_rng(N).standard_normal(d)).astype(np.float32)
    got1 = ar.attnres_bwd(reps, parts, w, dh, dev(g1), wl.eps, H)
    ref1 = orc.block_bwd(wl.reps, wl.partials, wl.w, g1, wl.eps, H, wl.dh)
    check(host(got1[0]), ref1[0], "bf16", "d_reps (shared gain)")
    check(host(got1[3]), ref1[3], "f32_from_bf16", "dgain (shared gain)")


@pytest.mark.parametrize("N,S,d,H", [(9, 6, 2048, 1), (4, 8, 4096, 2), (8, 5, 1024, 1)])
def test_bwd_chunks_accumulate(N, S, d, H):
    """A block of more than 4 destinations runs as two chunks; with accumulate
    the rep gradients of both chunks are added to the given d_reps before the
    one rounding, and the other outputs are added to as usual."""
    T = 260
    name = ar.attnres_kernel_variant(ar.OP_BWD, N, S, T, d, H)
    say(f"bwd chunks accumulate N={N} S={S} d={d} H={H} T={T}: {name}")
    assert name.startswith("bwd_fast") and "S0=%d" % ((S + 1) // 2) in name, name
    wl = synth.block_workload(T=T, d=d, N=N, S=S, H=H, rep_std_step=0.3, dtype="bf16", seed=90 + N + S,
                              with_dh=True)
    reps, w, g, dh = dev(wl.reps, True), dev(wl.w), dev(wl.gain), dev(wl.dh, True)
    parts = dev(wl.partials, True)
    rng = np.random.default_rng(N * 16 + S)
    base = [rng.standard_normal(x.shape) for x in (wl.reps, wl.partials, wl.w, wl.gain)]
    base[0] = host(dev(base[0], True))  # bf16-exact starting values
    base[1] = host(dev(base[1], True))
    outs = [dev(base[0], True), dev(base[1], True), dev(base[2]), dev(base[3])]
    ar.attnres_bwd(reps, parts, w, dh, g, wl.eps, H, d_reps=outs[0], d_partials=outs[1], dw=outs[2],
                   dgain=outs[3], accumulate=True)
    ref = orc.block_bwd(wl.reps, wl.partials, wl.w, wl.gain, wl.eps, H, wl.dh)
    check(host(outs[0]), base[0] + ref[0], "bf16", "d_reps accumulated")
    check(host(outs[1]), base[1] + ref[1], "bf16", "d_partials accumulated")
    check(host(outs[2]), base[2] + ref[2], "f32_from_bf16", "dw accumulated")
    check(host(outs[3]), base[3] + ref[3], "f32_from_bf16", "dgain accumulated")


@pytest.mark.parametrize("H", [1, 8])
@pytest.mark.parametrize("policy", [0, 1], ids=["auto", "general"])
def test_peaked_softmax(H, policy):
    """Scores in the hundreds: the depth softmax is all but one-hot, and the
    merge weight exp(lse - m) or exp(s_p - m) underflows to zero."""
    prev = ar.attnres_set_kernel_policy(policy)
    try:
        wl = synth.block_workload(T=300, d=4096, N=8, S=4, H=H, rep_std_step=0.3, dtype="bf16", seed=77,
                                  with_dh=True)
        wbig = (wl.w * 300.0).astype(np.float32)
        s = orc.block_phase1(wl.reps[:, :4], wbig, wl.gain, wl.eps, H)[1]
        say(f"peaked softmax H={H} policy={policy}: |lse| up to {np.abs(s).max():.0f}")
        assert np.abs(s).max() > 100
        reps, w, g = dev(wl.reps, True), dev(wbig), dev(wl.gain)
        h = ar.mhar_fwd(reps, dev(wl.partials, True), w, g, wl.eps, H)
        ref = orc.block_direct(wl.reps, wl.partials, wbig, wl.gain, wl.eps, H)
        assert np.all(np.isfinite(host(h)))
        check(host(h), ref, "bf16", "peaked mhar_fwd")
        got = ar.attnres_bwd(reps, dev(wl.partials, True), w, dev(wl.dh, True), g, wl.eps, H)
        ref_b = orc.block_bwd(wl.reps, wl.partials, wbig, wl.gain, wl.eps, H, wl.dh)
        check(host(got[0]), ref_b[0], "bf16", "peaked d_reps")
        check(host(got[1]), ref_b[1], "bf16", "peaked d_partials")
    finally:
        ar.attnres_set_kernel_policy(prev)


# (T, d, L, n_dst, gain, kernel[, H])
FULL_BWD_CASES = [
    (300, 2048, 32, 32, "per", "full_bwd_res"),
    (517, 1024, 17, 5, "shared", "full_bwd_res"),
    (403, 1280, 9, 9, "none", "full_bwd_res"),
    (300, 1536, 32, 1, "per", "full_bwd_one"),
    (290, 1792, 1, 1, "per", "full_bwd_res"),
    (261, 2048, 20, 13, "shared", "full_bwd_res"),
    (40, 4096, 32, 32, "per", "full_bwd_fast"),
    (333, 512, 12, 7, "per", "full_bwd_fast"),
    (300, 2048, 16, 16, "per", "full_bwd_res", 8),
    (261, 2048, 20, 13, "shared", "full_bwd_res", 4),
    (517, 1024, 17, 5, "none", "full_bwd_res", 2),
    (403, 1024, 9, 9, "per", "full_bwd_res", 4),
    (290, 1536, 12, 1, "per", "full_bwd_res", 2),
    (7, 2048, 1, 1, "none", "full_bwd_res", 8),
    (19, 2048, 32, 32, "per", "full_bwd_res", 8),
    # 33 .. 64 sources, up to 32 destinations: two source tiles
    (300, 2048, 55, 1, "per", "full_bwd_one"),
    (261, 1024, 33, 32, "shared", "full_bwd_wide"),
    (530, 2048, 64, 32, "per", "full_bwd_wide"),
    (40, 4096, 40, 7, "none", "full_bwd_wide"),
    (7, 1536, 47, 20, "per", "full_bwd_wide"),
    (1, 2048, 55, 1, "none", "full_bwd_one"),
    (77, 4096, 48, 1, "per", "full_bwd_wide"),
    # one destination, one head, up to 32 sources, d <= 4096: the vector kernel (T past its
    # workgroup count gives each several tokens and a ragged tail)
    (2000, 4096, 32, 1, "shared", "full_bwd_one"),
    (1100, 512, 9, 1, "none", "full_bwd_one"),
    (1, 2048, 32, 1, "per", "full_bwd_one"),
    (777, 1024, 17, 1, "per", "full_bwd_one"),
    (1500, 3072, 5, 1, "shared", "full_bwd_one"),
    (600, 2048, 1, 1, "per", "full_bwd_one"),
    (2100, 2048, 16, 1, "shared", "full_bwd_one"),
    (900, 4096, 12, 1, "per", "full_bwd_one"),
    # 33 .. 64 sources: 64 rows of 4 channels per thread (d <= 2048)
    (1200, 1024, 64, 1, "shared", "full_bwd_one"),
    (333, 512, 33, 1, "per", "full_bwd_one"),
    (1030, 2048, 47, 1, "none", "full_bwd_one"),
    # ... with heads of whole waves
    (1000, 4096, 32, 1, "per", "full_bwd_one", 8),
    (600, 2048, 55, 1, "shared", "full_bwd_one", 8),
    (333, 2048, 20, 1, "none", "full_bwd_one", 4),
    (1, 4096, 9, 1, "per", "full_bwd_one", 2),
]


def _gain_arg(wl, gain, n_dst, d):
    if gain == "none":
        return None
    if gain == "shared":
        return (1 + 0.1 * np.random.default_rng(d).standard_normal(d)).astype(np.float32)
    return wl.gain


@pytest.mark.parametrize("L,d,gain,H", [(9, 1024, "shared", 1), (32, 2048, "per", 1), (47, 1024, "shared", 1),
                                          (20, 2048, "shared", 4)])
def test_full_bwd_one_accumulates_parameter_grads(L, d, gain, H):
    """One destination: dw and dgain (shared or per destination) are added to
    the given values, d_src too, each against the oracle."""
    T = 700
    name = ar.attnres_kernel_variant(ar.OP_FULL_BWD, L, 1, T, d, H)
    say(f"full bwd one accumulate T={T} d={d} L={L} gain={gain} H={H}: {name}")
    assert name == "full_bwd_one", name
    wl = synth.full_workload(T=T, d=d, L=L, std_step=0.2, dtype="bf16", seed=300 + L, gain_variance=0.02, n_dst=1,
                             with_dout=True)
    g = _gain_arg(wl, gain, 1, d)
    ref = orc.full_bwd(wl.src, wl.w, g, wl.eps, H, wl.dh)
    rng = np.random.default_rng(L)
    base = [synth.bf16_round(rng.standard_normal(wl.src.shape).astype(np.float32)),
            rng.standard_normal(wl.w.shape).astype(np.float32), rng.standard_normal(g.shape).astype(np.float32)]
    outs = [dev(base[0], True), dev(base[1]), dev(base[2])]
    ar.attnres_full_bwd(dev(wl.src, True), dev(wl.w), dev(wl.dh, True), dev(g), wl.eps, H, d_src=outs[0],
                        dw=outs[1], dgain=outs[2], accumulate=True)
    check(host(outs[0]), base[0] + ref[0], "bf16", "d_src accumulated")
    check(host(outs[1]), base[1] + ref[1], "f32_from_bf16", "dw accumulated")
    check(host(outs[2]), base[2] + ref[2], "f32_from_bf16", "dgain accumulated")


@pytest.mark.parametrize("case", FULL_BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_full_bwd_variant(case):
    T, d, L, n_dst, gain, kernel = case[:6]
    H = case[6] if len(case) > 6 else 1
    name = ar.attnres_kernel_variant(ar.OP_FULL_BWD, L, n_dst, T, d, H)
    say(f"full bwd T={T} d={d} L={L} n_dst={n_dst} H={H} gain={gain}: {name}")
    assert name == kernel, name
    wl = synth.full_workload(T=T, d=d, L=L, std_step=0.2, dtype="bf16", seed=90 + L + n_dst + H, gain_variance=0.02,
                             n_dst=n_dst, with_dout=True)
    g = _gain_arg(wl, gain, n_dst, d)
    ref = orc.full_bwd(wl.src, wl.w, g, wl.eps, H, wl.dh)
    src, w, dout = dev(wl.src, True), dev(wl.w), dev(wl.dh, True)
    gd = dev(g) if g is not None else None
    got = ar.attnres_full_bwd(src, w, dout, gd, wl.eps, H)
    check(host(got[0]), ref[0], "bf16", "d_src")
    check(host(got[1]), ref[1], "f32_from_bf16", "dw")
    if g is not None:
        check(host(got[2]), ref[2], "f32_from_bf16", "dgain")
    # accumulate: the gradient is added in fp32 to the given d_src before one rounding
    rng = np.random.default_rng(T)
    base = synth.bf16_round(rng.standard_normal(wl.src.shape).astype(np.float32))
    d_src = dev(base, True)
    ar.attnres_full_bwd(src, w, dout, gd, wl.eps, H, d_src=d_src, accumulate=True)
    check(host(d_src), base + ref[0], "bf16", "d_src accumulated")
    # the general kernel on the same inputs (where its tables hold the shape):
    # the same d_src within the bar
    if n_dst * H * L <= 1024:
        prev = ar.attnres_set_kernel_policy(1)
        try:
            gen = ar.attnres_full_bwd(src, w, dout, gd, wl.eps, H)
        finally:
            ar.attnres_set_kernel_policy(prev)
        check(host(gen[0]), ref[0], "bf16", "d_src (general kernel)")


# (T, d, L, n_dst, H, gain)
FULL_FWD_HEAD_CASES = [
    (700, 2048, 32, 32, 8, "per"),
    (19, 2048, 32, 32, 8, "per"),
    (600, 2048, 32, 32, 4, "shared"),
    (530, 2048, 32, 32, 2, "none"),
    (300, 1024, 17, 5, 8, "per"),
    (290, 1536, 9, 9, 4, "per"),
    (1, 512, 32, 1, 8, "shared"),
    (333, 512, 20, 13, 2, "per"),
    (7, 1024, 1, 1, 4, "none"),
    # one destination with heads of whole 512-channel waves: the vector kernel
    (1500, 4096, 32, 1, 8, "per"),
    (700, 2048, 55, 1, 4, "shared"),
    (300, 2048, 20, 1, 2, "none"),
    (1, 4096, 64, 1, 8, "per"),
    (900, 2048, 55, 1, 8, "per"),
    (350, 1024, 32, 1, 4, "shared"),
]


@pytest.mark.parametrize("T,d,L,n_dst,H,gain", FULL_FWD_HEAD_CASES)
def test_full_fwd_heads(T, d, L, n_dst, H, gain):
    name = ar.attnres_kernel_variant(ar.OP_FULL_FWD, L, n_dst, T, d, H)
    say(f"full fwd heads T={T} d={d} L={L} n_dst={n_dst} H={H} gain={gain}: {name}")
    one = n_dst == 1 and ((d // H) % 512 == 0 or ((d // H) % 256 == 0 and d <= 2048))
    assert name == ("full_one" if one else "full_fast"), name
    wl = synth.full_workload(T=T, d=d, L=L, std_step=0.2, dtype="bf16", seed=120 + H + L, gain_variance=0.02,
                             n_dst=n_dst)
    g = _gain_arg(wl, gain, n_dst, d)
    ref = orc.full_fwd(wl.src, wl.w, g, wl.eps, H)
    src, w = dev(wl.src, True), dev(wl.w)
    gd = dev(g) if g is not None else None
    out = ar.attnres_full_fwd(src, w, gd, wl.eps, H)
    check(host(out), ref, "bf16", "out")
    prev = ar.attnres_set_kernel_policy(1)
    try:
        gen = ar.attnres_full_fwd(src, w, gd, wl.eps, H)
    finally:
        ar.attnres_set_kernel_policy(prev)
    check(host(gen), ref, "bf16", "out (general kernel)")


# Full forward over 33 .. 64 sources: (T, d, L, n_dst, gain).  Two source
# tiles; n_dst > 32 takes two destination tiles.  T above the 512 resident
# workgroups gives each several tokens and a ragged tail.  One destination with
# d <= 4096 runs the vector kernel that reads each row once.
FULL_WIDE_CASES = [
    (530, 2048, 55, 54, "per"),
    (1100, 1024, 33, 33, "shared"),
    (600, 2048, 55, 1, "per"),
    (300, 512, 64, 64, "none"),
    (300, 4096, 40, 32, "per"),
    (1, 2048, 55, 1, "none"),
    (37, 1536, 47, 20, "shared"),
    (513, 2560, 64, 1, "per"),
    (2000, 4096, 64, 1, "per"),
    (777, 512, 33, 1, "shared"),
    (1025, 1024, 48, 1, "none"),
    (64, 8192, 40, 1, "per"),
    # up to 16 sources: the 16-row tile
    (2500, 2048, 16, 1, "per"),
    (333, 4096, 3, 1, "shared"),
    (1, 512, 1, 1, "none"),
]


@pytest.mark.parametrize("T,d,L,n_dst,gain", FULL_WIDE_CASES)
def test_full_fwd_wide(T, d, L, n_dst, gain):
    name = ar.attnres_kernel_variant(ar.OP_FULL_FWD, L, n_dst, T, d, 1)
    say(f"full fwd wide T={T} d={d} L={L} n_dst={n_dst} gain={gain}: {name}")
    assert name == ("full_one" if n_dst == 1 and d <= 4096 else "full_wide"), name
    wl = synth.full_workload(T=T, d=d, L=L, std_step=0.2, dtype="bf16", seed=140 + L + n_dst, gain_variance=0.02,
                             n_dst=n_dst)
    g = _gain_arg(wl, gain, n_dst, d)
    ref = orc.full_fwd(wl.src, wl.w, g, wl.eps, 1)
    src, w = dev(wl.src, True), dev(wl.w)
    gd = dev(g) if g is not None else None
    out = ar.attnres_full_fwd(src, w, gd, wl.eps, 1)
    check(host(out), ref, "bf16", "out")
    prev = ar.attnres_set_kernel_policy(1)
    try:
        gen = ar.attnres_full_fwd(src, w, gd, wl.eps, 1)
    finally:
        ar.attnres_set_kernel_policy(prev)
    check(host(gen), ref, "bf16", "out (general kernel)")
