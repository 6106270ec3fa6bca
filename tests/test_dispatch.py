"""Which kernel each call runs, from its sizes alone (attnres_kernel_variant is
host logic; no GPU needed).  These tables are the contract the GPU parity
matrix (tests/test_gpu_variants.py) covers: every variant named here has a
parity case there, so the dispatcher cannot drift to an untested kernel."""

import re

import pytest

binding = pytest.importorskip("depth_wise_attention_amd.binding")

F32, BF16, F16 = binding.F32, binding.BF16, binding.F16


def variant(op, N, S, T, d, H=1, dtype=BF16, o_dtype=F16):
    return binding.attnres_kernel_variant(op, N, S, T, d, H, dtype, o_dtype)


def phase1(N, S, d, H=1, **kw):
    return variant(binding.OP_PHASE1, N, S, 100, d, H, **kw)


def parse(name):
    m = re.match(r"(\w+)<(.*)> B=(\d+)", name)
    assert m, name
    fields = dict(kv.split("=") for kv in m.group(2).split(","))
    return m.group(1), {k: int(v) for k, v in fields.items()}, int(m.group(3))


@pytest.mark.parametrize("N", range(1, 13))
@pytest.mark.parametrize("S", range(1, 9))
def test_phase1_every_block_depth_at_d4096(N, S):
    """Block n of a model reads n reps: every N up to 12 and S up to 8 has a fast kernel
    at d = 4096 -- two 8-channel chunks per thread where N <= 8 and S <= 4, else one."""
    kind, f, B = parse(phase1(N, S, 4096))
    assert kind == "phase1_fast" and f["N"] == N and f["S"] == S and f["MH"] == 0
    assert (f["CH"], B) == ((2, 256) if N <= 8 and S <= 4 else (1, 512))


@pytest.mark.parametrize("d,ch,B", [(512, 1, 64), (1024, 2, 64), (1536, 1, 192), (2048, 2, 128), (3072, 2, 192),
                                    (4096, 2, 256), (8192, 2, 512)])
def test_phase1_widths(d, ch, B):
    kind, f, b = parse(phase1(8, 4, d))
    assert kind == "phase1_fast" and f["CH"] == ch and b == B


@pytest.mark.parametrize("d", [1024, 2048, 4096, 8192])
def test_phase1_heads_of_whole_512_segments(d):
    for H in (1, 2, 4, 8, 16):
        name = phase1(8, 4, d, H)
        if (d // H) % 512 == 0:
            kind, f, _ = parse(name)
            assert kind == "phase1_fast" and f["MH"] == int(H > 1), (d, H)
        else:
            assert name == "phase1_generic", (d, H)


def test_phase1_general_kernel_cases():
    assert phase1(8, 5, 8192) == "phase1_generic"       # one chunk per thread would need 1024 threads
    assert phase1(9, 4, 8192) == "phase1_generic"
    assert phase1(13, 4, 4096) == "phase1_generic"      # beyond the built rep counts
    assert phase1(8, 9, 4096) == "phase1_generic"
    assert phase1(8, 4, 4096, dtype=F32, o_dtype=F32) == "phase1_generic"
    assert phase1(8, 4, 1000) == "phase1_generic"       # not a multiple of 512
    assert parse(phase1(8, 4, 4096, o_dtype=F32))[0] == "phase1_fast"  # fp32 state
    assert parse(phase1(9, 4, 4096, H=8))[1]["CH"] == 1  # heads with more than 8 reps: one chunk


@pytest.mark.parametrize("N", range(1, 13))
@pytest.mark.parametrize("S", range(1, 9))
def test_bwd_every_block_depth(N, S):
    """Every N up to 12 and S up to 8; more than 4 destinations run as two chunks,
    the first the larger (S0 destinations)."""
    kind, f, B = parse(variant(binding.OP_BWD, N, S, 100, 4096))
    assert kind == "bwd_fast" and f["N"] == N and f["S"] == S and f["HH"] == 1 and B == 512
    assert f["S0"] == (S if S <= 4 else (S + 1) // 2)


def test_bwd_widths_heads_and_limits():
    for d in (512, 1024, 1536, 2048, 4096):
        for H in (1, 2, 4, 8):
            name = variant(binding.OP_BWD, 8, 4, 100, d, H)
            if (d // 512) % H == 0:
                kind, f, B = parse(name)
                assert kind == "bwd_fast" and f["HH"] == H and B == d // 8, (d, H)
            else:
                assert name == "bwd_generic", (d, H)
    assert variant(binding.OP_BWD, 8, 9, 100, 4096) == "bwd_generic"
    for d in (1024, 2048, 4096):
        for S in (5, 6, 8):
            kind, f, B = parse(variant(binding.OP_BWD, 9, S, 100, d, 2 if d > 1024 else 1))
            assert kind == "bwd_fast" and f["S0"] == (S + 1) // 2 and B == d // 8, (d, S)
    assert variant(binding.OP_BWD, 8, 4, 100, 8192) == "bwd_generic"
    assert variant(binding.OP_BWD, 8, 4, 100, 4096, dtype=F32) == "bwd_generic"


def test_phase2_full_and_policy():
    assert variant(binding.OP_PHASE2, 8, 4, 100, 4096) == "phase2_fast<CPL=8,MH=0>"
    assert variant(binding.OP_PHASE2, 8, 4, 100, 2048, H=4) == "phase2_fast<CPL=4,MH=1>"
    assert variant(binding.OP_PHASE2, 8, 4, 100, 1024) == "phase2_generic"
    assert variant(binding.OP_FULL_FWD, 32, 32, 100, 2048) == "full_fast"
    # 33 .. 64 sources: the two-tile kernel (one head, bf16, d a multiple of 512)
    for L, n_dst, d in ((33, 33, 2048), (55, 54, 2048), (64, 64, 512), (40, 32, 4096), (47, 20, 1536),
                        (40, 1, 8192), (33, 2, 2048)):
        assert variant(binding.OP_FULL_FWD, L, n_dst, 100, d) == "full_wide", (L, n_dst, d)
    # one destination, one head, d <= 4096: the vector kernel that reads each row once
    for L, d in ((55, 2048), (64, 2560), (33, 512), (64, 4096), (32, 2048), (9, 4096), (1, 512), (17, 1536)):
        assert variant(binding.OP_FULL_FWD, L, 1, 100, d) == "full_one", (L, d)
    assert variant(binding.OP_FULL_FWD, 32, 1, 100, 8192) == "full_fast"
    # ... and with heads of whole 512-channel waves (d / H a multiple of 512)
    for L, d, H in ((32, 2048, 2), (32, 4096, 8), (55, 4096, 4), (9, 1024, 2)):
        assert variant(binding.OP_FULL_FWD, L, 1, 100, d, H=H) == "full_one", (L, d, H)
    # ... or of whole 256-channel waves (4 channels per thread) with d <= 2048
    for L, d, H in ((32, 2048, 8), (55, 2048, 8), (64, 1024, 4), (1, 512, 2)):
        assert variant(binding.OP_FULL_FWD, L, 1, 100, d, H=H) == "full_one", (L, d, H)
    assert variant(binding.OP_FULL_FWD, 32, 1, 100, 1024, H=8) == "full_fast"
    assert variant(binding.OP_FULL_FWD, 55, 1, 100, 1024, H=8) == "full_generic"
    assert variant(binding.OP_FULL_FWD, 55, 1, 100, 4096, H=16) == "full_generic"
    assert variant(binding.OP_FULL_FWD, 32, 1, 100, 2048, dtype=F32) == "full_generic"
    assert variant(binding.OP_FULL_FWD, 55, 54, 100, 2048, H=8) == "full_generic"
    assert variant(binding.OP_FULL_FWD, 55, 54, 100, 768) == "full_generic"
    # heads on the matrix cores: whole waves of the resident kernel (d <= 2048)
    for H in (2, 4, 8):
        for d in (512, 1024, 1536, 2048):
            assert variant(binding.OP_FULL_FWD, 32, 32, 100, d, H=H) == "full_fast"
    assert variant(binding.OP_FULL_FWD, 32, 32, 100, 2048, H=16) == "full_generic"
    assert variant(binding.OP_FULL_FWD, 32, 32, 100, 4096, H=8) == "full_generic"
    assert variant(binding.OP_FULL_FWD, 32, 32, 100, 2048, H=3) == "full_generic"
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 2048) == "full_bwd_res"
    for d in (1024, 1280, 1536, 1792):
        assert variant(binding.OP_FULL_BWD, 17, 5, 100, d) == "full_bwd_res"
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 4096) == "full_bwd_fast"
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 512) == "full_bwd_fast"
    # 33 .. 64 sources and up to 32 destinations: the two-tile backward (one head, d a multiple of 512)
    for L, n_dst, d in ((33, 32, 2048), (55, 1, 4096), (64, 32, 512), (40, 7, 4096), (47, 20, 1536), (55, 2, 2048)):
        assert variant(binding.OP_FULL_BWD, L, n_dst, 100, d) == "full_bwd_wide", (L, n_dst, d)
    # one destination, one head: the vector kernel that reads each row once (up to 32 sources with
    # d <= 4096, 33 .. 64 with d <= 2048)
    for L, d in ((32, 2048), (1, 512), (9, 4096), (17, 1536), (32, 1024), (55, 2048), (64, 512), (33, 1536)):
        assert variant(binding.OP_FULL_BWD, L, 1, 100, d) == "full_bwd_one", (L, d)
    assert variant(binding.OP_FULL_BWD, 32, 1, 100, 8192) == "full_bwd_fast"
    # ... and with heads of whole waves (512 channels at up to 32 sources, 256 above)
    for L, d, H in ((32, 2048, 2), (32, 4096, 8), (55, 2048, 8), (9, 1024, 2), (64, 512, 2)):
        assert variant(binding.OP_FULL_BWD, L, 1, 100, d, H=H) == "full_bwd_one", (L, d, H)
    assert variant(binding.OP_FULL_BWD, 32, 1, 100, 2048, H=8) == "full_bwd_res"
    assert variant(binding.OP_FULL_BWD, 55, 1, 100, 4096, H=2) == "full_bwd_generic"
    assert variant(binding.OP_FULL_BWD, 32, 2, 100, 2048) == "full_bwd_res"
    assert variant(binding.OP_FULL_BWD, 32, 1, 100, 2048, dtype=F32) == "full_bwd_generic"
    assert variant(binding.OP_FULL_BWD, 33, 33, 100, 2048) == "full_bwd_generic"
    assert variant(binding.OP_FULL_BWD, 55, 2, 100, 2048, H=2) == "full_bwd_generic"
    assert variant(binding.OP_FULL_BWD, 55, 1, 100, 768) == "full_bwd_generic"
    # heads on the resident kernel: runs of whole 256-channel waves
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 2048, H=8) == "full_bwd_res"
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 1024, H=4) == "full_bwd_res"
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 1536, H=2) == "full_bwd_res"
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 1024, H=8) == "full_bwd_generic"
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 1536, H=4) == "full_bwd_generic"
    assert variant(binding.OP_FULL_BWD, 32, 32, 100, 4096, H=8) == "full_bwd_generic"
    prev = binding.attnres_set_kernel_policy(1)
    try:
        assert phase1(8, 4, 4096) == "phase1_generic"
        assert variant(binding.OP_BWD, 8, 4, 100, 4096) == "bwd_generic"
        assert variant(binding.OP_PHASE2, 8, 4, 100, 4096) == "phase2_generic"
    finally:
        binding.attnres_set_kernel_policy(prev)


def test_variant_query_rejects_bad_requests():
    with pytest.raises(binding.AttnResError):
        binding.attnres_kernel_variant(9, 8, 4, 100, 4096, 1, BF16, F16)
    L = binding.lib()
    assert L.attnres_kernel_variant(0, 8, 4, 100, 4096, 1, BF16, F16, None, 16) == -1
