"""The C ABI without a GPU: exports, versions, workspace sizes and argument
validation.  Every call here fails validation, which the library performs
before its first HIP call, so nothing is ever enqueued."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")

binding = pytest.importorskip("depth_wise_attention_amd.binding")

OK, EINVAL, EUNSUP, EHIP, EWS = 0, -1, -2, -3, -4
F32, BF16, F16 = 0, 1, 2
FAKE = 0x7F0000000000  # never dereferenced: every call below is rejected first


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


fake_ptrs = pytest.mark.skipif(_gpu_visible(), reason="calls with fake pointers run only on hosts without a GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("attnres_full_fwd", "attnres_block_phase1", "attnres_block_phase2_merge",
                 "attnres_block_phase2_merge_update", "mhar_fwd", "mhar_fwd_chunked", "attnres_msar_fwd",
                 "attnres_msar_fwd_workspace_size", "attnres_block_msar_phase1", "attnres_block_msar_phase2",
                 "attnres_block_msar_phase1_workspace_size", "attnres_block_msar_phase2_workspace_size",
                 "attnres_bwd", "attnres_full_bwd", "attnres_full_fwd_workspace_size", "mhar_fwd_workspace_size",
                 "attnres_bwd_workspace_size", "attnres_full_bwd_workspace_size",
                 "attnres_last_error", "attnres_version", "attnres_set_kernel_policy"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_policy():
    assert binding.attnres_version() >> 16 == 2
    assert binding.attnres_version() & 0xFFFF >= 6
    prev = binding.attnres_set_kernel_policy(1)
    assert binding.attnres_set_kernel_policy(prev) == 1
    with pytest.raises(binding.AttnResError):
        binding.attnres_set_kernel_policy(7)


def test_workspace_sizes():
    N, S, T, d, H = 8, 4, 16384, 4096, 1
    lse = S * H * T * 4
    up = lambda x: (x + 255) // 256 * 256
    # The Phase-1 state lives in h (in place): the workspace holds lse and the scales only.
    assert binding.mhar_fwd_workspace_size(N, S, T, d, H) == up(lse) + up(4 * T)
    assert binding.mhar_fwd_workspace_size(N, 4, T, d, 8) == up(4 * 8 * T * 4) + up(4 * T)
    assert binding.mhar_fwd_workspace_size(N, 1, 5, 3, 1) == up(4 * 5) + up(4 * 5)
    assert binding.mhar_fwd_workspace_size(N, 0, T, d, H) == 0
    assert binding.attnres_bwd_workspace_size(N, S, 8192, d, H) == 1024 * S * d * 4
    assert binding.attnres_bwd_workspace_size(N, S, 5, d, H) == 8 * S * d * 4
    assert binding.attnres_bwd_workspace_size(N, S, 0, d, H) == 0
    # more than 4 destinations: two chunks, the first chunk's rep gradients kept in fp32
    assert binding.attnres_bwd_workspace_size(9, 6, 8192, d, H) == 1024 * 6 * d * 4 + 9 * 8192 * d * 4
    assert binding.attnres_bwd_workspace_size(2, 5, 5, 1024, H) == 8 * 5 * 1024 * 4 + 2 * 5 * 1024 * 4


def _rc_full(**kw):
    a = dict(src=FAKE, n_src=4, T=8, d=16, w=FAKE + (1 << 30), n_dst=4, gain=None, gain_ld=0, eps=1e-6,
             H=1, dtype=BF16, out=FAKE + (2 << 30), ws=FAKE + (5 << 30), ws_bytes=1 << 20, stream=None)
    a.update(kw)
    L = binding.lib()
    return L.attnres_full_fwd(a["src"], a["n_src"], a["T"], a["d"], a["w"], a["n_dst"], a["gain"],
                              a["gain_ld"], a["eps"], a["H"], a["dtype"], a["out"], a["ws"], a["ws_bytes"],
                              a["stream"])


def test_full_workspace_size():
    # bf16, at most 32 sources, one head (any d) or H = 2, 4, 8 heads with d = 512 .. 2048 in steps
    # of 512: q = w * gain as two bf16 parts, [2, 32, d].
    assert binding.attnres_full_fwd_workspace_size(32, 32, 2048, 1, BF16) == 2 * 32 * 2048 * 2
    assert binding.attnres_full_fwd_workspace_size(8, 1, 4096, 1, BF16) == 2 * 32 * 4096 * 2
    for H in (2, 4, 8):
        assert binding.attnres_full_fwd_workspace_size(8, 8, 2048, H, BF16) == 2 * 32 * 2048 * 2
        assert binding.attnres_full_fwd_workspace_size(32, 1, 512, H, BF16) == 2 * 32 * 512 * 2
    # 33 .. 64 sources, one head, d a multiple of 512: one [2, 32, d] block per 32 destinations.
    assert binding.attnres_full_fwd_workspace_size(33, 1, 2048, 1, BF16) == 2 * 32 * 2048 * 2
    assert binding.attnres_full_fwd_workspace_size(55, 32, 4096, 1, BF16) == 2 * 32 * 4096 * 2
    assert binding.attnres_full_fwd_workspace_size(55, 54, 2048, 1, BF16) == 2 * 64 * 2048 * 2
    assert binding.attnres_full_fwd_workspace_size(64, 33, 512, 1, BF16) == 2 * 64 * 512 * 2
    for args in [(32, 32, 2048, 1, F32), (33, 1, 2048, 2, BF16), (33, 1, 768, 1, BF16), (65, 1, 2048, 1, BF16),
                 (40, 40, 2048, 1, F32), (8, 8, 2048, 16, BF16), (8, 8, 4096, 8, BF16),
                 (8, 8, 2048, 3, BF16), (4, 5, 64, 1, BF16), (0, 0, 64, 1, BF16), (4, 4, 0, 1, BF16)]:
        assert binding.attnres_full_fwd_workspace_size(*args) == 0, args


@fake_ptrs
def test_full_workspace_checks():
    assert _rc_full(ws=None) == EWS
    assert "workspace" in binding.attnres_last_error()
    assert _rc_full(ws_bytes=2 * 32 * 16 * 2 - 1) == EWS
    # The workspace is an output: it may not overlap the sources (checked before any launch).
    assert _rc_full(ws=FAKE + 64) == EINVAL
    assert "overlaps" in binding.attnres_last_error()
    # fp32 needs none: a NULL workspace passes the workspace check (aliased output rejects the call).
    assert _rc_full(dtype=F32, ws=None, out=FAKE + 16) == EINVAL
    assert "overlaps" in binding.attnres_last_error()


@fake_ptrs
def test_full_rejects_bad_scalars():
    cases = [dict(dtype=7), dict(T=-1), dict(d=0), dict(H=0), dict(H=3), dict(eps=-1.0),
             dict(eps=float("nan")), dict(eps=float("inf")), dict(n_src=0), dict(n_src=65),
             dict(n_dst=0), dict(n_dst=5), dict(gain=FAKE + (3 << 30), gain_ld=7)]
    for c in cases:
        assert _rc_full(**c) == EINVAL, c
        assert binding.attnres_last_error() != ""


@fake_ptrs
def test_full_rejects_null_pointers():
    assert _rc_full(src=None) == EINVAL
    assert "src" in binding.attnres_last_error()
    assert _rc_full(w=None) == EINVAL
    assert _rc_full(out=None) == EINVAL


@fake_ptrs
def test_full_rejects_aliasing():
    assert _rc_full(out=FAKE + 16) == EINVAL
    assert "overlaps" in binding.attnres_last_error()


@fake_ptrs
def test_empty_token_count_is_a_no_op():
    # T == 0 enqueues nothing, even with NULL tensors and no stream.
    assert _rc_full(T=0, src=None, out=None, w=None) == OK
    assert binding.attnres_last_error() == ""
    L = binding.lib()
    assert L.attnres_block_phase1(None, 8, 0, 64, None, 4, None, 0, 1e-6, 1, BF16, None, None, F32, None,
                                  None, None) == OK
    assert L.attnres_block_phase2_merge(None, F32, None, None, None, 0, 64, None, None, 1e-6, 1, BF16, None,
                                        None) == OK
    assert L.mhar_fwd(None, 8, None, 4, 0, 64, None, None, 0, 1e-6, 1, BF16, None, None, 0, None) == OK


def _rc_phase1(**kw):
    a = dict(reps=FAKE, N=8, T=8, d=64, w=FAKE + (1 << 30), S=4, gain=None, gain_ld=0, eps=1e-6, H=1,
             dtype=BF16, h=FAKE + (4 << 30), o=FAKE + (2 << 30), o_dtype=F32, lse=FAKE + (3 << 30),
             scale=None)
    a.update(kw)
    return binding.lib().attnres_block_phase1(a["reps"], a["N"], a["T"], a["d"], a["w"], a["S"], a["gain"],
                                              a["gain_ld"], a["eps"], a["H"], a["dtype"], a["h"], a["o"],
                                              a["o_dtype"], a["lse"], a["scale"], None)


@fake_ptrs
def test_phase1_rejects_bad_arguments():
    for c in [dict(N=0), dict(N=64), dict(S=0), dict(o_dtype=5), dict(dtype=F32, o_dtype=BF16),
              dict(lse=None), dict(o=None), dict(h=None), dict(reps=None), dict(H=5), dict(d=63, H=2),
              dict(dtype=F32, o_dtype=F16, scale=FAKE + (5 << 30)), dict(o_dtype=F16, scale=None)]:
        assert _rc_phase1(**c) == EINVAL, c


@fake_ptrs
def test_bf16_state_is_refused():
    """A bf16 Phase-1 state (8 bits, rounded again by the merge) misses the bf16
    bar at full size, so every call that would take one refuses it."""
    assert _rc_phase1(o_dtype=BF16) == EUNSUP
    assert "bf16 Phase-1 state" in binding.attnres_last_error()
    assert _rc_phase2(o_dtype=BF16) == EUNSUP
    assert _rc_update(o_dtype=BF16) == EUNSUP


@fake_ptrs
def test_phase1_rejects_overlapping_outputs():
    assert _rc_phase1(lse=FAKE + (2 << 30) + 64) == EINVAL
    assert _rc_phase1(o=FAKE + 8) == EINVAL
    assert _rc_phase1(h=FAKE + (2 << 30) + 16) == EINVAL
    assert _rc_phase1(o_dtype=F16, scale=FAKE + (3 << 30) + 32) == EINVAL  # scale over lse


def _rc_phase2(**kw):
    a = dict(o=FAKE, o_dtype=F32, scale=None, lse=FAKE + (1 << 30), partial=FAKE + (2 << 30), T=8, d=64,
             w=FAKE + (3 << 30), gain=None, eps=1e-6, H=1, dtype=BF16, h=FAKE + (4 << 30))
    a.update(kw)
    return binding.lib().attnres_block_phase2_merge(a["o"], a["o_dtype"], a["scale"], a["lse"], a["partial"],
                                                    a["T"], a["d"], a["w"], a["gain"], a["eps"], a["H"],
                                                    a["dtype"], a["h"], None)


@fake_ptrs
def test_phase2_rejects_bad_arguments():
    for c in [dict(o_dtype=3), dict(partial=None), dict(lse=None), dict(w=None), dict(h=None),
              dict(H=7), dict(o_dtype=F16, scale=None), dict(o_dtype=F16, dtype=F32, scale=FAKE + (5 << 30))]:
        assert _rc_phase2(**c) == EINVAL, c


@fake_ptrs
def test_phase2_in_place_needs_matching_dtype():
    assert _rc_phase2(h=FAKE) == EINVAL          # o is fp32, h bf16: cannot share storage
    assert "in-place" in binding.attnres_last_error()
    assert _rc_update(o_dtype=F32, h=FAKE) == EINVAL
    assert _rc_phase2(h=FAKE + (2 << 30)) == EINVAL  # h over the partial


def _rc_update(**kw):
    G = 1 << 30
    a = dict(o=FAKE, o_dtype=F32, scale=None, lse=FAKE + G, prev=FAKE + 2 * G, f=FAKE + 3 * G, T=8, d=64,
             w=FAKE + 4 * G, gain=None, eps=1e-6, H=1, dtype=BF16, pout=FAKE + 5 * G, h=FAKE + 6 * G,
             norm_eps=1e-6, rms=FAKE + 7 * G)
    a.update(kw)
    return binding.lib().attnres_block_phase2_merge_update(
        a["o"], a["o_dtype"], a["scale"], a["lse"], a["prev"], a["f"], a["T"], a["d"], a["w"], a["gain"],
        a["eps"], a["H"], a["dtype"], a["pout"], a["h"], a["norm_eps"], a["rms"], None)


@fake_ptrs
def test_phase2_update_rejects_bad_arguments():
    G = 1 << 30
    for c in [dict(f=None), dict(pout=None), dict(h=None), dict(o=None), dict(lse=None), dict(w=None),
              dict(o_dtype=3), dict(H=7), dict(norm_eps=-1.0), dict(norm_eps=float("nan")),
              dict(o_dtype=F16, scale=None)]:
        assert _rc_update(**c) == EINVAL, c
    # Overlaps: the updated partial over f, h over the updated partial, the
    # statistic over h, and h over o with different dtypes.
    for c in [dict(pout=FAKE + 3 * G), dict(h=FAKE + 5 * G + 64), dict(rms=FAKE + 6 * G),
              dict(o_dtype=F32, h=FAKE), dict(prev=FAKE + 5 * G + 2), dict(f=FAKE + 6 * G)]:
        assert _rc_update(**c) == EINVAL, c
    assert _rc_update(T=0, o=None, f=None, pout=None, h=None) == OK
    assert _rc_update(T=-1) == EINVAL


def _rc_mhar(**kw):
    a = dict(reps=FAKE, N=8, partials=FAKE + (1 << 30), S=4, T=8, d=64, w=FAKE + (2 << 30), gain=None,
             gain_ld=0, eps=1e-6, H=1, dtype=BF16, h=FAKE + (3 << 30), ws=FAKE + (4 << 30), ws_bytes=1 << 20)
    a.update(kw)
    return binding.lib().mhar_fwd(a["reps"], a["N"], a["partials"], a["S"], a["T"], a["d"], a["w"],
                                  a["gain"], a["gain_ld"], a["eps"], a["H"], a["dtype"], a["h"], a["ws"],
                                  a["ws_bytes"], None)


@fake_ptrs
def test_mhar_rejects_bad_arguments():
    assert _rc_mhar(partials=None) == EINVAL
    assert _rc_mhar(N=0) == EINVAL
    assert _rc_mhar(ws=None) == EWS
    assert _rc_mhar(ws_bytes=16) == EWS
    assert "workspace" in binding.attnres_last_error()


def _rc_chunked(**kw):
    a = dict(reps=FAKE, N=8, partials=FAKE + (1 << 30), S=4, T=1000, d=64, w=FAKE + (2 << 30), gain=None,
             gain_ld=0, eps=1e-6, H=1, dtype=BF16, h=FAKE + (3 << 30), chunk=100, ws=FAKE + (4 << 30),
             ws_bytes=1 << 20)
    a.update(kw)
    return binding.lib().mhar_fwd_chunked(a["reps"], a["N"], a["partials"], a["S"], a["T"], a["d"], a["w"],
                                          a["gain"], a["gain_ld"], a["eps"], a["H"], a["dtype"], a["h"],
                                          a["chunk"], a["ws"], a["ws_bytes"], None)


@fake_ptrs
def test_mhar_chunked_rejects_bad_arguments():
    for c in [dict(chunk=0), dict(chunk=-5), dict(N=0), dict(S=0), dict(reps=None), dict(h=None),
              dict(partials=None), dict(H=3), dict(ws=FAKE + (3 << 30))]:
        assert _rc_chunked(**c) == EINVAL, c
    # the workspace is sized by the chunk: one byte short of a 100-token chunk fails
    need = binding.mhar_fwd_workspace_size(8, 4, 100, 64, 1)
    assert _rc_chunked(ws_bytes=need - 1) == EWS
    assert binding.mhar_fwd_workspace_size(8, 4, 1000, 64, 1) > 5 * need
    assert _rc_chunked(T=0, reps=None, h=None) == OK


@fake_ptrs
def test_noalloc_refuses_requests_beyond_its_scratch():
    """mhar_fwd_noalloc takes no workspace; a request needing more scratch than
    the static array is refused before any HIP call."""
    L = binding.lib()
    G = 1 << 30
    call = lambda T, H: L.mhar_fwd_noalloc(FAKE, 1, FAKE + G, 4, T, 512, FAKE + 2 * G, None, 0, 1e-6, H, BF16,
                                           FAKE + 3 * G, None)
    assert call(70000, 8) == EUNSUP
    assert "scratch" in binding.attnres_last_error()
    assert L.mhar_fwd_noalloc(None, 1, None, 4, 0, 512, None, None, 0, 1e-6, 1, BF16, None, None) == OK
    assert call(10, 3) == EINVAL  # 512 is not divisible by 3


@fake_ptrs
def test_mhar_rejects_workspace_over_inputs():
    assert _rc_mhar(ws=FAKE + 64) == EINVAL


def _rc_bwd(**kw):
    a = dict(reps=FAKE, N=8, partials=FAKE + (1 << 30), S=4, T=8, d=64, w=FAKE + (2 << 30), gain=None,
             gain_ld=0, eps=1e-6, H=1, dtype=BF16, dh=FAKE + (3 << 30), d_reps=FAKE + (4 << 30),
             d_partials=FAKE + (5 << 30), dw=FAKE + (6 << 30), dgain=None, accumulate=0,
             ws=FAKE + (7 << 30), ws_bytes=1 << 24)
    a.update(kw)
    return binding.lib().attnres_bwd(a["reps"], a["N"], a["partials"], a["S"], a["T"], a["d"], a["w"],
                                     a["gain"], a["gain_ld"], a["eps"], a["H"], a["dtype"], a["dh"],
                                     a["d_reps"], a["d_partials"], a["dw"], a["dgain"], a["accumulate"],
                                     a["ws"], a["ws_bytes"], None)


@fake_ptrs
def test_bwd_rejects_bad_arguments():
    for c in [dict(N=0), dict(S=0), dict(accumulate=2), dict(dh=None), dict(d_reps=None),
              dict(d_partials=None), dict(dw=None), dict(gain=FAKE + (8 << 30), dgain=None)]:
        assert _rc_bwd(**c) == EINVAL, c
    assert _rc_bwd(N=60, S=6) == EUNSUP
    assert _rc_bwd(ws=None) == EWS
    assert _rc_bwd(ws_bytes=100) == EWS
    # more than 4 destinations: the Z slabs alone are too short, the fp32 rep gradients need room too
    slabs = 8 * 6 * 64 * 4
    assert _rc_bwd(S=6, ws_bytes=slabs) == EWS
    assert _rc_bwd(S=6, ws_bytes=slabs + 8 * 8 * 64 * 4 - 4) == EWS
    assert binding.attnres_bwd_workspace_size(8, 6, 8, 64, 1) == slabs + 8 * 8 * 64 * 4


@fake_ptrs
def test_bwd_rejects_aliasing():
    assert _rc_bwd(d_reps=FAKE + 2) == EINVAL
    assert _rc_bwd(dw=FAKE + (6 << 30), ws=FAKE + (6 << 30) + 4) == EINVAL


@fake_ptrs
def test_error_message_is_thread_local():
    import threading
    assert _rc_full(dtype=9) == EINVAL
    seen = {}

    def other():
        seen["msg"] = binding.attnres_last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "dtype" in binding.attnres_last_error()


def test_full_bwd_workspace_size():
    # the larger of the two paths' needs:
    #   general: one [n_dst, d] fp32 slab per wavefront, T rounded up to 4, at most 1024 slabs;
    #   matrix cores: split q and q^T (256 d bytes) + r*c per token (T x 32 x 32 fp32, or
    #                 T x 32 x 64 with more than 32 sources)
    #                 + one [n_dst, d] fp32 slab per token group (min(T, 64) groups)
    general = lambda n_dst, T, d: min((T + 3) // 4 * 4, 1024) * n_dst * d * 4
    fast = lambda n_dst, T, d: 256 * d + T * 4096 + min(T, 64) * n_dst * d * 4
    for n_src, n_dst, T, d in [(32, 32, 4096, 2048), (8, 3, 5, 64), (32, 32, 1, 512)]:
        want = max(general(n_dst, T, d), fast(n_dst, T, d))
        assert binding.attnres_full_bwd_workspace_size(n_src, n_dst, T, d, 1) == want
    assert binding.attnres_full_bwd_workspace_size(32, 32, 4096, 2048, 1) == 1024 * 32 * 2048 * 4
    # heads: r * c per head, T x H x 32 x 32 fp32
    fast_h = lambda n_dst, T, d, H: 256 * d + T * 4096 * H + min(T, 64) * n_dst * d * 4
    assert binding.attnres_full_bwd_workspace_size(8, 8, 1000, 2048, 8) == max(
        general(8, 1000, 2048), fast_h(8, 1000, 2048, 8))
    assert binding.attnres_full_bwd_workspace_size(32, 1, 40, 1024, 4) == max(
        general(1, 40, 1024), fast_h(1, 40, 1024, 4))
    # 33 .. 64 sources: r * c per token is T x 32 x 64 fp32
    fast_w = lambda n_dst, T, d: 256 * d + T * 8192 + min(T, 64) * n_dst * d * 4
    for n_src, n_dst, T, d in [(55, 1, 4096, 2048), (64, 32, 300, 512), (33, 33, 7, 1024)]:
        want = max(general(n_dst, T, d), fast_w(n_dst, T, d))
        assert binding.attnres_full_bwd_workspace_size(n_src, n_dst, T, d, 1) == want, (n_src, n_dst, T, d)
    # one destination, one head, up to 32 sources, d = 512 .. 4096 in steps of 512: the vector kernel
    # keeps one [d] fp32 slab per workgroup, at most min(T, 1024) of them (never more than the
    # general path's slabs)
    one = lambda T, d: min(T, 1024) * d * 4
    for n_src, T, d in [(32, 4096, 4096), (9, 4096, 2048), (32, 5, 512), (1, 1, 1024), (17, 100000, 3072)]:
        want = max(general(1, T, d), fast(1, T, d), one(T, d))
        assert binding.attnres_full_bwd_workspace_size(n_src, 1, T, d, 1) == want, (n_src, T, d)
    assert binding.attnres_full_bwd_workspace_size(8, 3, 0, 64, 1) == 0
    assert binding.attnres_full_bwd_workspace_size(8, 0, 16, 64, 1) == 0


def _rc_full_bwd(**kw):
    a = dict(src=FAKE, n_src=4, T=8, d=16, w=FAKE + (1 << 30), n_dst=4, gain=None, gain_ld=0, eps=1e-6, H=1,
             dtype=BF16, dout=FAKE + (2 << 30), d_src=FAKE + (3 << 30), dw=FAKE + (4 << 30), dgain=None,
             acc=0, ws=FAKE + (5 << 30), ws_bytes=1 << 20)
    a.update(kw)
    return binding.lib().attnres_full_bwd(a["src"], a["n_src"], a["T"], a["d"], a["w"], a["n_dst"], a["gain"],
                                          a["gain_ld"], a["eps"], a["H"], a["dtype"], a["dout"], a["d_src"],
                                          a["dw"], a["dgain"], a["acc"], a["ws"], a["ws_bytes"], None)


@fake_ptrs
def test_full_bwd_rejects_bad_arguments():
    for c in [dict(n_src=0), dict(n_src=65), dict(n_dst=0), dict(n_dst=5), dict(acc=2), dict(dtype=7),
              dict(H=3), dict(eps=-1.0), dict(w=None), dict(dw=None), dict(src=None), dict(dout=None),
              dict(d_src=None), dict(gain=FAKE + (6 << 30), gain_ld=16, dgain=None),
              dict(d_src=FAKE + 64), dict(ws=FAKE + (2 << 30) + 64)]:
        assert _rc_full_bwd(**c) == EINVAL, c
        assert binding.attnres_last_error() != ""
    assert _rc_full_bwd(ws=None) == EWS
    assert _rc_full_bwd(ws_bytes=16) == EWS
    # n_dst * H * n_src beyond the general kernel's 1024-entry tables
    assert _rc_full_bwd(n_src=64, n_dst=17, d=64) == EUNSUP
    assert "1024" in binding.attnres_last_error()


def _rc_msar(**kw):
    G = 1 << 30
    a = dict(src=FAKE, n_src=9, T=100, d=64, w=FAKE + G, conv=FAKE + 2 * G, mix=FAKE + 3 * G, n_dst=1, eps=1e-6,
             dtype=BF16, out=FAKE + 4 * G, ws=None, ws_bytes=0)
    a.update(kw)
    return binding.lib().attnres_msar_fwd(a["src"], a["n_src"], a["T"], a["d"], a["w"], a["conv"], a["mix"],
                                          a["n_dst"], a["eps"], a["dtype"], a["out"], a["ws"], a["ws_bytes"], None)


@fake_ptrs
def test_msar_rejects_bad_arguments():
    G = 1 << 30
    for c in [dict(n_src=0), dict(n_src=65), dict(n_dst=0), dict(n_dst=10), dict(src=None), dict(w=None),
              dict(conv=None), dict(mix=None), dict(out=None), dict(eps=-1.0), dict(dtype=7), dict(d=0),
              dict(T=-1), dict(out=FAKE + 1000), dict(out=FAKE + 2 * G + 8), dict(out=FAKE + 3 * G)]:
        assert _rc_msar(**c) == EINVAL, c
    assert _rc_msar(T=0, src=None, out=None) == OK


def _rc_bm1(**kw):
    G = 1 << 30
    a = dict(reps=FAKE, N=8, T=100, d=512, w=FAKE + G, S=4, conv=FAKE + 2 * G, mix=FAKE + 3 * G, eps=1e-6,
             dtype=BF16, h1=FAKE + 4 * G, o=FAKE + 5 * G, sc=FAKE + 8 * G, lse=FAKE + 6 * G, ws=FAKE + 7 * G,
             ws_bytes=1 << 30)
    a.update(kw)
    return binding.lib().attnres_block_msar_phase1(a["reps"], a["N"], a["T"], a["d"], a["w"], a["S"], a["conv"],
                                                   a["mix"], a["eps"], a["dtype"], a["h1"], a["o"], a["sc"], a["lse"],
                                                   a["ws"], a["ws_bytes"], None)


def _rc_bm2(**kw):
    G = 1 << 30
    a = dict(o=FAKE, sc=FAKE + 8 * G, lse=FAKE + G, p=FAKE + 2 * G, T=100, d=512, w=FAKE + 3 * G,
             conv=FAKE + 4 * G, mix=FAKE + 5 * G, eps=1e-6, dtype=BF16, h=FAKE + 6 * G, ws=FAKE + 7 * G,
             ws_bytes=1 << 30)
    a.update(kw)
    return binding.lib().attnres_block_msar_phase2(a["o"], a["sc"], a["lse"], a["p"], a["T"], a["d"], a["w"],
                                                   a["conv"], a["mix"], a["eps"], a["dtype"], a["h"], a["ws"],
                                                   a["ws_bytes"], None)


@fake_ptrs
def test_block_msar_rejects_bad_arguments():
    G = 1 << 30
    for c, want in [(dict(dtype=F32), EUNSUP), (dict(N=13), EUNSUP), (dict(S=5), EUNSUP), (dict(d=500), EUNSUP),
                    (dict(N=0), EINVAL), (dict(S=0), EINVAL), (dict(reps=None), EINVAL), (dict(h1=None), EINVAL),
                    (dict(o=None), EINVAL), (dict(eps=-1.0), EINVAL), (dict(ws_bytes=16), EWS),
                    (dict(h1=FAKE + 8), EINVAL), (dict(lse=FAKE + 4 * G + 64), EINVAL),
                    (dict(ws=FAKE + 5 * G), EINVAL)]:
        assert _rc_bm1(**c) == want, c
    assert _rc_bm1(S=1, o=None, lse=None, ws_bytes=16) == EWS     # S == 1 needs no state
    assert _rc_bm1(sc=None) == EINVAL
    assert _rc_bm2(sc=None) == EINVAL
    assert _rc_bm1(T=0, reps=None) == OK
    for c, want in [(dict(dtype=F32), EUNSUP), (dict(d=1000), EUNSUP), (dict(o=None), EINVAL),
                    (dict(p=None), EINVAL), (dict(h=None), EINVAL), (dict(ws_bytes=16), EWS),
                    (dict(h=FAKE + 2 * G + 32), EINVAL), (dict(ws=FAKE + G), EINVAL)]:
        assert _rc_bm2(**c) == want, c
    assert _rc_bm2(T=0, o=None) == OK


def test_stream_probe_library_validates_before_launch():
    """The streaming-pattern probe (bench.py --ceilings) lives in its own library;
    invalid arguments are rejected with -1 before any HIP call."""
    from depth_wise_attention_amd import build as b

    if not os.path.exists(b.PROBE_LIB):
        pytest.skip("probe library not built")
    probe = ctypes.CDLL(b.PROBE_LIB)
    fn = probe.attnres_probe_stream
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below is rejected first
    assert fn(fake, 0, fake, 0, 8, 64, fake, 1, 0, None) == -1       # nothing to move
    assert fn(fake, 1, fake, 1, 8, 60, fake, 1, 0, None) == -1       # d not a multiple of 8
    assert fn(fake, 65, fake, 1, 8, 64, fake, 1, 0, None) == -1      # too many rows
    assert fn(None, 1, fake, 1, 8, 64, fake, 1, 0, None) == -1       # missing source
    assert fn(fake, 1, fake, 1, 8, 64, None, 1, 0, None) == -1       # missing sink
    assert fn(ctypes.c_void_p((1 << 20) + 4), 1, fake, 1, 8, 64, fake, 1, 0, None) == -1  # misaligned
    assert fn(fake, 1, fake, 1, 8, 64, fake, 1, 8, None) == -1       # unknown mode
    assert fn(fake, 1, fake, 1, 8, 72, fake, 1, 4, None) == -1       # 32-byte pieces need d % 16 == 0
