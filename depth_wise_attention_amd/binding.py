"""Thin ctypes binding of libattnres.so.

Argument marshalling only: every function here fills in sizes and pointers
from torch tensors (torch supplies device memory and the stream) and calls the
C entry point of the same name.  All arithmetic runs in the library's HIP
kernels; there is no fallback.  A missing library raises at first use.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# ATTNRES_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("ATTNRES_LIB") or os.path.join(_PKG, "libattnres.so")

F32 = 0
BF16 = 1
F16 = 2  # Phase-1 state only: fp16 scaled per token by a power of two

_lib = None


class AttnResError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"attnres error {code}: {message}")
        self.code = code
        self.message = message


def lib() -> ctypes.CDLL:
    """Load libattnres.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with depth_wise_attention_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.attnres_full_fwd_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    L.attnres_full_fwd.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, f32, i32, i32, vp, vp, sz, vp]
    L.attnres_block_phase1.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, f32, i32, i32, vp, vp, i32, vp, vp,
                                       vp]
    L.attnres_block_phase2_merge.argtypes = [vp, i32, vp, vp, vp, i64, i64, vp, vp, f32, i32, i32, vp, vp]
    L.attnres_block_phase2_merge_update.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, vp, vp, f32, i32, i32,
                                                    vp, vp, f32, vp, vp]
    L.mhar_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i32]
    L.mhar_fwd.argtypes = [vp, i64, vp, i64, i64, i64, vp, vp, i64, f32, i32, i32, vp, vp, sz, vp]
    L.mhar_fwd_chunked.argtypes = [vp, i64, vp, i64, i64, i64, vp, vp, i64, f32, i32, i32, vp, i64, vp, sz, vp]
    L.attnres_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i32]
    L.attnres_bwd.argtypes = [vp, i64, vp, i64, i64, i64, vp, vp, i64, f32, i32, i32, vp, vp, vp, vp,
                              vp, i32, vp, sz, vp]
    L.attnres_full_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i32]
    L.attnres_full_bwd.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, f32, i32, i32, vp, vp, vp, vp, i32, vp,
                                   sz, vp]
    L.attnres_msar_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i32]
    L.attnres_msar_fwd_workspace_size.restype = sz
    L.attnres_msar_fwd.argtypes = [vp, i64, i64, i64, vp, vp, vp, i64, f32, i32, vp, vp, sz, vp]
    L.attnres_msar_fwd.restype = ctypes.c_int
    L.attnres_block_msar_phase1_workspace_size.argtypes = [i64, i64, i64, i64]
    L.attnres_block_msar_phase1_workspace_size.restype = sz
    L.attnres_block_msar_phase1.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, f32, i32, vp, vp, vp, vp, vp, sz,
                                            vp]
    L.attnres_block_msar_phase1.restype = ctypes.c_int
    L.attnres_block_msar_phase2_workspace_size.argtypes = [i64, i64]
    L.attnres_block_msar_phase2_workspace_size.restype = sz
    L.attnres_block_msar_phase2.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp, vp, f32, i32, vp, vp, sz, vp]
    L.attnres_block_msar_phase2.restype = ctypes.c_int
    L.attnres_set_kernel_policy.argtypes = [i32]
    for name in ("attnres_full_fwd", "attnres_block_phase1", "attnres_block_phase2_merge",
                 "attnres_block_phase2_merge_update", "mhar_fwd", "mhar_fwd_chunked",
                 "attnres_bwd", "attnres_full_bwd", "attnres_version", "attnres_set_kernel_policy"):
        getattr(L, name).restype = ctypes.c_int
    L.attnres_full_fwd_workspace_size.restype = sz
    L.mhar_fwd_workspace_size.restype = sz
    L.attnres_bwd_workspace_size.restype = sz
    L.attnres_full_bwd_workspace_size.restype = sz
    L.attnres_last_error.restype = ctypes.c_char_p
    L.attnres_last_error.argtypes = []
    L.attnres_version.argtypes = []
    _lib = L
    return L


def attnres_last_error() -> str:
    return lib().attnres_last_error().decode()


def attnres_version() -> int:
    return lib().attnres_version()


def attnres_set_kernel_policy(policy: int) -> int:
    rc = lib().attnres_set_kernel_policy(policy)
    if rc < 0:
        raise AttnResError(rc, attnres_last_error())
    return rc


def attnres_full_fwd_workspace_size(n_src: int, n_dst: int, d: int, H: int, dtype: int) -> int:
    return lib().attnres_full_fwd_workspace_size(n_src, n_dst, d, H, dtype)


def mhar_fwd_workspace_size(N: int, S: int, T: int, d: int, H: int) -> int:
    return lib().mhar_fwd_workspace_size(N, S, T, d, H)


def attnres_full_bwd_workspace_size(n_src: int, n_dst: int, T: int, d: int, H: int) -> int:
    return lib().attnres_full_bwd_workspace_size(n_src, n_dst, T, d, H)


def attnres_bwd_workspace_size(N: int, S: int, T: int, d: int, H: int) -> int:
    return lib().attnres_bwd_workspace_size(N, S, T, d, H)


# ----------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


_CODES = {}


def _code(t) -> int:
    if not _CODES:
        torch = _torch()
        _CODES.update({torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16})
    code = _CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    """Raw HIP stream: the given torch stream, else torch's current stream on the
    current device (read without building a Stream object: at decode sizes the
    call overhead is comparable to the kernels)."""
    if stream is not None:
        return stream.cuda_stream
    C = _torch()._C
    return C._cuda_getCurrentRawStream(C._cuda_getDevice())


def _gain(gain, rows: int, d: int):
    """(pointer, gain_ld) for a gain tensor: [rows, d] -> ld d, [d] -> ld 0, None -> NULL."""
    if gain is None:
        return None, 0
    if gain.dim() == 1:
        return _p(gain), 0
    if tuple(gain.shape) != (rows, d):
        raise ValueError(f"gain must be [{rows}, {d}] or [{d}]")
    return _p(gain), d


def _check(rc: int) -> None:
    if rc != 0:
        raise AttnResError(rc, attnres_last_error())


# ----------------------------------------------------------------- entry points
def attnres_full_fwd(src, w, gain=None, eps: float = 1e-6, H: int = 1, out=None, ws=None, stream=None):
    """Full AttnRes forward.  src [n_src, T, d]; w [n_dst, d] -> out [n_dst, T, d]."""
    torch = _torch()
    n_src, T, d = src.shape
    n_dst = w.shape[0]
    if out is None:
        out = torch.empty((n_dst, T, d), dtype=src.dtype, device=src.device)
    need = attnres_full_fwd_workspace_size(n_src, n_dst, d, H, _code(src))
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=src.device)
    gp, gld = _gain(gain, n_dst, d)
    _check(lib().attnres_full_fwd(_p(src), n_src, T, d, _p(w), n_dst, gp, gld, eps, H, _code(src),
                                  _p(out), _p(ws), _nbytes(ws), _stream(stream)))
    return out


def attnres_block_phase1(reps, w, gain=None, eps: float = 1e-6, H: int = 1, h_first=None, o_state=None,
                         o_dtype=None, lse=None, o_scale=None, stream=None):
    """Block Phase 1.  reps [N, T, d]; w [S, d] ->
    (h_first [T, d], o_state [S-1, T, d], lse [S, H, T], o_scale [T] or None).

    o_dtype: torch.float32 (default), reps.dtype, or torch.float16 (the scaled
    fp16 state, bf16 reps only; o_scale then holds the per-token scales)."""
    torch = _torch()
    N, T, d = reps.shape
    S = w.shape[0]
    if h_first is None:
        h_first = torch.empty((T, d), dtype=reps.dtype, device=reps.device)
    if o_state is None:
        o_state = torch.empty((S - 1, T, d), dtype=torch.float32 if o_dtype is None else o_dtype,
                              device=reps.device)
    if lse is None:
        lse = torch.empty((S, H, T), dtype=torch.float32, device=reps.device)
    scaled = o_state.dtype == torch.float16
    if o_scale is None and scaled:
        o_scale = torch.empty((T,), dtype=torch.float32, device=reps.device)
    gp, gld = _gain(gain, S, d)
    _check(lib().attnres_block_phase1(_p(reps), N, T, d, _p(w), S, gp, gld, eps, H, _code(reps),
                                      _p(h_first), _p(o_state) if S > 1 else None, _code(o_state),
                                      _p(lse), _p(o_scale) if scaled else None, _stream(stream)))
    return h_first, o_state, lse, (o_scale if scaled else None)


def attnres_block_phase2_merge(o_i, lse_i, partial, w_i, gain_i=None, eps: float = 1e-6, H: int = 1,
                               h_i=None, o_scale=None, stream=None):
    """Block Phase 2 merge.  o_i [T, d]; lse_i [H, T]; partial [T, d] -> h_i [T, d].

    o_scale [T] is required when o_i is the scaled fp16 state."""
    T, d = partial.shape
    if h_i is None:
        h_i = _torch().empty((T, d), dtype=partial.dtype, device=partial.device)
    _check(lib().attnres_block_phase2_merge(_p(o_i), _code(o_i), _p(o_scale), _p(lse_i), _p(partial), T, d,
                                            _p(w_i), _p(gain_i), eps, H, _code(partial), _p(h_i),
                                            _stream(stream)))
    return h_i


def attnres_block_phase2_merge_update(o_i, lse_i, partial_prev, f_prev, w_i, gain_i=None, eps: float = 1e-6,
                                      H: int = 1, partial_out=None, h_i=None, norm_eps: float = 1e-6,
                                      h_inv_rms=None, o_scale=None, stream=None):
    """Phase 2 merge fused with the partial-sum update and the inverse RMS of h_i.

    partial_prev [T, d] or None (the block's first update); f_prev [T, d].
    Returns (partial_out, h_i, h_inv_rms).  Pass partial_out=partial_prev to
    update in place, and h_inv_rms=False to skip the statistic."""
    torch = _torch()
    T, d = f_prev.shape
    dev = f_prev.device
    if partial_out is None:
        partial_out = torch.empty((T, d), dtype=f_prev.dtype, device=dev)
    if h_i is None:
        h_i = torch.empty((T, d), dtype=f_prev.dtype, device=dev)
    if h_inv_rms is None:
        h_inv_rms = torch.empty((T,), dtype=torch.float32, device=dev)
    rms = None if h_inv_rms is False else h_inv_rms
    _check(lib().attnres_block_phase2_merge_update(
        _p(o_i), _code(o_i), _p(o_scale), _p(lse_i), _p(partial_prev), _p(f_prev), T, d, _p(w_i), _p(gain_i),
        eps, H, _code(f_prev), _p(partial_out), _p(h_i), norm_eps, _p(rms), _stream(stream)))
    return partial_out, h_i, rms


def mhar_fwd(reps, partials, w, gain=None, eps: float = 1e-6, H: int = 1, h=None, ws=None,
             stream=None):
    """One block of (multi-head) Block AttnRes: Phase 1 + S-1 merges -> h [S, T, d]."""
    torch = _torch()
    N, T, d = reps.shape
    S = w.shape[0]
    if h is None:
        h = torch.empty((S, T, d), dtype=reps.dtype, device=reps.device)
    need = mhar_fwd_workspace_size(N, S, T, d, H)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=reps.device)
    gp, gld = _gain(gain, S, d)
    _check(lib().mhar_fwd(_p(reps), N, _p(partials) if S > 1 else None, S, T, d, _p(w), gp, gld, eps, H,
                          _code(reps), _p(h), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return h


def mhar_fwd_chunked(reps, partials, w, chunk_T: int, gain=None, eps: float = 1e-6, H: int = 1, h=None, ws=None,
                     stream=None):
    """mhar_fwd over T-chunks of chunk_T tokens, with a workspace sized for one chunk."""
    torch = _torch()
    N, T, d = reps.shape
    S = w.shape[0]
    if h is None:
        h = torch.empty((S, T, d), dtype=reps.dtype, device=reps.device)
    need = mhar_fwd_workspace_size(N, S, max(1, min(T, chunk_T)), d, H)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=reps.device)
    gp, gld = _gain(gain, S, d)
    _check(lib().mhar_fwd_chunked(_p(reps), N, _p(partials) if S > 1 else None, S, T, d, _p(w), gp, gld, eps, H,
                                  _code(reps), _p(h), chunk_T, _p(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))
    return h


def attnres_msar_fwd_workspace_size(n_src: int, n_dst: int, T: int, d: int, dtype: int) -> int:
    return lib().attnres_msar_fwd_workspace_size(n_src, n_dst, T, d, dtype)


def attnres_msar_fwd(src, w, conv, mix, eps: float = 1e-6, out=None, ws=None, stream=None):
    """MSAR forward.  src [n_src, T, d]; w [n_dst, 4, d]; conv [24, d]; mix [n_dst, 4 d, 4]
    -> out [n_dst, T, d]."""
    torch = _torch()
    n_src, T, d = src.shape
    n_dst = w.shape[0]
    if out is None:
        out = torch.empty((n_dst, T, d), dtype=src.dtype, device=src.device)
    need = attnres_msar_fwd_workspace_size(n_src, n_dst, T, d, _code(src))
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=src.device)
    _check(lib().attnres_msar_fwd(_p(src), n_src, T, d, _p(w), _p(conv), _p(mix), n_dst, eps, _code(src), _p(out),
                                  _p(ws), _nbytes(ws), _stream(stream)))
    return out


def attnres_block_msar_phase1_workspace_size(N: int, S: int, T: int, d: int) -> int:
    return lib().attnres_block_msar_phase1_workspace_size(N, S, T, d)


def attnres_block_msar_phase2_workspace_size(T: int, d: int) -> int:
    return lib().attnres_block_msar_phase2_workspace_size(T, d)


def attnres_block_msar_phase1(reps, w, conv, mix1, eps: float = 1e-6, h1=None, o_state=None, o_scale=None, lse=None,
                              ws=None, stream=None):
    """Block MSAR Phase 1.  reps [N, T, d] bf16; w [S, 4, d]; conv [24, d]; mix1 [4 d, 4]
    -> (h1 [T, d], o_state [S-1, 4, T, d] fp16, o_scale [T] fp32, lse [S-1, 4, T] fp32)."""
    torch = _torch()
    N, T, d = reps.shape
    S = w.shape[0]
    dev = reps.device
    if h1 is None:
        h1 = torch.empty((T, d), dtype=reps.dtype, device=dev)
    if o_state is None:
        o_state = torch.empty((max(S - 1, 0), 4, T, d), dtype=torch.float16, device=dev)
    if o_scale is None:
        o_scale = torch.empty((T,), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((max(S - 1, 0), 4, T), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(max(1, attnres_block_msar_phase1_workspace_size(N, S, T, d)), dtype=torch.uint8,
                         device=dev)
    _check(lib().attnres_block_msar_phase1(_p(reps), N, T, d, _p(w), S, _p(conv), _p(mix1), eps, _code(reps),
                                           _p(h1), _p(o_state) if S > 1 else None, _p(o_scale),
                                           _p(lse) if S > 1 else None, _p(ws), _nbytes(ws), _stream(stream)))
    return h1, o_state, o_scale, lse


def attnres_block_msar_phase2(o_i, o_scale, lse_i, partial, w_i, conv, mix_i, eps: float = 1e-6, h_i=None, ws=None,
                              stream=None):
    """Block MSAR Phase 2 for one sublayer: o_i [4, T, d] fp16, o_scale [T], lse_i [4, T], partial [T, d]
    -> h_i [T, d]."""
    torch = _torch()
    T, d = partial.shape
    if h_i is None:
        h_i = torch.empty((T, d), dtype=partial.dtype, device=partial.device)
    if ws is None:
        ws = torch.empty(max(1, attnres_block_msar_phase2_workspace_size(T, d)), dtype=torch.uint8,
                         device=partial.device)
    _check(lib().attnres_block_msar_phase2(_p(o_i), _p(o_scale), _p(lse_i), _p(partial), T, d, _p(w_i), _p(conv), _p(mix_i), eps,
                                           _code(partial), _p(h_i), _p(ws), _nbytes(ws), _stream(stream)))
    return h_i


def attnres_bwd(reps, partials, w, dh, gain=None, eps: float = 1e-6, H: int = 1, d_reps=None,
                d_partials=None, dw=None, dgain=None, accumulate: bool = False, ws=None, stream=None):
    """Backward of mhar_fwd -> (d_reps, d_partials, dw, dgain)."""
    torch = _torch()
    N, T, d = reps.shape
    S = w.shape[0]
    dev = reps.device
    if d_reps is None:
        d_reps = torch.empty_like(reps)
    if d_partials is None and S > 1:
        d_partials = torch.empty((S - 1, T, d), dtype=reps.dtype, device=dev)
    if dw is None:
        dw = torch.empty((S, d), dtype=torch.float32, device=dev)
    if dgain is None and gain is not None:
        dgain = torch.empty(tuple(gain.shape), dtype=torch.float32, device=dev)
    need = attnres_bwd_workspace_size(N, S, T, d, H)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    gp, gld = _gain(gain, S, d)
    _check(lib().attnres_bwd(_p(reps), N, _p(partials) if S > 1 else None, S, T, d, _p(w), gp, gld, eps,
                             H, _code(reps), _p(dh), _p(d_reps), _p(d_partials) if S > 1 else None,
                             _p(dw), _p(dgain), int(bool(accumulate)), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)))
    return d_reps, d_partials, dw, dgain


def attnres_full_bwd(src, w, dout, gain=None, eps: float = 1e-6, H: int = 1, d_src=None, dw=None, dgain=None,
                     accumulate: bool = False, ws=None, stream=None):
    """Backward of attnres_full_fwd -> (d_src, dw, dgain)."""
    torch = _torch()
    n_src, T, d = src.shape
    n_dst = w.shape[0]
    dev = src.device
    if d_src is None:
        d_src = torch.empty_like(src)
    if dw is None:
        dw = torch.empty((n_dst, d), dtype=torch.float32, device=dev)
    if dgain is None and gain is not None:
        dgain = torch.empty(tuple(gain.shape), dtype=torch.float32, device=dev)
    need = attnres_full_bwd_workspace_size(n_src, n_dst, T, d, H)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    gp, gld = _gain(gain, n_dst, d)
    _check(lib().attnres_full_bwd(_p(src), n_src, T, d, _p(w), n_dst, gp, gld, eps, H, _code(src), _p(dout),
                                  _p(d_src), _p(dw), _p(dgain), int(bool(accumulate)), _p(ws), _nbytes(ws),
                                  _stream(stream)))
    return d_src, dw, dgain
