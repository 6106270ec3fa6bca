"""Thin ctypes binding of libattnres.so.

Argument marshalling only: every function here checks the tensors it is given
(device, dtype, shape, contiguity), fills in sizes and pointers from them
(torch supplies device memory and the stream) and calls the C entry point of
the same name.  All arithmetic runs in the library's HIP kernels; there is no
fallback.  A missing library raises at first use.

The C ABI receives bare pointers and cannot see a tensor's device or dtype, so
those checks happen here, before any call into the library: a CPU tensor, a
wrong dtype or a wrong shape raises TypeError or ValueError and nothing is
enqueued.  Tensors the binding allocates (outputs left as None, workspaces) are
allocated on the stream the call runs on, so the caching allocator does not
hand their memory to other work while the call still uses it.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattnres.so")

F32 = 0
BF16 = 1
F16 = 2  # Phase-1 state only: fp16 scaled per token by a power of two

OP_PHASE1, OP_PHASE2, OP_BWD, OP_FULL_FWD, OP_FULL_BWD = 0, 1, 2, 3, 4

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
    sig = {
        "attnres_full_fwd_workspace_size": ([i64, i64, i64, i32, i32], sz),
        "attnres_full_fwd": ([vp, i64, i64, i64, vp, i64, vp, i64, f32, i32, i32, vp, vp, sz, vp], ctypes.c_int),
        "attnres_block_phase1": ([vp, i64, i64, i64, vp, i64, vp, i64, f32, i32, i32, vp, vp, i32, vp, vp, vp],
                                 ctypes.c_int),
        "attnres_block_phase2_merge": ([vp, i32, vp, vp, vp, i64, i64, vp, vp, f32, i32, i32, vp, vp], ctypes.c_int),
        "attnres_block_phase2_merge_update": ([vp, i32, vp, vp, vp, vp, i64, i64, vp, vp, f32, i32, i32, vp, vp, f32,
                                               vp, vp], ctypes.c_int),
        "mhar_fwd_workspace_size": ([i64, i64, i64, i64, i32], sz),
        "mhar_fwd": ([vp, i64, vp, i64, i64, i64, vp, vp, i64, f32, i32, i32, vp, vp, sz, vp], ctypes.c_int),
        "mhar_fwd_chunked": ([vp, i64, vp, i64, i64, i64, vp, vp, i64, f32, i32, i32, vp, i64, vp, sz, vp],
                             ctypes.c_int),
        "mhar_fwd_noalloc": ([vp, i64, vp, i64, i64, i64, vp, vp, i64, f32, i32, i32, vp, vp], ctypes.c_int),
        "attnres_bwd_workspace_size": ([i64, i64, i64, i64, i32], sz),
        "attnres_bwd": ([vp, i64, vp, i64, i64, i64, vp, vp, i64, f32, i32, i32, vp, vp, vp, vp, vp, i32, vp, sz,
                         vp], ctypes.c_int),
        "attnres_full_bwd_workspace_size": ([i64, i64, i64, i64, i32], sz),
        "attnres_full_bwd": ([vp, i64, i64, i64, vp, i64, vp, i64, f32, i32, i32, vp, vp, vp, vp, i32, vp, sz, vp],
                             ctypes.c_int),
        "attnres_msar_fwd_workspace_size": ([i64, i64, i64, i64, i32], sz),
        "attnres_msar_fwd": ([vp, i64, i64, i64, vp, vp, vp, i64, f32, i32, vp, vp, sz, vp], ctypes.c_int),
        "attnres_block_msar_phase1_workspace_size": ([i64, i64, i64, i64], sz),
        "attnres_block_msar_phase1": ([vp, i64, i64, i64, vp, i64, vp, vp, f32, i32, vp, vp, vp, vp, vp, sz, vp],
                                      ctypes.c_int),
        "attnres_block_msar_phase2_workspace_size": ([i64, i64], sz),
        "attnres_block_msar_phase2": ([vp, vp, vp, vp, i64, i64, vp, vp, vp, f32, i32, vp, vp, sz, vp], ctypes.c_int),
        "attnres_set_kernel_policy": ([i32], ctypes.c_int),
        "attnres_kernel_variant": ([i32, i64, i64, i64, i64, i32, i32, i32, ctypes.c_char_p, sz], ctypes.c_int),
        "attnres_last_error": ([], ctypes.c_char_p),
        "attnres_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
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


def attnres_kernel_variant(op: int, N: int, S: int, T: int, d: int, H: int = 1, dtype: int = BF16,
                           o_dtype: int = F16) -> str:
    """Name of the kernel a call would run (host logic only; no GPU needed)."""
    buf = ctypes.create_string_buffer(256)
    rc = lib().attnres_kernel_variant(op, N, S, T, d, H, dtype, o_dtype, buf, len(buf))
    if rc != 0:
        raise AttnResError(rc, attnres_last_error())
    return buf.value.decode()


def attnres_full_fwd_workspace_size(n_src: int, n_dst: int, d: int, H: int, dtype: int) -> int:
    return lib().attnres_full_fwd_workspace_size(n_src, n_dst, d, H, dtype)


def mhar_fwd_workspace_size(N: int, S: int, T: int, d: int, H: int) -> int:
    return lib().mhar_fwd_workspace_size(N, S, T, d, H)


def attnres_full_bwd_workspace_size(n_src: int, n_dst: int, T: int, d: int, H: int) -> int:
    return lib().attnres_full_bwd_workspace_size(n_src, n_dst, T, d, H)


def attnres_bwd_workspace_size(N: int, S: int, T: int, d: int, H: int) -> int:
    return lib().attnres_bwd_workspace_size(N, S, T, d, H)


def attnres_msar_fwd_workspace_size(n_src: int, n_dst: int, T: int, d: int, dtype: int) -> int:
    return lib().attnres_msar_fwd_workspace_size(n_src, n_dst, T, d, dtype)


def attnres_block_msar_phase1_workspace_size(N: int, S: int, T: int, d: int) -> int:
    return lib().attnres_block_msar_phase1_workspace_size(N, S, T, d)


def attnres_block_msar_phase2_workspace_size(T: int, d: int) -> int:
    return lib().attnres_block_msar_phase2_workspace_size(T, d)


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
    return None if t is None else t.data_ptr()


def _act(t, name: str):
    """An activation tensor: fp32 or bf16 on a GPU, contiguous."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _chk(t, name: str, shape, dtype, device, optional: bool = False):
    """Check a tensor argument against its expected shape, dtype and device."""
    torch = _torch()
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise TypeError(f"{name} must be {' or '.join(str(x) for x in allowed)}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ws(t, name: str, device):
    """A caller's workspace: any shape, on the device, contiguous."""
    if t is None:
        return None
    return _chk(t, name, None, None, device)


def _stream(stream) -> int:
    """Raw HIP stream: the given torch stream, else torch's current stream on the
    current device (read without building a Stream object: at decode sizes the
    call overhead is comparable to the kernels)."""
    if stream is not None:
        return stream.cuda_stream
    C = _torch()._C
    return C._cuda_getCurrentRawStream(C._cuda_getDevice())


def _on(stream):
    """Allocations made inside belong to `stream` (when one is given)."""
    return _torch().cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _gain(gain, rows: int, d: int, device):
    """(pointer, gain_ld) for a gain tensor: [rows, d] -> ld d, [d] -> ld 0, None -> NULL."""
    if gain is None:
        return None, 0
    torch = _torch()
    if gain.dim() == 1:
        _chk(gain, "gain", (d,), torch.float32, device)
        return _p(gain), 0
    _chk(gain, "gain", (rows, d), torch.float32, device)
    return _p(gain), d


def _check(rc: int) -> None:
    if rc != 0:
        raise AttnResError(rc, attnres_last_error())


# ----------------------------------------------------------------- entry points
def attnres_full_fwd(src, w, gain=None, eps: float = 1e-6, H: int = 1, out=None, ws=None, stream=None):
    """Full AttnRes forward.  src [n_src, T, d]; w [n_dst, d] -> out [n_dst, T, d]."""
    torch = _torch()
    _act(src, "src")
    n_src, T, d = src.shape
    dev = src.device
    n_dst = _chk(w, "w", None, torch.float32, dev).shape[0]
    _chk(w, "w", (n_dst, d), torch.float32, dev)
    gp, gld = _gain(gain, n_dst, d, dev)
    _chk(out, "out", (n_dst, T, d), src.dtype, dev, optional=True)
    _ws(ws, "ws", dev)
    with _on(stream):
        if out is None:
            out = torch.empty((n_dst, T, d), dtype=src.dtype, device=dev)
        need = attnres_full_fwd_workspace_size(n_src, n_dst, d, H, _code(src))
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        _check(lib().attnres_full_fwd(_p(src), n_src, T, d, _p(w), n_dst, gp, gld, eps, H, _code(src),
                                      _p(out), _p(ws), _nbytes(ws), _stream(stream)))
    return out


def attnres_block_phase1(reps, w, gain=None, eps: float = 1e-6, H: int = 1, h_first=None, o_state=None,
                         o_dtype=None, lse=None, o_scale=None, stream=None):
    """Block Phase 1.  reps [N, T, d]; w [S, d] ->
    (h_first [T, d], o_state [S-1, T, d], lse [S, H, T], o_scale [T] or None).

    o_dtype: torch.float32 (default) or torch.float16 (the scaled fp16 state,
    bf16 reps only; o_scale then holds the per-token scales)."""
    torch = _torch()
    _act(reps, "reps")
    N, T, d = reps.shape
    dev = reps.device
    S = _chk(w, "w", None, torch.float32, dev).shape[0]
    _chk(w, "w", (S, d), torch.float32, dev)
    gp, gld = _gain(gain, S, d, dev)
    _chk(h_first, "h_first", (T, d), reps.dtype, dev, optional=True)
    state_dt = o_state.dtype if o_state is not None else (torch.float32 if o_dtype is None else o_dtype)
    if state_dt not in (torch.float32, torch.float16, torch.bfloat16):
        raise TypeError(f"o_dtype must be float32 or float16, got {state_dt}")
    _chk(o_state, "o_state", (S - 1, T, d), state_dt, dev, optional=True)
    _chk(lse, "lse", (S, H, T), torch.float32, dev, optional=True)
    scaled = state_dt == torch.float16
    _chk(o_scale, "o_scale", (T,), torch.float32, dev, optional=True)
    with _on(stream):
        if h_first is None:
            h_first = torch.empty((T, d), dtype=reps.dtype, device=dev)
        if o_state is None:
            o_state = torch.empty((S - 1, T, d), dtype=state_dt, device=dev)
        if lse is None:
            lse = torch.empty((S, H, T), dtype=torch.float32, device=dev)
        if o_scale is None and scaled:
            o_scale = torch.empty((T,), dtype=torch.float32, device=dev)
        _check(lib().attnres_block_phase1(_p(reps), N, T, d, _p(w), S, gp, gld, eps, H, _code(reps),
                                          _p(h_first), _p(o_state) if S > 1 else None, _code(o_state),
                                          _p(lse), _p(o_scale) if scaled else None, _stream(stream)))
    return h_first, o_state, lse, (o_scale if scaled else None)


def _merge_inputs(o_i, lse_i, w_i, gain_i, H, T, d, dev, o_scale):
    torch = _torch()
    _chk(o_i, "o_i", (T, d), (torch.float32, torch.float16, torch.bfloat16), dev)
    _chk(lse_i, "lse_i", (H, T), torch.float32, dev)
    _chk(w_i, "w_i", (d,), torch.float32, dev)
    _chk(gain_i, "gain_i", (d,), torch.float32, dev, optional=True)
    _chk(o_scale, "o_scale", (T,), torch.float32, dev, optional=o_i.dtype != torch.float16)


def attnres_block_phase2_merge(o_i, lse_i, partial, w_i, gain_i=None, eps: float = 1e-6, H: int = 1,
                               h_i=None, o_scale=None, stream=None):
    """Block Phase 2 merge.  o_i [T, d]; lse_i [H, T]; partial [T, d] -> h_i [T, d].

    o_scale [T] is required when o_i is the scaled fp16 state.  h_i may be o_i
    itself when the state has the I/O element size (in place)."""
    _act(partial, "partial")
    T, d = partial.shape
    dev = partial.device
    _merge_inputs(o_i, lse_i, w_i, gain_i, H, T, d, dev, o_scale)
    _chk(h_i, "h_i", (T, d), None, dev, optional=True)
    with _on(stream):
        if h_i is None:
            h_i = _torch().empty((T, d), dtype=partial.dtype, device=dev)
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
    _act(f_prev, "f_prev")
    T, d = f_prev.shape
    dev = f_prev.device
    _merge_inputs(o_i, lse_i, w_i, gain_i, H, T, d, dev, o_scale)
    _chk(partial_prev, "partial_prev", (T, d), f_prev.dtype, dev, optional=True)
    _chk(partial_out, "partial_out", (T, d), f_prev.dtype, dev, optional=True)
    _chk(h_i, "h_i", (T, d), None, dev, optional=True)
    if h_inv_rms is not None and h_inv_rms is not False:
        _chk(h_inv_rms, "h_inv_rms", (T,), torch.float32, dev)
    with _on(stream):
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


def _block_inputs(reps, partials, w, S_expected=None):
    torch = _torch()
    _act(reps, "reps")
    N, T, d = reps.shape
    dev = reps.device
    S = _chk(w, "w", None, torch.float32, dev).shape[0]
    _chk(w, "w", (S, d), torch.float32, dev)
    if S > 1:
        _chk(partials, "partials", (S - 1, T, d), reps.dtype, dev)
    return N, S, T, d, dev


def mhar_fwd(reps, partials, w, gain=None, eps: float = 1e-6, H: int = 1, h=None, ws=None,
             stream=None):
    """One block of (multi-head) Block AttnRes: Phase 1 + S-1 merges -> h [S, T, d]."""
    torch = _torch()
    N, S, T, d, dev = _block_inputs(reps, partials, w)
    gp, gld = _gain(gain, S, d, dev)
    _chk(h, "h", (S, T, d), reps.dtype, dev, optional=True)
    _ws(ws, "ws", dev)
    with _on(stream):
        if h is None:
            h = torch.empty((S, T, d), dtype=reps.dtype, device=dev)
        if ws is None:
            ws = torch.empty(max(mhar_fwd_workspace_size(N, S, T, d, H), 1), dtype=torch.uint8, device=dev)
        _check(lib().mhar_fwd(_p(reps), N, _p(partials) if S > 1 else None, S, T, d, _p(w), gp, gld, eps, H,
                              _code(reps), _p(h), _p(ws), _nbytes(ws), _stream(stream)))
    return h


def mhar_fwd_noalloc(reps, partials, w, h, gain=None, eps: float = 1e-6, H: int = 1, stream=None):
    """mhar_fwd with its workspace in the library's static per-device scratch:
    the call allocates nothing (h is the caller's [S, T, d] output)."""
    N, S, T, d, dev = _block_inputs(reps, partials, w)
    gp, gld = _gain(gain, S, d, dev)
    _chk(h, "h", (S, T, d), reps.dtype, dev)
    _check(lib().mhar_fwd_noalloc(_p(reps), N, _p(partials) if S > 1 else None, S, T, d, _p(w), gp, gld, eps, H,
                                  _code(reps), _p(h), _stream(stream)))
    return h


def mhar_fwd_chunked(reps, partials, w, chunk_T: int, gain=None, eps: float = 1e-6, H: int = 1, h=None, ws=None,
                     stream=None):
    """mhar_fwd over T-chunks of chunk_T tokens, with a workspace sized for one chunk."""
    torch = _torch()
    N, S, T, d, dev = _block_inputs(reps, partials, w)
    gp, gld = _gain(gain, S, d, dev)
    _chk(h, "h", (S, T, d), reps.dtype, dev, optional=True)
    _ws(ws, "ws", dev)
    with _on(stream):
        if h is None:
            h = torch.empty((S, T, d), dtype=reps.dtype, device=dev)
        if ws is None:
            need = mhar_fwd_workspace_size(N, S, max(1, min(T, chunk_T)), d, H)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _check(lib().mhar_fwd_chunked(_p(reps), N, _p(partials) if S > 1 else None, S, T, d, _p(w), gp, gld, eps,
                                      H, _code(reps), _p(h), chunk_T, _p(ws), _nbytes(ws), _stream(stream)))
    return h


def attnres_msar_fwd(src, w, conv, mix, eps: float = 1e-6, out=None, ws=None, stream=None):
    """MSAR forward.  src [n_src, T, d]; w [n_dst, 4, d]; conv [24, d]; mix [n_dst, 4 d, 4]
    -> out [n_dst, T, d]."""
    torch = _torch()
    _act(src, "src")
    n_src, T, d = src.shape
    dev = src.device
    n_dst = _chk(w, "w", None, torch.float32, dev).shape[0]
    _chk(w, "w", (n_dst, 4, d), torch.float32, dev)
    _chk(conv, "conv", (24, d), torch.float32, dev)
    _chk(mix, "mix", (n_dst, 4 * d, 4), torch.float32, dev)
    _chk(out, "out", (n_dst, T, d), src.dtype, dev, optional=True)
    _ws(ws, "ws", dev)
    with _on(stream):
        if out is None:
            out = torch.empty((n_dst, T, d), dtype=src.dtype, device=dev)
        need = attnres_msar_fwd_workspace_size(n_src, n_dst, T, d, _code(src))
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        _check(lib().attnres_msar_fwd(_p(src), n_src, T, d, _p(w), _p(conv), _p(mix), n_dst, eps, _code(src),
                                      _p(out), _p(ws), _nbytes(ws), _stream(stream)))
    return out


def attnres_block_msar_phase1(reps, w, conv, mix1, eps: float = 1e-6, h1=None, o_state=None, o_scale=None, lse=None,
                              ws=None, stream=None):
    """Block MSAR Phase 1.  reps [N, T, d] bf16; w [S, 4, d]; conv [24, d]; mix1 [4 d, 4]
    -> (h1 [T, d], o_state [S-1, 4, T, d] fp16, o_scale [T] fp32, lse [S-1, 4, T] fp32)."""
    torch = _torch()
    _act(reps, "reps")
    N, T, d = reps.shape
    dev = reps.device
    S = _chk(w, "w", None, torch.float32, dev).shape[0]
    _chk(w, "w", (S, 4, d), torch.float32, dev)
    _chk(conv, "conv", (24, d), torch.float32, dev)
    _chk(mix1, "mix1", (4 * d, 4), torch.float32, dev)
    _chk(h1, "h1", (T, d), reps.dtype, dev, optional=True)
    _chk(o_state, "o_state", (max(S - 1, 0), 4, T, d), torch.float16, dev, optional=True)
    _chk(o_scale, "o_scale", (T,), torch.float32, dev, optional=True)
    _chk(lse, "lse", (max(S - 1, 0), 4, T), torch.float32, dev, optional=True)
    _ws(ws, "ws", dev)
    with _on(stream):
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
    _act(partial, "partial")
    T, d = partial.shape
    dev = partial.device
    _chk(o_i, "o_i", (4, T, d), torch.float16, dev)
    _chk(o_scale, "o_scale", (T,), torch.float32, dev)
    _chk(lse_i, "lse_i", (4, T), torch.float32, dev)
    _chk(w_i, "w_i", (4, d), torch.float32, dev)
    _chk(conv, "conv", (24, d), torch.float32, dev)
    _chk(mix_i, "mix_i", (4 * d, 4), torch.float32, dev)
    _chk(h_i, "h_i", (T, d), partial.dtype, dev, optional=True)
    _ws(ws, "ws", dev)
    with _on(stream):
        if h_i is None:
            h_i = torch.empty((T, d), dtype=partial.dtype, device=dev)
        if ws is None:
            ws = torch.empty(max(1, attnres_block_msar_phase2_workspace_size(T, d)), dtype=torch.uint8, device=dev)
        _check(lib().attnres_block_msar_phase2(_p(o_i), _p(o_scale), _p(lse_i), _p(partial), T, d, _p(w_i),
                                               _p(conv), _p(mix_i), eps, _code(partial), _p(h_i), _p(ws), _nbytes(ws),
                                               _stream(stream)))
    return h_i


def attnres_bwd(reps, partials, w, dh, gain=None, eps: float = 1e-6, H: int = 1, d_reps=None,
                d_partials=None, dw=None, dgain=None, accumulate: bool = False, ws=None, stream=None):
    """Backward of mhar_fwd -> (d_reps, d_partials, dw, dgain)."""
    torch = _torch()
    N, S, T, d, dev = _block_inputs(reps, partials, w)
    gp, gld = _gain(gain, S, d, dev)
    _chk(dh, "dh", (S, T, d), reps.dtype, dev)
    _chk(d_reps, "d_reps", (N, T, d), reps.dtype, dev, optional=True)
    _chk(d_partials, "d_partials", (S - 1, T, d), reps.dtype, dev, optional=True)
    _chk(dw, "dw", (S, d), torch.float32, dev, optional=True)
    if gain is not None:
        _chk(dgain, "dgain", tuple(gain.shape), torch.float32, dev, optional=True)
    _ws(ws, "ws", dev)
    with _on(stream):
        if d_reps is None:
            d_reps = torch.empty_like(reps)
        if d_partials is None and S > 1:
            d_partials = torch.empty((S - 1, T, d), dtype=reps.dtype, device=dev)
        if dw is None:
            dw = torch.empty((S, d), dtype=torch.float32, device=dev)
        if dgain is None and gain is not None:
            dgain = torch.empty(tuple(gain.shape), dtype=torch.float32, device=dev)
        if ws is None:
            ws = torch.empty(max(attnres_bwd_workspace_size(N, S, T, d, H), 1), dtype=torch.uint8, device=dev)
        _check(lib().attnres_bwd(_p(reps), N, _p(partials) if S > 1 else None, S, T, d, _p(w), gp, gld, eps,
                                 H, _code(reps), _p(dh), _p(d_reps), _p(d_partials) if S > 1 else None,
                                 _p(dw), _p(dgain), int(bool(accumulate)), _p(ws), _nbytes(ws), _stream(stream)))
    return d_reps, d_partials, dw, dgain


def attnres_full_bwd(src, w, dout, gain=None, eps: float = 1e-6, H: int = 1, d_src=None, dw=None, dgain=None,
                     accumulate: bool = False, ws=None, stream=None):
    """Backward of attnres_full_fwd -> (d_src, dw, dgain)."""
    torch = _torch()
    _act(src, "src")
    n_src, T, d = src.shape
    dev = src.device
    n_dst = _chk(w, "w", None, torch.float32, dev).shape[0]
    _chk(w, "w", (n_dst, d), torch.float32, dev)
    gp, gld = _gain(gain, n_dst, d, dev)
    _chk(dout, "dout", (n_dst, T, d), src.dtype, dev)
    _chk(d_src, "d_src", (n_src, T, d), src.dtype, dev, optional=True)
    _chk(dw, "dw", (n_dst, d), torch.float32, dev, optional=True)
    if gain is not None:
        _chk(dgain, "dgain", tuple(gain.shape), torch.float32, dev, optional=True)
    _ws(ws, "ws", dev)
    with _on(stream):
        if d_src is None:
            d_src = torch.empty_like(src)
        if dw is None:
            dw = torch.empty((n_dst, d), dtype=torch.float32, device=dev)
        if dgain is None and gain is not None:
            dgain = torch.empty(tuple(gain.shape), dtype=torch.float32, device=dev)
        if ws is None:
            ws = torch.empty(max(attnres_full_bwd_workspace_size(n_src, n_dst, T, d, H), 1), dtype=torch.uint8,
                             device=dev)
        _check(lib().attnres_full_bwd(_p(src), n_src, T, d, _p(w), n_dst, gp, gld, eps, H, _code(src), _p(dout),
                                      _p(d_src), _p(dw), _p(dgain), int(bool(accumulate)), _p(ws), _nbytes(ws),
                                      _stream(stream)))
    return d_src, dw, dgain
