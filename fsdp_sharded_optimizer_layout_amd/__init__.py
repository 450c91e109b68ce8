"""Python binding of libfsdpshard.so: one rank's share of a fully sharded training step on MI355X.

Argument marshalling only.  Every computation runs in the library (host layout code and gfx950
kernels); this module turns tensors into pointers and sizes, picks the current HIP stream, and
raises on a non-zero status.  There is no fallback: if the library is missing, every call raises.

Calls (same names as the C ABI in include/fsdpshard.h):
  shard_layout      flat layout + floor-rule slice of one rank (host)
  reduce_shard      fp32 rank-order sum of F bf16 contributions (GPU)
  adamw_shard_step  fused reduce + AdamW + bf16 unflatten of one slice (GPU)
  unflatten_bf16    bf16 copy of an fp32 master slice into the flat layout (GPU)
bf16 tensors may be torch.bfloat16, torch.int16 or torch.uint16 (bit patterns); fp32 tensors
are torch.float32.  All device tensors must be contiguous.
"""

import ctypes
import os
from collections import namedtuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsdpshard.so")
MAX_FAN_IN = 64
STATE_BLOCK = 512          # elements per block of the blocked state layout
SEG_WEIGHT_DECAY = 1
SEG_PADDING = 2

c_i64, c_i32, c_u32, c_vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p


class _Segment(ctypes.Structure):
    _fields_ = [("shard_begin", c_i64), ("length", c_i64), ("tensor_offset", c_i64),
                ("tensor_id", c_i32), ("flags", c_u32)]


class _Layout(ctypes.Structure):
    _fields_ = [("P", c_i64), ("lo", c_i64), ("hi", c_i64), ("n", c_i64), ("n_real", c_i64),
                ("n_segments", c_i32), ("n_tensors", c_i32)]


class _AdamW(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("grad_scale", ctypes.c_double), ("step", c_i64),
                ("max_grad_norm", ctypes.c_double), ("grad_sumsq", c_vp)]


class _Piece(ctypes.Structure):
    _fields_ = [("src_offset", c_i64), ("dst_offset", c_i64), ("length", c_i64),
                ("src_rank", c_i32), ("reserved", c_i32)]


PIECE_DTYPE = np.dtype([("src_offset", "<i8"), ("dst_offset", "<i8"), ("length", "<i8"),
                        ("src_rank", "<i4"), ("reserved", "<i4")])
assert PIECE_DTYPE.itemsize == ctypes.sizeof(_Piece) == 32

# numpy view of fsdpshard_segment (32 bytes)
SEGMENT_DTYPE = np.dtype([("shard_begin", "<i8"), ("length", "<i8"), ("tensor_offset", "<i8"),
                          ("tensor_id", "<i4"), ("flags", "<u4")])
assert SEGMENT_DTYPE.itemsize == ctypes.sizeof(_Segment) == 32

Layout = namedtuple("Layout", "P lo hi n n_real n_segments n_tensors")


class FsdpShardError(RuntimeError):
    def __init__(self, call, code):
        self.code = code
        super().__init__(f"{call} failed: {strerror(code)} (status {code})")


_lib_handle = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m fsdp_sharded_optimizer_layout_amd.build`")
    h = ctypes.CDLL(LIB_PATH)
    h.shard_layout.argtypes = [ctypes.POINTER(c_i64), c_i32, c_i64, ctypes.POINTER(ctypes.c_uint8),
                               c_i32, c_i32, ctypes.POINTER(_Layout), ctypes.POINTER(_Segment), c_i32]
    h.reduce_shard.argtypes = [ctypes.POINTER(c_vp), c_i32, c_i64, ctypes.c_float, c_vp, c_vp]
    h.adamw_shard_step.argtypes = [c_vp, c_vp, c_vp, ctypes.POINTER(c_vp), c_i32, c_i64, c_vp,
                                   c_i32, ctypes.POINTER(_AdamW), c_vp, c_i64, c_i64, c_vp]
    h.unflatten_bf16.argtypes = [c_vp, c_i64, c_vp, c_i32, c_vp, c_i64, c_i64, c_vp]
    h.adamw_shard_step_f32grad.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_i32,
                                           ctypes.POINTER(_AdamW), c_vp, c_i64, c_i64, c_vp]
    h.state_blocked_elems.argtypes = [c_i64]
    h.state_blocked_elems.restype = c_i64
    h.adamw_shard_step_blocked.argtypes = [c_vp, ctypes.POINTER(c_vp), c_i32, c_i64, c_vp, c_i32,
                                           ctypes.POINTER(_AdamW), c_vp, c_i64, c_i64, c_vp]
    h.adamw_shard_step_f32grad_blocked.argtypes = [c_vp, c_vp, c_i64, c_vp, c_i32,
                                                   ctypes.POINTER(_AdamW), c_vp, c_i64, c_i64,
                                                   c_vp]
    h.grads_interleaved_elems.argtypes = [c_i32, c_i64]
    h.grads_interleaved_elems.restype = c_i64
    h.adamw_shard_step_interleaved.argtypes = [c_vp, c_vp, c_i32, c_i64, c_vp, c_i32,
                                               ctypes.POINTER(_AdamW), c_vp, c_i64, c_i64, c_vp]
    h.grads_to_interleaved.argtypes = [ctypes.POINTER(c_vp), c_i32, c_i64, c_vp, c_vp]
    h.grad_sumsq_shard_interleaved.argtypes = [c_vp, c_i32, c_i64, c_vp, c_i32, ctypes.c_float,
                                               c_vp, c_i64, c_vp, c_vp]
    h.reduce_shard_interleaved.argtypes = [c_vp, c_i32, c_i64, ctypes.c_float, c_vp, c_i32, c_vp]
    h.reduce_shard_sumsq_interleaved.argtypes = [c_vp, c_i32, c_i64, ctypes.c_float, c_vp, c_i32,
                                                 c_vp, c_i32, c_vp, c_i64, c_vp, c_vp]
    h.state_to_blocked.argtypes = [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp]
    h.state_from_blocked.argtypes = [c_vp, c_i64, c_vp, c_vp, c_vp, c_vp]
    h.reduce_shard_accumulate.argtypes = [ctypes.POINTER(c_vp), c_i32, c_i64, ctypes.c_float,
                                          c_vp, c_vp]
    h.grad_sumsq_workspace_bytes.argtypes = [c_i64]
    h.grad_sumsq_workspace_bytes.restype = c_i64
    h.grad_sumsq_shard.argtypes = [ctypes.POINTER(c_vp), c_i32, c_vp, c_i64, c_vp, c_i32,
                                   ctypes.c_float, c_vp, c_i64, c_vp, c_vp]
    h.grad_sumsq_shard_noalloc.argtypes = [ctypes.POINTER(c_vp), c_i32, c_vp, c_i64, c_vp, c_i32,
                                           ctypes.c_float, c_vp, c_vp]
    h.reduce_shard_sumsq.argtypes = [ctypes.POINTER(c_vp), c_i32, c_i64, ctypes.c_float, c_vp,
                                     c_i32, c_vp, c_i32, c_vp, c_i64, c_vp, c_vp]
    h.reshard_plan.argtypes = [ctypes.POINTER(c_i64), c_i32, c_i64, c_i32, c_i64, c_i32, c_i32,
                               ctypes.POINTER(_Piece), c_i32, ctypes.POINTER(c_i32)]
    h.reshard_copy.argtypes = [ctypes.POINTER(c_vp), ctypes.POINTER(c_i64), c_i32, c_vp, c_i64,
                               ctypes.POINTER(_Piece), c_i32, c_i32, c_vp]
    h.fsdpshard_strerror.argtypes = [ctypes.c_int]
    h.fsdpshard_strerror.restype = ctypes.c_char_p
    h.fsdpshard_abi_version.argtypes = []
    h.fsdpshard_stream_copy.argtypes = [c_vp, c_vp, c_i64, c_vp]
    h.fsdpshard_stream_mix.argtypes = [ctypes.POINTER(c_vp), c_i32, c_vp, c_vp, c_vp, c_vp, c_i64,
                                       c_vp]
    h.fsdpshard_stream_mix_blocked.argtypes = [ctypes.POINTER(c_vp), c_i32, c_vp, c_vp, c_i64,
                                               c_vp]
    h.fsdpshard_stream_rw.argtypes = [ctypes.POINTER(c_vp), c_i32, ctypes.POINTER(c_vp), c_i32,
                                      c_i64, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]
    h.fsdpshard_stream_mix_interleaved.argtypes = [c_vp, c_i32, c_vp, c_vp, c_i64, c_vp]
    h.fsdpshard_stream_mix_shaped.argtypes = [ctypes.POINTER(c_vp), c_i32, c_vp, c_vp, c_i64,
                                              c_i32, c_i32, c_i32, c_i32, c_vp]
    for name in ("shard_layout", "reduce_shard", "adamw_shard_step", "unflatten_bf16",
                 "adamw_shard_step_f32grad", "reduce_shard_accumulate", "grad_sumsq_shard",
                 "reshard_plan", "reshard_copy",
                 "fsdpshard_abi_version", "fsdpshard_stream_copy", "fsdpshard_stream_rw",
                 "fsdpshard_stream_mix", "fsdpshard_stream_mix_blocked",
                 "fsdpshard_stream_mix_shaped", "fsdpshard_stream_mix_interleaved",
                 "reduce_shard_sumsq", "grad_sumsq_shard_noalloc",
                 "adamw_shard_step_blocked", "adamw_shard_step_f32grad_blocked",
                 "adamw_shard_step_interleaved", "grads_to_interleaved",
                 "grad_sumsq_shard_interleaved", "reduce_shard_interleaved",
                 "reduce_shard_sumsq_interleaved",
                 "state_to_blocked", "state_from_blocked"):
        getattr(h, name).restype = ctypes.c_int
    _lib_handle = h
    return h


def strerror(code):
    return lib().fsdpshard_strerror(int(code)).decode()


def abi_version():
    return lib().fsdpshard_abi_version()


def _check(call, code):
    if code != 0:
        raise FsdpShardError(call, code)


# ------------------------------------------------------------------------------ host layout

def shard_layout(numels, world_size, rank, pad_multiple=1, wd_mask=None):
    """Flat layout and rank ``rank``'s slice.  Returns (Layout, segments) where segments is a
    numpy array of SEGMENT_DTYPE describing [0, n) of the slice in flat order."""
    sizes = np.ascontiguousarray(np.asarray(numels, dtype=np.int64).reshape(-1))
    T = int(sizes.size)
    mask = None
    if wd_mask is not None:
        mask = np.ascontiguousarray(np.asarray(wd_mask, dtype=np.uint8).reshape(-1))
        if mask.size != T:
            raise ValueError("wd_mask needs one entry per tensor")
    h = lib()
    out = _Layout()
    sizes_p = sizes.ctypes.data_as(ctypes.POINTER(c_i64)) if T else None
    mask_p = mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)) if mask is not None else None
    _check("shard_layout", h.shard_layout(sizes_p, T, int(pad_multiple), mask_p, int(world_size),
                                          int(rank), ctypes.byref(out), None, 0))
    segs = np.zeros(out.n_segments, dtype=SEGMENT_DTYPE)
    if out.n_segments:
        _check("shard_layout", h.shard_layout(
            sizes_p, T, int(pad_multiple), mask_p, int(world_size), int(rank), ctypes.byref(out),
            segs.ctypes.data_as(ctypes.POINTER(_Segment)), out.n_segments))
    return Layout(out.P, out.lo, out.hi, out.n, out.n_real, out.n_segments, out.n_tensors), segs


def segments_to_device(segs, device="cuda"):
    """Upload a SEGMENT_DTYPE array as a device byte tensor (pass it as ``segs`` below)."""
    import torch
    raw = np.ascontiguousarray(segs).view(np.uint8)
    return torch.from_numpy(raw.copy()).to(device)


# ------------------------------------------------------------------------------ GPU calls

_BF16_DTYPES = None


def _bf16_dtypes():
    global _BF16_DTYPES
    if _BF16_DTYPES is None:
        import torch
        _BF16_DTYPES = {torch.bfloat16, torch.int16, getattr(torch, "uint16", torch.int16)}
    return _BF16_DTYPES


def _ptr(t, what, dtypes=None, numel=None):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{what} has dtype {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what} holds {t.numel()} elements, {numel} needed")
    return t.data_ptr()


def _need_bytes(t, what, nbytes):
    """The library sees only pointers, so the binding checks that a tensor holds `nbytes`."""
    if t is None or isinstance(t, int):
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes, {nbytes} needed")


def _segs(segs, n_segments):
    _need_bytes(segs, "segs", SEGMENT_DTYPE.itemsize * int(n_segments))
    return _ptr(segs, "segs")


def _stream(stream, like=None):
    if stream is None:
        import torch
        dev = like.device if like is not None and hasattr(like, "device") else None
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call_workspace(nbytes, device, stream):
    """Workspace for one call, allocated through PyTorch's caching allocator.  The block is tied
    to the current stream; when the call runs on another stream, that stream is recorded on the
    tensor so the block is not handed out again before the call's kernels have run."""
    import torch
    ws = torch.empty(max(int(nbytes), 8), dtype=torch.uint8, device=device)
    handle = _stream(stream, ws)
    if handle != torch.cuda.current_stream(ws.device).cuda_stream:
        ws.record_stream(torch.cuda.ExternalStream(handle, device=ws.device))
    return ws


def _contrib_array(contribs, n):
    if not 1 <= len(contribs) <= MAX_FAN_IN:
        raise ValueError(f"fan-in must be 1..{MAX_FAN_IN}")
    arr = (c_vp * len(contribs))()
    for r, c in enumerate(contribs):
        arr[r] = _ptr(c, f"contribution {r}", _bf16_dtypes(), n)
    return arr


def reduce_shard(contribs, out, scale=1.0, n=None, stream=None):
    """out[i] = scale * sum over ranks r (in order) of contribs[r][i], in float32."""
    import torch
    n = out.numel() if n is None else int(n)
    arr = _contrib_array(contribs, n)
    _check("reduce_shard", lib().reduce_shard(
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), n, float(scale),
        _ptr(out, "out", {torch.float32}, n), _stream(stream, out)))


def _hp(step, lr, beta1, beta2, eps, weight_decay, grad_scale, max_grad_norm, grad_sumsq):
    import torch
    sumsq = None
    if max_grad_norm:
        if grad_sumsq is None:
            raise ValueError("clipping needs grad_sumsq (a device float64 tensor)")
        sumsq = _ptr(grad_sumsq, "grad_sumsq", {torch.float64}, 1)
    return _AdamW(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                  float(grad_scale), int(step), float(max_grad_norm or 0.0), sumsq)


def adamw_shard_step(master, m, v, contribs, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                     weight_decay=0.0, grad_scale=1.0, segs=None, n_segments=0, flat=None,
                     flat_index0=0, lo=0, n=None, max_grad_norm=0.0, grad_sumsq=None,
                     stream=None):
    """Fused reduce + AdamW + bf16 unflatten of one slice (see adamw_shard_step in the header).

    ``segs``: device byte tensor from segments_to_device (or None), with ``n_segments`` entries.
    ``flat``: device bf16 window of the flat parameter vector starting at flat index
    ``flat_index0``; the slice's elements land at flat indices [lo, lo + n).
    ``max_grad_norm`` > 0 clips by the global norm whose square is in ``grad_sumsq`` (device).
    """
    import torch
    n = master.numel() if n is None else int(n)
    f32 = {torch.float32}
    arr = _contrib_array(contribs, n)
    hp = _hp(step, lr, beta1, beta2, eps, weight_decay, grad_scale, max_grad_norm, grad_sumsq)
    if flat is not None and not isinstance(flat, int):
        _ptr(flat, "flat", _bf16_dtypes(), n + int(lo) - int(flat_index0))
    _check("adamw_shard_step", lib().adamw_shard_step(
        _ptr(master, "master", f32, n), _ptr(m, "m", f32, n), _ptr(v, "v", f32, n),
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), n,
        _segs(segs, n_segments), int(n_segments), ctypes.byref(hp),
        _ptr(flat, "flat"), int(flat_index0), int(lo), _stream(stream, master)))


def adamw_shard_step_f32grad(master, m, v, grad, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                             weight_decay=0.0, grad_scale=1.0, segs=None, n_segments=0,
                             flat=None, flat_index0=0, lo=0, n=None, max_grad_norm=0.0,
                             grad_sumsq=None, stream=None):
    """As adamw_shard_step, fed by one fp32 gradient shard ``grad``."""
    import torch
    n = master.numel() if n is None else int(n)
    f32 = {torch.float32}
    hp = _hp(step, lr, beta1, beta2, eps, weight_decay, grad_scale, max_grad_norm, grad_sumsq)
    if flat is not None and not isinstance(flat, int):
        _ptr(flat, "flat", _bf16_dtypes(), n + int(lo) - int(flat_index0))
    _check("adamw_shard_step_f32grad", lib().adamw_shard_step_f32grad(
        _ptr(master, "master", f32, n), _ptr(m, "m", f32, n), _ptr(v, "v", f32, n),
        _ptr(grad, "grad", f32, n), n, _segs(segs, n_segments), int(n_segments), ctypes.byref(hp),
        _ptr(flat, "flat"), int(flat_index0), int(lo), _stream(stream, master)))


def state_blocked_elems(n):
    """Floats in the blocked state array of an n-element slice (STATE_BLOCK-element blocks of
    master, then m, then v)."""
    v = int(lib().state_blocked_elems(int(n)))
    if v < 0:
        raise ValueError(f"slice length {n} out of range")
    return v


def adamw_shard_step_blocked(state, contribs, step, lr, n, beta1=0.9, beta2=0.999, eps=1e-8,
                             weight_decay=0.0, grad_scale=1.0, segs=None, n_segments=0, flat=None,
                             flat_index0=0, lo=0, max_grad_norm=0.0, grad_sumsq=None,
                             stream=None):
    """adamw_shard_step with the state of the n-element slice in the blocked layout."""
    import torch
    n = int(n)
    arr = _contrib_array(contribs, n)
    hp = _hp(step, lr, beta1, beta2, eps, weight_decay, grad_scale, max_grad_norm, grad_sumsq)
    if flat is not None and not isinstance(flat, int):
        _ptr(flat, "flat", _bf16_dtypes(), n + int(lo) - int(flat_index0))
    _check("adamw_shard_step_blocked", lib().adamw_shard_step_blocked(
        _ptr(state, "state", {torch.float32}, state_blocked_elems(n)),
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), n,
        _segs(segs, n_segments), int(n_segments), ctypes.byref(hp),
        _ptr(flat, "flat"), int(flat_index0), int(lo), _stream(stream, state)))


def adamw_shard_step_f32grad_blocked(state, grad, step, lr, n, beta1=0.9, beta2=0.999, eps=1e-8,
                                     weight_decay=0.0, grad_scale=1.0, segs=None, n_segments=0,
                                     flat=None, flat_index0=0, lo=0, max_grad_norm=0.0,
                                     grad_sumsq=None, stream=None):
    """adamw_shard_step_f32grad with the state of the n-element slice in the blocked layout."""
    import torch
    n = int(n)
    hp = _hp(step, lr, beta1, beta2, eps, weight_decay, grad_scale, max_grad_norm, grad_sumsq)
    if flat is not None and not isinstance(flat, int):
        _ptr(flat, "flat", _bf16_dtypes(), n + int(lo) - int(flat_index0))
    _check("adamw_shard_step_f32grad_blocked", lib().adamw_shard_step_f32grad_blocked(
        _ptr(state, "state", {torch.float32}, state_blocked_elems(n)),
        _ptr(grad, "grad", {torch.float32}, n), n, _segs(segs, n_segments), int(n_segments),
        ctypes.byref(hp), _ptr(flat, "flat"), int(flat_index0), int(lo), _stream(stream, state)))


def grads_interleaved_elems(fan_in, n):
    """Elements of the interleaved gradient array of fan_in contributions of an n-element slice
    (STATE_BLOCK-element blocks, one per rank in rank order, block after block)."""
    v = int(lib().grads_interleaved_elems(int(fan_in), int(n)))
    if v < 0:
        raise ValueError(f"fan-in {fan_in} or slice length {n} out of range")
    return v


def adamw_shard_step_interleaved(state, grads, fan_in, step, lr, n, beta1=0.9, beta2=0.999,
                                 eps=1e-8, weight_decay=0.0, grad_scale=1.0, segs=None,
                                 n_segments=0, flat=None, flat_index0=0, lo=0, max_grad_norm=0.0,
                                 grad_sumsq=None, stream=None):
    """adamw_shard_step_blocked fed by the fan_in contributions interleaved in one array
    ``grads`` of grads_interleaved_elems(fan_in, n) bf16 elements."""
    import torch
    n = int(n)
    fan_in = int(fan_in)
    hp = _hp(step, lr, beta1, beta2, eps, weight_decay, grad_scale, max_grad_norm, grad_sumsq)
    if flat is not None and not isinstance(flat, int):
        _ptr(flat, "flat", _bf16_dtypes(), n + int(lo) - int(flat_index0))
    _check("adamw_shard_step_interleaved", lib().adamw_shard_step_interleaved(
        _ptr(state, "state", {torch.float32}, state_blocked_elems(n)),
        _ptr(grads, "grads", _bf16_dtypes(), grads_interleaved_elems(fan_in, n)), fan_in, n,
        _segs(segs, n_segments), int(n_segments), ctypes.byref(hp),
        _ptr(flat, "flat"), int(flat_index0), int(lo), _stream(stream, state)))


def grads_to_interleaved(contribs, grads, n=None, stream=None):
    """Copy the separate contributions (n elements each) into the interleaved array ``grads``."""
    n = contribs[0].numel() if n is None else int(n)
    arr = _contrib_array(contribs, n)
    _check("grads_to_interleaved", lib().grads_to_interleaved(
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), n,
        _ptr(grads, "grads", _bf16_dtypes(), grads_interleaved_elems(len(contribs), n)),
        _stream(stream, grads)))


def state_to_blocked(master, m, v, state, n=None, stream=None):
    """Copy the separate master / m / v arrays of an n-element slice into the blocked array."""
    import torch
    n = master.numel() if n is None else int(n)
    f32 = {torch.float32}
    _check("state_to_blocked", lib().state_to_blocked(
        _ptr(master, "master", f32, n), _ptr(m, "m", f32, n), _ptr(v, "v", f32, n), n,
        _ptr(state, "state", f32, state_blocked_elems(n)), _stream(stream, state)))


def state_from_blocked(state, master, m, v, n=None, stream=None):
    """Copy the blocked array of an n-element slice back into separate master / m / v arrays."""
    import torch
    n = master.numel() if n is None else int(n)
    f32 = {torch.float32}
    _check("state_from_blocked", lib().state_from_blocked(
        _ptr(state, "state", f32, state_blocked_elems(n)), n, _ptr(master, "master", f32, n),
        _ptr(m, "m", f32, n), _ptr(v, "v", f32, n), _stream(stream, state)))


def reduce_shard_accumulate(contribs, acc, scale=1.0, n=None, stream=None):
    """acc[i] += scale * sum over ranks r (in order) of contribs[r][i], in float32."""
    import torch
    n = acc.numel() if n is None else int(n)
    arr = _contrib_array(contribs, n)
    _check("reduce_shard_accumulate", lib().reduce_shard_accumulate(
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), n, float(scale),
        _ptr(acc, "acc", {torch.float32}, n), _stream(stream, acc)))


def reduce_shard_interleaved(grads, fan_in, out, accumulate=False, scale=1.0, n=None,
                             stream=None):
    """reduce_shard (or, with ``accumulate``, reduce_shard_accumulate into ``out``) of fan_in
    contributions held in the interleaved array ``grads``."""
    import torch
    n = out.numel() if n is None else int(n)
    fan_in = int(fan_in)
    _check("reduce_shard_interleaved", lib().reduce_shard_interleaved(
        _ptr(grads, "grads", _bf16_dtypes(), grads_interleaved_elems(fan_in, n)), fan_in, n,
        float(scale), _ptr(out, "out", {torch.float32}, n), 1 if accumulate else 0,
        _stream(stream, out)))


def grad_sumsq_workspace_bytes(n):
    return int(lib().grad_sumsq_workspace_bytes(int(n)))


def grad_sumsq_shard(sumsq, contribs=None, grad=None, n=None, scale=1.0, segs=None,
                     n_segments=0, workspace=None, stream=None):
    """Sum of squares of the slice's reduced gradient (float64, fixed order) into ``sumsq`` (a
    device float64 tensor).  Give either the bf16 ``contribs`` or one fp32 ``grad`` shard.
    ``workspace``: device tensor of at least grad_sumsq_workspace_bytes(n) bytes (allocated here
    through PyTorch when omitted, and then safe to use with any ``stream``)."""
    import torch
    if (contribs is None) == (grad is None):
        raise ValueError("give exactly one of contribs and grad")
    if n is None:
        n = grad.numel() if grad is not None else contribs[0].numel()
    n = int(n)
    need = grad_sumsq_workspace_bytes(n)
    if workspace is None:
        workspace = _call_workspace(need, sumsq.device, stream)
    wbytes = workspace.numel() * workspace.element_size()
    if contribs is not None:
        arr = _contrib_array(contribs, n)
        arr_p, fan_in, gp = ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), None
    else:
        arr_p, fan_in, gp = None, 0, _ptr(grad, "grad", {torch.float32}, n)
    _check("grad_sumsq_shard", lib().grad_sumsq_shard(
        arr_p, fan_in, gp, n, _segs(segs, n_segments), int(n_segments), float(scale),
        _ptr(workspace, "workspace"), wbytes, _ptr(sumsq, "sumsq", {torch.float64}, 1),
        _stream(stream, sumsq)))


def grad_sumsq_shard_interleaved(sumsq, grads, fan_in, n, scale=1.0, segs=None, n_segments=0,
                                 workspace=None, stream=None):
    """grad_sumsq_shard of fan_in contributions held in the interleaved array ``grads``."""
    import torch
    n, fan_in = int(n), int(fan_in)
    need = grad_sumsq_workspace_bytes(n)
    if workspace is None:
        workspace = _call_workspace(need, sumsq.device, stream)
    wbytes = workspace.numel() * workspace.element_size()
    _check("grad_sumsq_shard_interleaved", lib().grad_sumsq_shard_interleaved(
        _ptr(grads, "grads", _bf16_dtypes(), grads_interleaved_elems(fan_in, n)), fan_in, n,
        _segs(segs, n_segments), int(n_segments), float(scale), _ptr(workspace, "workspace"),
        wbytes, _ptr(sumsq, "sumsq", {torch.float64}, 1), _stream(stream, sumsq)))


NOALLOC_MAX_ELEMS = 65536 * 32768


def grad_sumsq_shard_noalloc(sumsq, contribs=None, grad=None, n=None, scale=1.0, segs=None,
                             n_segments=0, stream=None):
    """grad_sumsq_shard without a workspace: the partials go to the library's own per-device
    array (slices up to NOALLOC_MAX_ELEMS elements; calls overlapping on one GPU race)."""
    import torch
    if (contribs is None) == (grad is None):
        raise ValueError("give exactly one of contribs and grad")
    if n is None:
        n = grad.numel() if grad is not None else contribs[0].numel()
    n = int(n)
    if contribs is not None:
        arr = _contrib_array(contribs, n)
        arr_p, fan_in, gp = ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), None
    else:
        arr_p, fan_in, gp = None, 0, _ptr(grad, "grad", {torch.float32}, n)
    _check("grad_sumsq_shard_noalloc", lib().grad_sumsq_shard_noalloc(
        arr_p, fan_in, gp, n, _segs(segs, n_segments), int(n_segments), float(scale),
        _ptr(sumsq, "sumsq", {torch.float64}, 1), _stream(stream, sumsq)))


def reduce_shard_sumsq(contribs, out, sumsq, accumulate=False, scale=1.0, n=None, segs=None,
                       n_segments=0, workspace=None, stream=None):
    """out = scale * sum (or out += scale * sum with ``accumulate``) over the contributions in
    rank order, in float32, and ``sumsq`` (device float64) = sum over real elements of out**2.
    ``workspace``: device tensor of at least grad_sumsq_workspace_bytes(n) bytes (allocated here
    through PyTorch when omitted)."""
    import torch
    n = out.numel() if n is None else int(n)
    need = grad_sumsq_workspace_bytes(n)
    if workspace is None:
        workspace = _call_workspace(need, sumsq.device, stream)
    wbytes = workspace.numel() * workspace.element_size()
    arr = _contrib_array(contribs, n)
    _check("reduce_shard_sumsq", lib().reduce_shard_sumsq(
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), n, float(scale),
        _ptr(out, "out", {torch.float32}, n), 1 if accumulate else 0,
        _segs(segs, n_segments), int(n_segments), _ptr(workspace, "workspace"), wbytes,
        _ptr(sumsq, "sumsq", {torch.float64}, 1), _stream(stream, out)))


def reduce_shard_sumsq_interleaved(grads, fan_in, out, sumsq, accumulate=False, scale=1.0, n=None,
                                   segs=None, n_segments=0, workspace=None, stream=None):
    """reduce_shard_sumsq of fan_in contributions held in the interleaved array ``grads``."""
    import torch
    n = out.numel() if n is None else int(n)
    fan_in = int(fan_in)
    need = grad_sumsq_workspace_bytes(n)
    if workspace is None:
        workspace = _call_workspace(need, sumsq.device, stream)
    wbytes = workspace.numel() * workspace.element_size()
    _check("reduce_shard_sumsq_interleaved", lib().reduce_shard_sumsq_interleaved(
        _ptr(grads, "grads", _bf16_dtypes(), grads_interleaved_elems(fan_in, n)), fan_in, n,
        float(scale), _ptr(out, "out", {torch.float32}, n), 1 if accumulate else 0,
        _segs(segs, n_segments), int(n_segments), _ptr(workspace, "workspace"), wbytes,
        _ptr(sumsq, "sumsq", {torch.float64}, 1), _stream(stream, out)))


def unflatten_bf16(master, flat, flat_index0=0, lo=0, segs=None, n_segments=0, n=None,
                   stream=None):
    """flat[lo + i - flat_index0] = bf16(master[i]) for real elements, +0 for padding."""
    import torch
    n = master.numel() if n is None else int(n)
    if not isinstance(flat, int):
        _ptr(flat, "flat", _bf16_dtypes(), n + int(lo) - int(flat_index0))
    _check("unflatten_bf16", lib().unflatten_bf16(
        _ptr(master, "master", {torch.float32}, n), n, _segs(segs, n_segments), int(n_segments),
        _ptr(flat, "flat"), int(flat_index0), int(lo), _stream(stream, master)))


def stream_copy(src, dst, nbytes=None, stream=None):
    """Measurement aid: plain 16-byte-vector device copy (bandwidth reference)."""
    nbytes = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _need_bytes(src, "src", nbytes)
    _need_bytes(dst, "dst", nbytes)
    _check("fsdpshard_stream_copy", lib().fsdpshard_stream_copy(
        _ptr(src, "src"), _ptr(dst, "dst"), nbytes, _stream(stream, src)))


def stream_rw(srcs, dsts, nbytes, vectors_per_thread=4, threads_per_group=256, per_cu=0,
              xcd_run=0, sink=None, stream=None):
    """Measurement aid: len(srcs) read streams and len(dsts) write streams of ``nbytes`` each in
    one launch shape (pure reads when ``dsts`` is empty; then ``sink`` is a device tensor of at
    least 4 bytes).  A destination that is one of the sources is read and written in place."""
    nbytes = int(nbytes)
    for i, t in enumerate(list(srcs) + list(dsts)):
        _need_bytes(t, f"stream {i}", nbytes)
    _need_bytes(sink, "sink", 4)
    like = next(iter(list(srcs) + list(dsts)), None)
    src_arr = (c_vp * max(1, len(srcs)))(*[_ptr(t, "source") for t in srcs])
    dst_arr = (c_vp * max(1, len(dsts)))(*[_ptr(t, "destination") for t in dsts])
    _check("fsdpshard_stream_rw", lib().fsdpshard_stream_rw(
        ctypes.cast(src_arr, ctypes.POINTER(c_vp)), len(srcs),
        ctypes.cast(dst_arr, ctypes.POINTER(c_vp)), len(dsts), nbytes, int(vectors_per_thread),
        int(threads_per_group), int(per_cu), int(xcd_run), _ptr(sink, "sink"),
        _stream(stream, like)))


def stream_mix(contribs, s0, s1, s2, out, n=None, stream=None):
    """Measurement aid: the fused step's traffic with trivial arithmetic (n a multiple of 8)."""
    n = s0.numel() if n is None else int(n)
    arr = _contrib_array(contribs, n)
    for t, what, b in ((s0, "s0", 4), (s1, "s1", 4), (s2, "s2", 4), (out, "out", 2)):
        _need_bytes(t, what, b * n)
    _check("fsdpshard_stream_mix", lib().fsdpshard_stream_mix(
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), _ptr(s0, "s0"), _ptr(s1, "s1"),
        _ptr(s2, "s2"), _ptr(out, "out"), n, _stream(stream, s0)))


def stream_mix_blocked(contribs, state, out, n, stream=None):
    """Measurement aid: stream_mix for the blocked state layout."""
    n = int(n)
    arr = _contrib_array(contribs, n)
    _need_bytes(state, "state", 4 * state_blocked_elems(n))
    _need_bytes(out, "out", 2 * n)
    _check("fsdpshard_stream_mix_blocked", lib().fsdpshard_stream_mix_blocked(
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), _ptr(state, "state"),
        _ptr(out, "out"), n, _stream(stream, state)))


def stream_mix_interleaved(grads, fan_in, state, out, n, stream=None):
    """Measurement aid: stream_mix_blocked fed by the fan_in contributions interleaved in one
    array ``grads``."""
    n, fan_in = int(n), int(fan_in)
    _need_bytes(grads, "grads", 2 * grads_interleaved_elems(fan_in, n))
    _need_bytes(state, "state", 4 * state_blocked_elems(n))
    _need_bytes(out, "out", 2 * n)
    _check("fsdpshard_stream_mix_interleaved", lib().fsdpshard_stream_mix_interleaved(
        _ptr(grads, "grads"), fan_in, _ptr(state, "state"), _ptr(out, "out"), n,
        _stream(stream, state)))


def stream_mix_shaped(contribs, state, out, n, groups_per_wave, per_cu, xcd_run, phased,
                      stream=None):
    """Measurement aid: stream_mix_blocked's bytes in another launch shape, optionally with each
    work-group's loads and stores in separate phases (see fsdpshard_stream_mix_shaped)."""
    n = int(n)
    arr = _contrib_array(contribs, n)
    _need_bytes(state, "state", 4 * state_blocked_elems(n))
    _need_bytes(out, "out", 2 * n)
    _check("fsdpshard_stream_mix_shaped", lib().fsdpshard_stream_mix_shaped(
        ctypes.cast(arr, ctypes.POINTER(c_vp)), len(contribs), _ptr(state, "state"),
        _ptr(out, "out"), n, int(groups_per_wave), int(per_cu), int(xcd_run),
        1 if phased else 0, _stream(stream, state)))


# ------------------------------------------------------------------------------ reshard

def reshard_plan(numels, src_pad, src_world, dst_pad, dst_world, dst_rank):
    """Pieces (numpy array of PIECE_DTYPE) that build destination rank ``dst_rank``'s shard of the
    (dst_pad, dst_world) layout from the shards of the (src_pad, src_world) layout."""
    sizes = np.ascontiguousarray(np.asarray(numels, dtype=np.int64).reshape(-1))
    T = int(sizes.size)
    sp = sizes.ctypes.data_as(ctypes.POINTER(c_i64)) if T else None
    count = c_i32(0)
    h = lib()
    _check("reshard_plan", h.reshard_plan(sp, T, int(src_pad), int(src_world), int(dst_pad),
                                          int(dst_world), int(dst_rank), None, 0,
                                          ctypes.byref(count)))
    pieces = np.zeros(count.value, dtype=PIECE_DTYPE)
    if count.value:
        _check("reshard_plan", h.reshard_plan(
            sp, T, int(src_pad), int(src_world), int(dst_pad), int(dst_world), int(dst_rank),
            pieces.ctypes.data_as(ctypes.POINTER(_Piece)), count.value, ctypes.byref(count)))
    return pieces


def reshard_copy(src_shards, dst, pieces, stream=None):
    """Execute a reshard plan: ``src_shards`` are the source ranks' device tensors (None for a rank
    no piece reads), ``dst`` the destination shard; all of one dtype (2, 4 or 8 bytes)."""
    like = next(t for t in list(src_shards) + [dst] if t is not None)
    elem = like.element_size()
    for t in list(src_shards) + [dst]:
        if t is not None and t.element_size() != elem:
            raise ValueError("all shards must share one element size")
    n_src = len(src_shards)
    ptrs = (c_vp * n_src)(*[None if t is None else _ptr(t, f"source shard {i}")
                            for i, t in enumerate(src_shards)])
    elems = (c_i64 * n_src)(*[0 if t is None else t.numel() for t in src_shards])
    pieces = np.ascontiguousarray(pieces, dtype=PIECE_DTYPE)
    _check("reshard_copy", lib().reshard_copy(
        ptrs, elems, n_src, _ptr(dst, "dst"), dst.numel(),
        pieces.ctypes.data_as(ctypes.POINTER(_Piece)) if pieces.size else None, int(pieces.size),
        elem, _stream(stream, dst)))
