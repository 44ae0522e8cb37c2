"""Thin Python binding over libgdn.so (C ABI in include/gdn.h).

Argument marshalling only: every step of the recurrence runs in the HIP
kernels behind the C entry points.  PyTorch supplies device memory and the
current stream.  The functions named like the C entry points
(``gdn_prefill``, ``gdn_prefill_direct``, ``gdn_decode_step``, ...) take the
same arguments, with torch tensors in place of raw pointers.  ``prefill``,
``prefill_direct`` and ``decode_step`` also allocate the outputs.

There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gdn.h")

GDN_OK, GDN_ERR_INVALID_ARGUMENT, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = range(5)
GDN_F32, GDN_BF16 = 0, 1
CHUNK = 64


class GdnDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int64),
                ("h_k", ctypes.c_int32), ("h_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("qk_l2norm", ctypes.c_int32), ("scale", ctypes.c_float)]


class GdnPrefillOptions(ctypes.Structure):
    _fields_ = [("scan_rows", ctypes.c_int32), ("reserved", ctypes.c_int32), ("segment_tokens", ctypes.c_int64)]


# bits of the prefill status word (gdn_prefill_status_offset)
GDN_PREFILL_STATUS_CU_SEQLENS_CLAMPED = 1
GDN_PREFILL_STATUS_NONFINITE = 2


class GdnError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__("%s: %s" % (status_str(status), detail))


_lock = threading.Lock()
_lib = None


def declared_functions():
    """Names of the functions include/gdn.h declares."""
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gdn_[a-z_0-9]+)\s*\(", src, re.M)))


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libgdn.so is not built (run __graft_entry__.build() or "
                                   "python -m linear_attention_recurrence_rule_amd.build)")
            L = ctypes.CDLL(LIB_PATH)
            vp, sz = ctypes.c_void_p, ctypes.c_size_t
            dp = ctypes.POINTER(GdnDesc)
            L.gdn_prefill_workspace_bytes.argtypes = [dp, ctypes.c_int32]
            L.gdn_prefill_workspace_bytes.restype = sz
            L.gdn_prefill.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, sz, vp]
            L.gdn_prefill.restype = ctypes.c_int
            L.gdn_prefill_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                         ctypes.POINTER(GdnPrefillOptions), vp, sz, vp]
            L.gdn_prefill_ex.restype = ctypes.c_int
            L.gdn_prefill_status_offset.argtypes = [dp, ctypes.c_int32]
            L.gdn_prefill_status_offset.restype = sz
            L.gdn_prefill_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp]
            L.gdn_prefill_noalloc.restype = ctypes.c_int
            L.gdn_prefill_prepare.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, sz, vp]
            L.gdn_prefill_prepare.restype = ctypes.c_int
            L.gdn_prefill_scan.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, sz, vp]
            L.gdn_prefill_scan.restype = ctypes.c_int
            L.gdn_prefill_segmented_workspace_bytes.argtypes = [dp, ctypes.c_int32, ctypes.c_int64]
            L.gdn_prefill_segmented_workspace_bytes.restype = sz
            L.gdn_prefill_segmented.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int64,
                                                vp, sz, vp]
            L.gdn_prefill_segmented.restype = ctypes.c_int
            L.gdn_prefill_two_level_workspace_bytes.argtypes = [dp, ctypes.c_int32, ctypes.c_int32]
            L.gdn_prefill_two_level_workspace_bytes.restype = sz
            L.gdn_prefill_two_level.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32,
                                                vp, sz, vp]
            L.gdn_prefill_two_level.restype = ctypes.c_int
            L.gdn_prefill_direct.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            L.gdn_prefill_direct.restype = ctypes.c_int
            L.gdn_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp]
            L.gdn_decode_step.restype = ctypes.c_int
            L.gdn_decode_step_slots.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp]
            L.gdn_decode_step_slots.restype = ctypes.c_int
            L.gdn_decode_step_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, ctypes.c_float, vp]
            L.gdn_decode_step_ex.restype = ctypes.c_int
            L.gdn_prefill_direct_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp,
                                                ctypes.c_float, vp]
            L.gdn_prefill_direct_ex.restype = ctypes.c_int
            L.gdn_status_str.argtypes = [ctypes.c_int]
            L.gdn_status_str.restype = ctypes.c_char_p
            L.gdn_last_error.argtypes = []
            L.gdn_last_error.restype = ctypes.c_char_p
            _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().gdn_status_str(int(status)).decode()


def last_error() -> str:
    return lib().gdn_last_error().decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != GDN_OK:
        raise GdnError(status, last_error())


def make_desc(*, num_seqs, total_tokens, h_k, h_v, d, io_dtype, out_dtype, qk_l2norm=True, scale=1.0):
    return GdnDesc(int(num_seqs), int(total_tokens), int(h_k), int(h_v), int(d), int(d),
                   int(io_dtype), int(out_dtype), int(bool(qk_l2norm)), float(scale))


# ---- entry points with the C names -------------------------------------------------------

def gdn_prefill_workspace_bytes(desc: GdnDesc, chunk: int = CHUNK) -> int:
    n = lib().gdn_prefill_workspace_bytes(ctypes.byref(desc), int(chunk))
    if n == 0 and desc.total_tokens > 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, last_error())
    return n


def gdn_prefill(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, chunk, workspace,
                workspace_bytes, stream=None):
    _check(lib().gdn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(cu_seqlens), int(chunk),
                             _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gdn_prefill_ex(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, chunk, options, workspace,
                   workspace_bytes, stream=None):
    """options: a GdnPrefillOptions, or None for the defaults (then this is gdn_prefill)."""
    opt = ctypes.byref(options) if options is not None else None
    _check(lib().gdn_prefill_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(cu_seqlens), int(chunk), opt,
                                _ptr(workspace), int(workspace_bytes), _stream(stream)))


GDN_PREFILL_NOALLOC_WORKSPACE_BYTES = 64 << 20


def gdn_prefill_noalloc(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, chunk, stream=None):
    """gdn_prefill with the library's static workspace (no allocation anywhere)."""
    _check(lib().gdn_prefill_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(cu_seqlens), int(chunk),
                                     _stream(stream)))


def gdn_prefill_status_offset(desc: GdnDesc, chunk: int = CHUNK) -> int:
    n = lib().gdn_prefill_status_offset(ctypes.byref(desc), int(chunk))
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, last_error())
    return n


def prefill_status(desc: GdnDesc, workspace: torch.Tensor, chunk: int = CHUNK) -> int:
    """The status word a prefill call left in `workspace` (a uint8 device tensor).  Reads it
    with a device-to-host copy, which waits for the current stream."""
    off = gdn_prefill_status_offset(desc, chunk)
    return int(workspace[off:off + 4].cpu().view(torch.int32).item()) & 0xFFFFFFFF


def gdn_prefill_prepare(desc, q, k, v, g, beta, cu_seqlens, chunk, workspace, workspace_bytes,
                        stream=None):
    _check(lib().gdn_prefill_prepare(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(cu_seqlens), int(chunk), _ptr(workspace), int(workspace_bytes),
                                     _stream(stream)))


def gdn_prefill_scan(desc, q, k, v, state_in, out, state_out, cu_seqlens, chunk, workspace, workspace_bytes,
                     stream=None):
    _check(lib().gdn_prefill_scan(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(state_in), _ptr(out),
                                  _ptr(state_out), _ptr(cu_seqlens), int(chunk), _ptr(workspace),
                                  int(workspace_bytes), _stream(stream)))


def gdn_prefill_segmented_workspace_bytes(desc: GdnDesc, segment_tokens: int, chunk: int = CHUNK) -> int:
    n = lib().gdn_prefill_segmented_workspace_bytes(ctypes.byref(desc), int(chunk), int(segment_tokens))
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, last_error())
    return n


def gdn_prefill_segmented(desc, q, k, v, g, beta, state_in, out, state_out, chunk, segment_tokens, workspace,
                          workspace_bytes, stream=None):
    _check(lib().gdn_prefill_segmented(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(state_in), _ptr(out), _ptr(state_out), int(chunk), int(segment_tokens),
                                       _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gdn_prefill_two_level_workspace_bytes(desc: GdnDesc, segments: int, chunk: int = CHUNK) -> int:
    n = lib().gdn_prefill_two_level_workspace_bytes(ctypes.byref(desc), int(chunk), int(segments))
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, last_error())
    return n


def gdn_prefill_two_level(desc, q, k, v, g, beta, state_in, out, state_out, chunk, segments, workspace,
                          workspace_bytes, stream=None):
    _check(lib().gdn_prefill_two_level(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(state_in), _ptr(out), _ptr(state_out), int(chunk), int(segments),
                                       _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gdn_prefill_direct(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, stream=None):
    _check(lib().gdn_prefill_direct(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(cu_seqlens),
                                    _stream(stream)))


def gdn_decode_step(desc, q, k, v, g, beta, state, out, stream=None):
    _check(lib().gdn_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(state), _ptr(out), _stream(stream)))


GDN_FUSE_GATE_ACTIVATIONS = 1
GDN_FUSE_OUTPUT_NORM = 2
GDN_STREAM_STATE = 4


def gdn_prefill_direct_ex(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, fuse, norm_weight,
                          norm_eps, stream=None):
    _check(lib().gdn_prefill_direct_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(cu_seqlens), int(fuse),
                                       _ptr(norm_weight), float(norm_eps), _stream(stream)))


def gdn_decode_step_ex(desc, q, k, v, g, beta, state, out, fuse, norm_weight, norm_eps, stream=None):
    _check(lib().gdn_decode_step_ex(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state), _ptr(out), int(fuse), _ptr(norm_weight), float(norm_eps),
                                    _stream(stream)))


def gdn_decode_step_slots(desc, q, k, v, g, beta, state_pool, num_slots, state_slots, out, stream=None):
    _check(lib().gdn_decode_step_slots(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(state_pool), int(num_slots), _ptr(state_slots), _ptr(out),
                                       _stream(stream)))


# ---- allocating wrappers ---------------------------------------------------------------

_TORCH_DT = {GDN_F32: torch.float32, GDN_BF16: torch.bfloat16}


def _io_dtype(t):
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32 (got %s)" % t.dtype)


def _need(t, name, dtype=None, device=None):
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s" % (name, device))


def prefill(q, k, v, g, beta, *, state_in=None, cu_seqlens=None, out_dtype=None, qk_l2norm=True,
            scale=1.0, want_state=True, workspace=None, stream=None, options=None):
    """q, k [T, h_k, d]; v [T, h_v, d]; g, beta [T, h_v] fp32; state_in [N, h_v, d, d] fp32 or
    None; cu_seqlens int32 [N+1] or None; options a GdnPrefillOptions (gdn_prefill_ex) or None.
    Returns (out [T, h_v, d], state_out or None)."""
    dev = q.device
    io = _io_dtype(q)
    T, h_k, d = q.shape
    h_v = v.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    N = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, dev)
    od = io if out_dtype is None else out_dtype
    desc = make_desc(num_seqs=N, total_tokens=T, h_k=h_k, h_v=h_v, d=d, io_dtype=io, out_dtype=od,
                     qk_l2norm=qk_l2norm, scale=scale)
    out = torch.empty((T, h_v, d), dtype=_TORCH_DT[od], device=dev)
    state_out = torch.empty((N, h_v, d, d), dtype=torch.float32, device=dev) if want_state else None
    nbytes = gdn_prefill_workspace_bytes(desc)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if options is None:
        gdn_prefill(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, CHUNK, workspace,
                    workspace.numel(), stream)
    else:
        gdn_prefill_ex(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, CHUNK, options, workspace,
                       workspace.numel(), stream)
    return out, state_out


def prefill_segmented(q, k, v, g, beta, *, segment_tokens, state_in=None, out_dtype=None, qk_l2norm=True,
                      scale=1.0, want_state=True, stream=None):
    """One long sequence in segments of ``segment_tokens`` (gdn_prefill_segmented); the workspace
    covers one segment.  Returns (out, state_out or None), bit for bit those of ``prefill``."""
    dev = q.device
    io = _io_dtype(q)
    T, h_k, d = q.shape
    h_v = v.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, dev)
    od = io if out_dtype is None else out_dtype
    desc = make_desc(num_seqs=1, total_tokens=T, h_k=h_k, h_v=h_v, d=d, io_dtype=io, out_dtype=od,
                     qk_l2norm=qk_l2norm, scale=scale)
    out = torch.empty((T, h_v, d), dtype=_TORCH_DT[od], device=dev)
    state_out = torch.empty((1, h_v, d, d), dtype=torch.float32, device=dev) if want_state else None
    nbytes = gdn_prefill_segmented_workspace_bytes(desc, segment_tokens)
    workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    gdn_prefill_segmented(desc, q, k, v, g, beta, state_in, out, state_out, CHUNK, segment_tokens, workspace,
                          nbytes, stream)
    return out, state_out


def prefill_two_level(q, k, v, g, beta, *, segments, state_in=None, out_dtype=None, qk_l2norm=True, scale=1.0,
                      want_state=True, stream=None):
    """One long sequence by the two-level scan (gdn_prefill_two_level) with ``segments``
    segments.  Returns (out, state_out or None)."""
    dev = q.device
    io = _io_dtype(q)
    T, h_k, d = q.shape
    h_v = v.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, dev)
    od = io if out_dtype is None else out_dtype
    desc = make_desc(num_seqs=1, total_tokens=T, h_k=h_k, h_v=h_v, d=d, io_dtype=io, out_dtype=od,
                     qk_l2norm=qk_l2norm, scale=scale)
    out = torch.empty((T, h_v, d), dtype=_TORCH_DT[od], device=dev)
    state_out = torch.empty((1, h_v, d, d), dtype=torch.float32, device=dev) if want_state else None
    nbytes = gdn_prefill_two_level_workspace_bytes(desc, segments)
    workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    gdn_prefill_two_level(desc, q, k, v, g, beta, state_in, out, state_out, CHUNK, segments, workspace, nbytes,
                          stream)
    return out, state_out


def prefill_direct(q, k, v, g, beta, *, state_in=None, state_out=None, cu_seqlens=None, out_dtype=None,
                   qk_l2norm=True, scale=1.0, want_state=True, raw_gates=False, output_norm=False,
                   norm_weight=None, norm_eps=1e-6, stream=None):
    """Token-by-token prefill (gdn_prefill_direct).  Same arguments as ``prefill``; pass
    ``state_out=state_in`` to update the states in place.  raw_gates and output_norm fold in
    the per-token operations of decode_step_fused (through gdn_prefill_direct_ex).
    Returns (out, state_out or None)."""
    dev = q.device
    io = _io_dtype(q)
    T, h_k, d = q.shape
    h_v = v.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    N = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, dev)
    od = io if out_dtype is None else out_dtype
    desc = make_desc(num_seqs=N, total_tokens=T, h_k=h_k, h_v=h_v, d=d, io_dtype=io, out_dtype=od,
                     qk_l2norm=qk_l2norm, scale=scale)
    out = torch.empty((T, h_v, d), dtype=_TORCH_DT[od], device=dev)
    if state_out is None and want_state:
        state_out = torch.empty((N, h_v, d, d), dtype=torch.float32, device=dev)
    fuse = (GDN_FUSE_GATE_ACTIVATIONS if raw_gates else 0) | (GDN_FUSE_OUTPUT_NORM if output_norm else 0)
    if fuse:
        if norm_weight is not None:
            _need(norm_weight, "norm_weight", torch.float32, dev)
            if norm_weight.numel() != d:
                raise ValueError("norm_weight must hold d = %d values (got %d)" % (d, norm_weight.numel()))
        gdn_prefill_direct_ex(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, fuse, norm_weight,
                              norm_eps, stream)
    else:
        gdn_prefill_direct(desc, q, k, v, g, beta, state_in, out, state_out, cu_seqlens, stream)
    return out, state_out


def decode_step(q, k, v, g, beta, state, *, out=None, out_dtype=None, qk_l2norm=True, scale=1.0,
                stream_state=False, stream=None):
    """One token per sequence: q, k [N, h_k, d]; v [N, h_v, d]; g, beta [N, h_v];
    state [N, h_v, d, d] fp32, updated in place.  Returns out [N, h_v, d].
    stream_state: nontemporal state accesses (GDN_STREAM_STATE), same results."""
    dev = q.device
    io = _io_dtype(q)
    N, h_k, d = q.shape
    h_v = v.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    od = io if out_dtype is None else out_dtype
    desc = make_desc(num_seqs=N, total_tokens=N, h_k=h_k, h_v=h_v, d=d, io_dtype=io, out_dtype=od,
                     qk_l2norm=qk_l2norm, scale=scale)
    if out is None:
        out = torch.empty((N, h_v, d), dtype=_TORCH_DT[od], device=dev)
    if stream_state:
        gdn_decode_step_ex(desc, q, k, v, g, beta, state, out, GDN_STREAM_STATE, None, 0.0, stream)
    else:
        gdn_decode_step(desc, q, k, v, g, beta, state, out, stream)
    return out


def decode_step_fused(q, k, v, g, beta, state, *, raw_gates=True, output_norm=True, norm_weight=None,
                      norm_eps=1e-6, out=None, out_dtype=None, qk_l2norm=True, scale=1.0, stream_state=False,
                      stream=None):
    """decode_step with the per-token operations beside it folded in: with
    raw_gates, g and beta are the raw inputs x_g, x_beta (alpha = 1 / (1 + e^x_g),
    beta = 1 / (1 + e^-x_beta)); with output_norm, each head's output is divided by
    its root-mean-square over d (plus norm_eps inside the root) and multiplied by
    norm_weight ([d] fp32, None for ones).  state is updated in place; stream_state as in
    decode_step."""
    dev = q.device
    io = _io_dtype(q)
    N, h_k, d = q.shape
    h_v = v.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", torch.float32, dev)
        if norm_weight.numel() != d:
            raise ValueError("norm_weight must hold d = %d values (got %d)" % (d, norm_weight.numel()))
    od = io if out_dtype is None else out_dtype
    desc = make_desc(num_seqs=N, total_tokens=N, h_k=h_k, h_v=h_v, d=d, io_dtype=io, out_dtype=od,
                     qk_l2norm=qk_l2norm, scale=scale)
    if out is None:
        out = torch.empty((N, h_v, d), dtype=_TORCH_DT[od], device=dev)
    fuse = ((GDN_FUSE_GATE_ACTIVATIONS if raw_gates else 0) | (GDN_FUSE_OUTPUT_NORM if output_norm else 0)
            | (GDN_STREAM_STATE if stream_state else 0))
    gdn_decode_step_ex(desc, q, k, v, g, beta, state, out, fuse, norm_weight, norm_eps, stream)
    return out


def decode_step_slots(q, k, v, g, beta, state_pool, state_slots, *, out=None, out_dtype=None, qk_l2norm=True,
                      scale=1.0, stream=None):
    """decode_step over a state pool: sequence n updates state_pool[state_slots[n]]
    in place.  state_pool [num_slots, h_v, d, d] fp32; state_slots [N] int32 on the
    device.  A slot outside [0, num_slots) skips the sequence (zero output rows)."""
    dev = q.device
    io = _io_dtype(q)
    N, h_k, d = q.shape
    h_v = v.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(state_pool, "state_pool", torch.float32, dev)
    _need(state_slots, "state_slots", torch.int32, dev)
    od = io if out_dtype is None else out_dtype
    desc = make_desc(num_seqs=N, total_tokens=N, h_k=h_k, h_v=h_v, d=d, io_dtype=io, out_dtype=od,
                     qk_l2norm=qk_l2norm, scale=scale)
    if out is None:
        out = torch.empty((N, h_v, d), dtype=_TORCH_DT[od], device=dev)
    gdn_decode_step_slots(desc, q, k, v, g, beta, state_pool, state_pool.shape[0], state_slots, out, stream)
    return out
