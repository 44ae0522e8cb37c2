"""Python front end of the fp64 CPU oracle for the gated delta rule.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the GPU library and never imports the product package.

The recurrence lives in ``gdn_oracle.c``.  That file cites the layer
description in "Optimizing on-device inference for Apple Silicon" (section
"Qwen creates three distinct workload shapes") and states the recurrence it
evaluates; for it this module only widens the caller's arrays to float64 and
passes pointers.  The two per-token operations beside the decode step (gate
activations and the output normalisation) are plain float64 numpy at the end
of this module.

Parity pins: every function here is checked by ``tests/test_oracle_pins.py``
against closed forms, brute-force matrix products, a hand-worked example and
invariants of the recurrence.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build_lib(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no hand vectorisation)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("GDN_ORACLE_LIB", _LIB)   # tests point this at mutated copies
            if path == _LIB and not os.path.exists(_LIB):
                build_lib()
            lib = ctypes.CDLL(path)
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int32)
            common = [ctypes.c_int32, ctypes.c_int64, ip, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                      dp, dp, dp, dp, dp, dp, dp, dp]
            lib.gdn_oracle_scan.argtypes = common + [ctypes.c_int32]
            lib.gdn_oracle_scan.restype = ctypes.c_int
            lib.gdn_oracle_chunked.argtypes = common + [ctypes.c_int32, ctypes.c_int32]
            lib.gdn_oracle_chunked.restype = ctypes.c_int
            _lib = lib
    return _lib


def widen(x) -> np.ndarray:
    """Exact widening to float64.  uint16 arrays hold bfloat16 bit patterns:
    a bf16 value is the top half of the float32 with the same bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _run(fn_name, q, k, v, g, beta, h_k, h_v, state_in, cu_seqlens, qk_l2norm, scale,
         threads, extra):
    lib = _load()
    q64, k64, v64 = widen(q), widen(k), widen(v)
    g64, b64 = widen(g), widen(beta)
    T = q64.shape[0]
    d_k = q64.shape[-1]
    d_v = v64.shape[-1]
    q64 = np.ascontiguousarray(q64.reshape(T, h_k, d_k))
    k64 = np.ascontiguousarray(k64.reshape(T, h_k, d_k))
    v64 = np.ascontiguousarray(v64.reshape(T, h_v, d_v))
    g64 = np.ascontiguousarray(g64.reshape(T, h_v))
    b64 = np.ascontiguousarray(b64.reshape(T, h_v))
    if cu_seqlens is None:
        N = 1
        cu = None
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    s_in = None if state_in is None else np.ascontiguousarray(widen(state_in).reshape(N, h_v, d_v, d_k))
    out = np.zeros((T, h_v, d_v), dtype=np.float64)
    s_out = np.zeros((N, h_v, d_v, d_k), dtype=np.float64)
    cup = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    rc = getattr(lib, fn_name)(N, T, cup, h_k, h_v, d_k, d_v, int(bool(qk_l2norm)), float(scale),
                               _ptr(q64), _ptr(k64), _ptr(v64), _ptr(g64), _ptr(b64),
                               _ptr(s_in), _ptr(out), _ptr(s_out), *extra, int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (%s rc=%d)" % (fn_name, rc))
    return out, s_out


def scan(q, k, v, g, beta, *, h_k, h_v, state_in=None, cu_seqlens=None, qk_l2norm=True,
         scale=1.0, threads=0):
    """Token-by-token fp64 scan (the definition).  Returns (out, final_state)
    as float64 arrays [T, h_v, d_v] and [N, h_v, d_v, d_k]."""
    return _run("gdn_oracle_scan", q, k, v, g, beta, h_k, h_v, state_in, cu_seqlens,
                qk_l2norm, scale, threads, ())


def chunked(q, k, v, g, beta, *, h_k, h_v, state_in=None, cu_seqlens=None, qk_l2norm=True,
            scale=1.0, chunk=64, threads=0):
    """The blocked fp64 evaluation (same result as ``scan`` in exact arithmetic)."""
    return _run("gdn_oracle_chunked", q, k, v, g, beta, h_k, h_v, state_in, cu_seqlens,
                qk_l2norm, scale, threads, (int(chunk),))


def decode_step(q, k, v, g, beta, state, *, h_k, h_v, qk_l2norm=True, scale=1.0, threads=0):
    """One decode step for N sequences: the scan with exactly one token per
    sequence.  q,k [N,h_k,d]; v [N,h_v,d]; g,beta [N,h_v]; state [N,h_v,d,d]."""
    N = np.asarray(q).shape[0]
    cu = np.arange(N + 1, dtype=np.int32)
    return scan(q, k, v, g, beta, h_k=h_k, h_v=h_v, state_in=state, cu_seqlens=cu,
                qk_l2norm=qk_l2norm, scale=scale, threads=threads)


# ---- the per-token ops beside the decode step --------------------------------------------
# The pages' decode path fuses "the recurrent update with its normalisation"
# (section "Reduce intermediate traffic and state traffic").  Two per-token
# operations sit next to the update.  The activations turn raw gate inputs into
# g and beta: the decode workload draws both raw inputs from N(0, 1) and sets
# g = -softplus(x_g), beta = sigmoid(x_beta).  The normalisation scales each
# head's output o to unit root-mean-square over d_v (with a per-channel weight).


def gate_activations(x_g, x_beta):
    """g = -softplus(x_g) = -log(1 + exp(x_g)), so alpha = exp(g) = 1 / (1 + exp(x_g)),
    and beta = 1 / (1 + exp(-x_beta)); fp64, finite for every finite input
    (softplus(x) = max(x, 0) + log1p(exp(-|x|)); the logistic function is taken on
    exp(-|y|) <= 1)."""
    x = widen(x_g)
    y = widen(x_beta)
    g = -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))
    e = np.exp(-np.abs(y))
    beta = np.where(y >= 0.0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g, beta


def output_rms_norm(o, weight=None, eps=1e-6):
    """Each head's output vector (last axis, d_v) divided by its root-mean-square,
    o / sqrt(mean_j o_j^2 + eps), then multiplied channel-wise by `weight` ([d_v];
    None for ones).  fp64."""
    o = widen(o)
    out = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + float(eps))
    if weight is not None:
        out = out * widen(weight)
    return out


def decode_step_ex(q, k, v, g, beta, state, *, h_k, h_v, raw_gates=False, output_norm=False,
                   norm_weight=None, norm_eps=1e-6, qk_l2norm=True, scale=1.0, threads=0):
    """decode_step with the per-token ops beside it: with raw_gates, `g` and `beta`
    are the raw inputs x_g, x_beta and pass through gate_activations first; with
    output_norm, each head's output passes through output_rms_norm.  The state
    update does not depend on the normalisation."""
    if raw_gates:
        g, beta = gate_activations(g, beta)
    o, s = decode_step(q, k, v, g, beta, state, h_k=h_k, h_v=h_v, qk_l2norm=qk_l2norm, scale=scale,
                       threads=threads)
    if output_norm:
        o = output_rms_norm(o, norm_weight, norm_eps)
    return o, s


def scan_ex(q, k, v, g, beta, *, h_k, h_v, state_in=None, cu_seqlens=None, raw_gates=False, output_norm=False,
            norm_weight=None, norm_eps=1e-6, qk_l2norm=True, scale=1.0, threads=0):
    """scan with the same per-token operations as decode_step_ex, token by token."""
    if raw_gates:
        g, beta = gate_activations(g, beta)
    o, s = scan(q, k, v, g, beta, h_k=h_k, h_v=h_v, state_in=state_in, cu_seqlens=cu_seqlens,
                qk_l2norm=qk_l2norm, scale=scale, threads=threads)
    if output_norm:
        o = output_rms_norm(o, norm_weight, norm_eps)
    return o, s
