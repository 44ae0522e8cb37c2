"""Seeded synthetic inputs for the gated delta rule.

This module only draws random numbers and lays them out.  It holds none of the
recurrence's arithmetic, and it is the one module that both the GPU path's
tests/benchmark and the CPU oracle's callers share.

Recipe (the same for every workload):
  * raw q, k, v ~ N(0, 1), drawn in float32 and rounded to the io dtype
    (bfloat16 by round-to-nearest-even, or kept as float32);
  * x_g, x_b ~ N(0, 1);  g = -softplus(x_g) (so alpha = exp(g) = sigmoid(-x_g));
    beta = sigmoid(x_b); both stored as float32;
  * initial state ~ N(0, std) as float32 where a workload asks for one.
Draw order: sequence lengths (varlen only), then q, k, v, x_g, x_b, state.
The generator is NumPy's PCG64 ``default_rng(seed)``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F32 = 0
BF16 = 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even).  Returns uint16 bit
    patterns.  NaN is not expected in generated data."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    seed: int
    num_seqs: int
    h_k: int
    h_v: int
    d: int
    io_dtype: int
    out_dtype: int
    total_tokens: int = 0          # prefill, fixed-length
    varlen: tuple = ()             # (low, high, count) for drawn lengths
    state_std: float = 0.0         # 0 => no initial state (zeros)
    steps: int = 0                 # decode
    chunk: int = 64
    gate_mean: float = 0.0         # mean of x_g (0 => alpha averages 0.5)


WORKLOADS = {
    w.name: w for w in [
        Workload("single_head_t256_d64_f32", "prefill", 0, 1, 1, 1, 64, F32, F32,
                 total_tokens=256),
        Workload("prefill_t4096_hv32_hk16_d128", "prefill", 1, 1, 16, 32, 128, BF16, BF16,
                 total_tokens=4096),
        Workload("prefill_t131072_hv32_hk16_d128", "prefill", 2, 1, 16, 32, 128, BF16, BF16,
                 total_tokens=131072, state_std=0.02),
        Workload("decode_n64_hv32_hk16_d128_512steps", "decode", 3, 64, 16, 32, 128, BF16, BF16,
                 state_std=0.02, steps=512),
        Workload("varlen_n16_hv32_hk16_d128", "prefill", 4, 16, 16, 32, 128, BF16, BF16,
                 varlen=(256, 16384, 16)),
    ]
}


def _qkv(rng, shape_qk, shape_v, io_dtype):
    q = rng.standard_normal(shape_qk, dtype=np.float32)
    k = rng.standard_normal(shape_qk, dtype=np.float32)
    v = rng.standard_normal(shape_v, dtype=np.float32)
    if io_dtype == BF16:
        return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return q, k, v


def _gates(rng, shape, gate_mean):
    """g and beta (float32), and the raw inputs x_g, x_b they come from (float32)."""
    xg = rng.standard_normal(shape, dtype=np.float32).astype(np.float64) + gate_mean
    xb = rng.standard_normal(shape, dtype=np.float32).astype(np.float64)
    return ((-_softplus(xg)).astype(np.float32), _sigmoid(xb).astype(np.float32),
            xg.astype(np.float32), xb.astype(np.float32))


def prefill_inputs(*, seed, total_tokens=None, lengths=None, h_k, h_v, d, io_dtype,
                   state_std=0.0, gate_mean=0.0, varlen=None):
    """Packed prefill inputs.  Give either ``total_tokens`` (one sequence),
    ``lengths`` (explicit per-sequence lengths) or ``varlen=(lo, hi, n)``
    (lengths drawn uniformly in [lo, hi] before anything else)."""
    rng = np.random.default_rng(seed)
    if varlen:
        lo, hi, n = varlen
        lengths = rng.integers(lo, hi + 1, n)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        T = int(cu[-1])
        N = len(lengths)
    else:
        T = int(total_tokens)
        cu = None
        N = 1
    q, k, v = _qkv(rng, (T, h_k, d), (T, h_v, d), io_dtype)
    g, beta, _, _ = _gates(rng, (T, h_v), gate_mean)
    s0 = None
    if state_std > 0:
        s0 = (state_std * rng.standard_normal((N, h_v, d, d), dtype=np.float32)).astype(np.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state_in=s0, cu_seqlens=cu,
                num_seqs=N, total_tokens=T, h_k=h_k, h_v=h_v, d=d, io_dtype=io_dtype)


def decode_inputs(*, seed, num_seqs, steps, h_k, h_v, d, io_dtype, state_std=0.02,
                  gate_mean=0.0):
    """``steps`` fresh tokens per sequence, pre-drawn: q,k [steps,N,h_k,d],
    v [steps,N,h_v,d], g,beta [steps,N,h_v], initial state [N,h_v,d,d]; also the
    raw gate inputs x_g, x_beta [steps,N,h_v] that g and beta come from."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, (steps, num_seqs, h_k, d), (steps, num_seqs, h_v, d), io_dtype)
    g, beta, x_g, x_b = _gates(rng, (steps, num_seqs, h_v), gate_mean)
    s0 = (state_std * rng.standard_normal((num_seqs, h_v, d, d), dtype=np.float32)).astype(np.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, x_g=x_g, x_beta=x_b, state=s0, num_seqs=num_seqs, steps=steps,
                h_k=h_k, h_v=h_v, d=d, io_dtype=io_dtype)


def workload_inputs(w: Workload, **over):
    if w.kind == "decode":
        kw = dict(seed=w.seed, num_seqs=w.num_seqs, steps=w.steps, h_k=w.h_k, h_v=w.h_v,
                  d=w.d, io_dtype=w.io_dtype, state_std=w.state_std, gate_mean=w.gate_mean)
        kw.update(over)
        return decode_inputs(**kw)
    kw = dict(seed=w.seed, h_k=w.h_k, h_v=w.h_v, d=w.d, io_dtype=w.io_dtype,
              state_std=w.state_std, gate_mean=w.gate_mean)
    if w.varlen:
        kw["varlen"] = w.varlen
    else:
        kw["total_tokens"] = w.total_tokens
    kw.update(over)
    return prefill_inputs(**kw)
