"""GPU parity of gdn_prefill (chunked, block length 64) against the fp64 oracle,
through the C ABI.

Tolerances (per output tensor, max|x - r| / max|r|): 1e-5 for fp32 inputs,
2e-3 for bf16 inputs.  The 2e-3 bound is checked on fp32-output runs.
bf16-output runs are checked elementwise against 2e-3*max|r| plus half a
bf16 ulp.  (Rounding a perfect result to bf16 alone can exceed 2e-3 relative.)
Final states are fp32 in every case and always take the bound directly.
"""
import os

import numpy as np
import pytest
import torch

from linear_attention_recurrence_rule_amd import gdn, inputs
from oracle import oracle
from tests.gpu_helpers import check_bf16_out, check_bf16_out_blocks, dev, gather_units, host, normwise, normwise_blocks

pytestmark = pytest.mark.gpu


def run_gpu(x, out_dtype, state=True, **kw):
    return gdn.prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                       state_in=dev(x["state_in"]), cu_seqlens=dev(x["cu_seqlens"]),
                       out_dtype=out_dtype, want_state=state, **kw)


def run_oracle(x, **kw):
    return oracle.scan(x["q"], x["k"], x["v"], x["g"], x["beta"], h_k=x["h_k"], h_v=x["h_v"],
                       state_in=x["state_in"], cu_seqlens=x["cu_seqlens"], **kw)


def test_single_head_fp32_workload():
    """T=256, one head, d=64, fp32 everything, zero initial state: 1e-5."""
    w = inputs.WORKLOADS["single_head_t256_d64_f32"]
    x = inputs.workload_inputs(w)
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("single-head fp32: out %.3g state %.3g" % (eo, es))
    assert eo <= 1e-5 and es <= 1e-5


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 257])
@pytest.mark.parametrize("io", [inputs.F32, inputs.BF16])
def test_ragged_lengths_d64(T, io):
    x = inputs.prefill_inputs(seed=T, total_tokens=T, h_k=2, h_v=4, d=64, io_dtype=io, state_std=0.3)
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x)
    tol = 1e-5 if io == inputs.F32 else 2e-3
    assert normwise(host(out), ro) <= tol
    assert normwise(host(st), rs) <= tol


@pytest.mark.parametrize("T", [1, 64, 100, 128, 333])
def test_bf16_d128_lengths(T):
    x = inputs.prefill_inputs(seed=100 + T, total_tokens=T, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16,
                              state_std=0.05)
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("T=%d: out %.3g state %.3g" % (T, eo, es))
    assert eo <= 2e-3 and es <= 2e-3


@pytest.mark.parametrize("h_k,h_v", [(3, 3), (1, 4), (2, 16)])
@pytest.mark.parametrize("d,io", [(128, inputs.BF16), (64, inputs.F32)])
def test_head_ratios(h_k, h_v, d, io):
    """v-heads per k-head of 1, 4 and 8 (the prep loops over a k-head's v-heads; the
    scan maps each v-head to its k-head's key records), packed ragged sequences,
    initial state."""
    x = inputs.prefill_inputs(seed=90 + h_v + d, lengths=[70, 129, 1], h_k=h_k, h_v=h_v, d=d, io_dtype=io,
                              state_std=0.1)
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x)
    tol = 1e-5 if io == inputs.F32 else 2e-3
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("h_k=%d h_v=%d d=%d: out %.3g state %.3g" % (h_k, h_v, d, eo, es))
    assert eo <= tol and es <= tol


def test_many_packed_sequences():
    """600 packed sequences of 0-40 tokens (the block planner walks sequences 256 at a
    time, carrying token and slot offsets across), initial state, against the oracle."""
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 41, 600)
    lens[::37] = 0
    x = inputs.prefill_inputs(seed=6, lengths=lens, h_k=1, h_v=2, d=64, io_dtype=inputs.BF16, state_std=0.1)
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x, threads=16)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("600 sequences: out %.3g state %.3g" % (eo, es))
    assert eo <= 2e-3 and es <= 2e-3
    # zero-length sequences pass their state through unchanged
    zero = np.flatnonzero(lens == 0)
    assert np.array_equal(host(st)[zero], x["state_in"][zero])


@pytest.mark.parametrize("qk_scale", [2.0 ** 16, 2.0 ** -20])
def test_extreme_qk_magnitudes(qk_scale):
    """q and k multiplied by 2^16 (beyond the fp16 range unscaled) or 2^-20 (fp16
    subnormals unscaled), exactly in bf16: the per-token power-of-two scaling keeps the
    matrix-core operands in range, and the normalised result matches the oracle."""
    x = inputs.prefill_inputs(seed=8, lengths=[150, 70], h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.1)
    for n in ("q", "k"):
        x[n] = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x[n]) * np.float32(qk_scale))
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("q, k x %g: out %.3g state %.3g" % (qk_scale, eo, es))
    assert np.isfinite(host(out)).all() and np.isfinite(host(st)).all()
    assert eo <= 2e-3 and es <= 2e-3


@pytest.mark.parametrize("d", [128, 64])
def test_scaled_fp16_operands_over_wide_ranges(d):
    """The bf16 path rounds its matrix-core operands to fp16 after scaling by powers of
    two: keys and queries per token, the state per 32-key block and state row.  Here
    every token's k and q carry their own factor 2^c, c in [-30, 30] (exact in bf16), and
    the initial state's rows and 32-key blocks their own factors 2^a * 2^b, a in
    [-24, 8], b in [-24, 0], with slow gates so that the initial state persists.  Each
    state row is compared with the oracle relative to that row's largest magnitude,
    and each output column (state row) relative to its own largest magnitude."""
    T = 320
    x = inputs.prefill_inputs(seed=41 + d, lengths=[T - 97, 97], h_k=2, h_v=4, d=d, io_dtype=inputs.BF16,
                              state_std=1.0, gate_mean=-7.0)
    rng = np.random.default_rng(42)
    for n in ("q", "k"):
        f = (2.0 ** rng.integers(-30, 31, size=(T, 2, 1))).astype(np.float32)
        x[n] = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x[n]) * f)
    N = 2
    rows = 2.0 ** rng.integers(-24, 9, size=(N, 4, d, 1))
    blocks = np.repeat(2.0 ** rng.integers(-24, 1, size=(N, 4, 1, d // 32)), 32, axis=3)
    x["state_in"] = (x["state_in"] * rows * blocks).astype(np.float32)
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x)
    o, s = host(out), host(st)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    err_rows = np.abs(s - rs).max(axis=3) / np.abs(rs).max(axis=3)       # [N, h_v, d_v]
    err_cols = np.abs(o - ro).max(axis=0) / np.abs(ro).max(axis=0)       # [h_v, d_v]
    print("wide ranges d=%d: worst state row %.3g, worst output column %.3g" % (d, err_rows.max(), err_cols.max()))
    assert err_rows.max() <= 2e-3 and err_cols.max() <= 2e-3


@pytest.mark.parametrize("d,h_k,h_v", [(128, 2, 2), (64, 2, 2), (128, 1, 3), (64, 3, 3)])
def test_odd_head_ratios_bf16(d, h_k, h_v):
    """v-heads per k-head of 1 and 3: the bf16 prepare kernel then takes one v-head per
    item instead of pairs (the pair kernel with NH = 1); outputs and final states
    against the oracle, packed sequences with a ragged tail and an initial state."""
    x = inputs.prefill_inputs(seed=50 + d + h_v, lengths=[130, 64, 7], h_k=h_k, h_v=h_v, d=d,
                              io_dtype=inputs.BF16, state_std=0.2)
    ro, rs = run_oracle(x)
    for od in (inputs.F32, inputs.BF16):
        out, st = run_gpu(x, od)
        if od == inputs.F32:
            assert normwise(host(out), ro) <= 2e-3
        else:
            check_bf16_out(host(out), ro, 2e-3)
        assert normwise(host(st), rs) <= 2e-3


@pytest.mark.parametrize("d,io", [(128, inputs.BF16), (64, inputs.F32)])
def test_extreme_gates(d, io):
    """Gates at their ends, mixed within blocks: no decay (g = 0), near-total forgetting
    (g = -30, a state reset inside a block), beta = 0 (no write) and beta = 1 (full
    overwrite), among ordinary values."""
    x = inputs.prefill_inputs(seed=12 + d, lengths=[200, 65], h_k=2, h_v=4, d=d, io_dtype=io, state_std=0.2)
    rng = np.random.default_rng(13)
    pick = rng.integers(0, 4, x["g"].shape)
    x["g"] = np.where(pick == 0, 0.0, np.where(pick == 1, -30.0, x["g"])).astype(np.float32)
    pick = rng.integers(0, 4, x["beta"].shape)
    x["beta"] = np.where(pick == 0, 0.0, np.where(pick == 1, 1.0, x["beta"])).astype(np.float32)
    tol = 1e-5 if io == inputs.F32 else 2e-3
    ro, rs = run_oracle(x)
    for run in (lambda: run_gpu(x, inputs.F32),
                lambda: gdn.prefill_direct(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                                           state_in=dev(x["state_in"]), cu_seqlens=dev(x["cu_seqlens"]),
                                           out_dtype=inputs.F32)):
        out, st = run()
        eo, es = normwise(host(out), ro), normwise(host(st), rs)
        print("extreme gates d=%d: out %.3g state %.3g" % (d, eo, es))
        assert eo <= tol and es <= tol


def test_large_values_within_contract():
    """Values up to ~2^12 and an initial state of std 100 (inside the documented range of
    |v|, |S| < 2^14): the fp16 operands of the bf16 path keep their relative accuracy."""
    x = inputs.prefill_inputs(seed=14, lengths=[190, 66], h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.1)
    x["v"] = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x["v"]) * np.float32(1000.0))
    x["state_in"] = (x["state_in"] * np.float32(1000.0)).astype(np.float32)
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("large values: out %.3g state %.3g (max |v| %.0f)" % (eo, es, np.abs(inputs.bf16_bits_to_f32(x["v"])).max()))
    assert np.isfinite(host(out)).all() and eo <= 2e-3 and es <= 2e-3


def test_no_tokens_passes_state_through():
    """total_tokens = 0: no output rows, and the final state equals the initial state."""
    x = inputs.prefill_inputs(seed=16, total_tokens=0, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.1)
    out, st = run_gpu(x, inputs.BF16)
    assert out.shape[0] == 0
    assert torch.equal(st, dev(x["state_in"]))


@pytest.mark.parametrize("d,io", [(128, inputs.BF16), (64, inputs.F32)])
@pytest.mark.parametrize("l2norm,scale", [(False, 0.5), (True, 0.125)])
def test_norm_modes_and_query_scale(d, io, l2norm, scale):
    """Without the in-kernel L2 norm (q and k scaled by 1/16, exactly, so the raw
    recurrence stays stable) and with it plus a query scale, against the oracle."""
    x = inputs.prefill_inputs(seed=17 + d, lengths=[140, 33], h_k=2, h_v=4, d=d, io_dtype=io, state_std=0.1)
    if not l2norm:
        for n in ("q", "k"):
            if io == inputs.BF16:
                x[n] = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x[n]) * np.float32(1 / 16))
            else:
                x[n] = (x[n] * np.float32(1 / 16)).astype(np.float32)
    out, st = run_gpu(x, inputs.F32, qk_l2norm=l2norm, scale=scale)
    ro, rs = run_oracle(x, qk_l2norm=l2norm, scale=scale)
    tol = 1e-5 if io == inputs.F32 else 2e-3
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("l2norm=%d scale=%g d=%d: out %.3g state %.3g" % (l2norm, scale, d, eo, es))
    assert eo <= tol and es <= tol


def test_malformed_cu_seqlens_stay_in_bounds():
    """cu_seqlens that decrease, overshoot total_tokens or go negative: the kernels clamp
    them (results are unspecified by contract), so the calls complete, write finite values
    and leave the rest of the GPU state intact."""
    T = 250
    x = inputs.prefill_inputs(seed=18, total_tokens=T, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.1)
    cu = dev(np.array([0, 300, 100, 5000, -7, 250], dtype=np.int32))
    s0 = dev((0.1 * np.random.default_rng(19).standard_normal((5, 4, 128, 128))).astype(np.float32))
    args = (dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]))
    desc5 = gdn.make_desc(num_seqs=5, total_tokens=T, h_k=2, h_v=4, d=128, io_dtype=gdn.GDN_BF16,
                          out_dtype=gdn.GDN_F32)
    ws = torch.full((gdn.gdn_prefill_workspace_bytes(desc5),), 0xAB, dtype=torch.uint8, device=s0.device)
    out, st = gdn.prefill(*args, state_in=s0, cu_seqlens=cu, out_dtype=inputs.F32, workspace=ws)
    assert gdn.prefill_status(desc5, ws) == gdn.GDN_PREFILL_STATUS_CU_SEQLENS_CLAMPED
    # the same call with a well-formed array leaves a clear status word in the same workspace
    gdn.prefill(*args, state_in=s0, cu_seqlens=dev(np.array([0, 50, 50, 120, 200, 250], dtype=np.int32)),
                out_dtype=inputs.F32, workspace=ws)
    assert gdn.prefill_status(desc5, ws) == 0
    out_d, st_d = gdn.prefill_direct(*args, state_in=s0, cu_seqlens=cu, out_dtype=inputs.F32)
    torch.cuda.synchronize()
    for t in (out, st, out_d, st_d):
        assert torch.isfinite(t).all()
    # a well-formed call afterwards still matches the oracle
    good = inputs.prefill_inputs(seed=20, lengths=[100, 150], h_k=2, h_v=4, d=128, io_dtype=inputs.BF16,
                                 state_std=0.1)
    o2, s2 = run_gpu(good, inputs.F32)
    ro, rs = run_oracle(good)
    assert normwise(host(o2), ro) <= 2e-3 and normwise(host(s2), rs) <= 2e-3


def _status_run(x, out_dtype, **kw):
    """Prefill x with a caller workspace; returns (out, state, status word)."""
    T, h_k, d = x["q"].shape
    h_v = x["v"].shape[1]
    N = 1 if x["cu_seqlens"] is None else len(x["cu_seqlens"]) - 1
    desc = gdn.make_desc(num_seqs=N, total_tokens=T, h_k=h_k, h_v=h_v, d=d,
                         io_dtype=gdn.GDN_BF16 if x["q"].dtype == np.uint16 else gdn.GDN_F32,
                         out_dtype=gdn.GDN_BF16 if out_dtype == inputs.BF16 else gdn.GDN_F32)
    ws = torch.full((gdn.gdn_prefill_workspace_bytes(desc),), 0xFF, dtype=torch.uint8, device="cuda")
    out, st = run_gpu(x, out_dtype, workspace=ws, **kw)
    return out, st, gdn.prefill_status(desc, ws)


def test_status_word_clean_run():
    """An ordinary call leaves a zero status word (the word starts as garbage)."""
    x = inputs.prefill_inputs(seed=23, lengths=[100, 1, 190], h_k=2, h_v=4, d=128, io_dtype=inputs.BF16,
                              state_std=0.1)
    _, _, status = _status_run(x, inputs.F32)
    assert status == 0
    x = inputs.prefill_inputs(seed=24, total_tokens=300, h_k=1, h_v=2, d=64, io_dtype=inputs.F32, state_std=0.1)
    _, _, status = _status_run(x, inputs.F32)
    assert status == 0


@pytest.mark.parametrize("what", ["v", "state"])
def test_large_values_are_reported_or_exact(what):
    """Values up to 2^20 or an initial state of size 2^16 go beyond the fp16 range of the
    bf16 path's token contractions.  The call must then either meet the 2e-3 bound or raise
    GDN_PREFILL_STATUS_NONFINITE in the status word, as gdn.h documents.  The fp32 path
    has no such limit: on the same data at d = 64 it meets 1e-5 with a clear status."""
    for d, io in ((128, inputs.BF16), (64, inputs.F32)):
        x = inputs.prefill_inputs(seed=25, total_tokens=200, h_k=2, h_v=4, d=d, io_dtype=io, state_std=0.1)
        if what == "v":
            rng = np.random.default_rng(26)
            big = (2.0 ** rng.integers(12, 21, size=x["v"].shape)).astype(np.float32) * \
                rng.choice([-1.0, 1.0], size=x["v"].shape).astype(np.float32)
            x["v"] = inputs.f32_to_bf16_bits(big) if io == inputs.BF16 else big  # powers of two: exact
        else:
            x["state_in"] = (x["state_in"] * (2.0 ** 16 / 0.1)).astype(np.float32)
        out, st, status = _status_run(x, inputs.F32)
        ro, rs = run_oracle(x)
        if io == inputs.F32:
            assert status == 0
            assert normwise(host(out), ro) <= 1e-5 and normwise(host(st), rs) <= 1e-5
        elif status & gdn.GDN_PREFILL_STATUS_NONFINITE:
            assert not (torch.isfinite(out).all() and torch.isfinite(st).all())
        else:
            assert normwise(host(out), ro) <= 2e-3 and normwise(host(st), rs) <= 2e-3


def test_nonfinite_input_is_reported():
    """A NaN in the input reaches the outputs; the status word says so."""
    x = inputs.prefill_inputs(seed=27, total_tokens=130, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.1)
    x["state_in"][0, 1, 3, 5] = np.nan
    _, _, status = _status_run(x, inputs.BF16)
    assert status == gdn.GDN_PREFILL_STATUS_NONFINITE


@pytest.mark.parametrize("gate_mean", [0.0, -4.0])
def test_fp32_long_sequence(gate_mean):
    """fp32 path over 64 blocks (T = 4096, d = 64): the 1e-5 bound holds along the whole
    block chain, with ordinary gates and with slow ones (alpha ~ 0.98, long memory)."""
    x = inputs.prefill_inputs(seed=21, total_tokens=4096, h_k=1, h_v=2, d=64, io_dtype=inputs.F32, state_std=0.1,
                              gate_mean=gate_mean)
    out, st = run_gpu(x, inputs.F32)
    ro, rs = run_oracle(x)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("fp32 T=4096 gate mean %g: out %.3g state %.3g" % (gate_mean, eo, es))
    assert eo <= 1e-5 and es <= 1e-5


def test_long_prompt_runs_as_segments():
    """A single sequence can run inside gdn_prefill_ex as consecutive segments (explicit
    lengths, or the automatic choice gdn_prefill makes): bit-identical to one pass (also
    without a state output, where the carried state lives in the workspace, and in place),
    and within tolerance of the oracle."""
    x = inputs.prefill_inputs(seed=22, total_tokens=8256, h_k=16, h_v=32, d=128, io_dtype=inputs.BF16,
                              state_std=0.05)
    o1, s1 = run_gpu(x, inputs.BF16, options=gdn.GdnPrefillOptions(0, 0, -1))  # one pass
    for seg in (1024, 4096 + 64):
        o2, s2 = run_gpu(x, inputs.BF16, options=gdn.GdnPrefillOptions(0, 0, seg))
        assert torch.equal(o1, o2) and torch.equal(s1, s2), seg
    o2, s2 = run_gpu(x, inputs.BF16)  # automatic
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o3, _ = run_gpu(x, inputs.BF16, state=False, options=gdn.GdnPrefillOptions(0, 0, 1024))
    assert torch.equal(o3, o1)
    # in place through the C ABI: state_in == state_out
    st = dev(x["state_in"])
    desc = gdn.make_desc(num_seqs=1, total_tokens=x["total_tokens"], h_k=16, h_v=32, d=128, io_dtype=gdn.GDN_BF16,
                         out_dtype=gdn.GDN_BF16)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(desc), dtype=torch.uint8, device=st.device)
    o4 = torch.empty_like(o1)
    gdn.gdn_prefill(desc, dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]), st, o4, st, None, 64,
                    ws, ws.numel())
    torch.cuda.synchronize()
    assert torch.equal(o4, o1) and torch.equal(st, s1)
    ro, rs = run_oracle(x, threads=16)
    check_bf16_out(host(o1), ro, 2e-3)
    assert normwise(host(s1), rs) <= 2e-3


def test_prefill_4k_workload():
    """T=4096, 32 v-heads over 16 q/k heads, d=128, bf16, zero state: full compare."""
    w = inputs.WORKLOADS["prefill_t4096_hv32_hk16_d128"]
    x = inputs.workload_inputs(w)
    ro, rs = run_oracle(x, threads=16)
    out, st = run_gpu(x, inputs.F32)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("4k fp32-out: out %.3g state %.3g" % (eo, es))
    assert eo <= 2e-3 and es <= 2e-3
    out_b, st_b = run_gpu(x, inputs.BF16)
    check_bf16_out(host(out_b), ro, 2e-3)
    assert normwise(host(st_b), rs) <= 2e-3


def test_prefill_4k_long_memory():
    """Slow gates (alpha ~ 0.98): long-range carry across blocks."""
    x = inputs.prefill_inputs(seed=77, total_tokens=4096, h_k=4, h_v=8, d=128, io_dtype=inputs.BF16,
                              state_std=0.02, gate_mean=-4.0)
    ro, rs = run_oracle(x, threads=16)
    out, st = run_gpu(x, inputs.F32)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("4k long-memory: out %.3g state %.3g" % (eo, es))
    assert eo <= 2e-3 and es <= 2e-3


def test_prefill_varlen_workload_full():
    """16 packed sequences, lengths drawn in [256, 16384]: every (sequence, v-head)
    unit, every output and every final state against the oracle."""
    w = inputs.WORKLOADS["varlen_n16_hv32_hk16_d128"]
    x = inputs.workload_inputs(w)
    ro, rs = run_oracle(x, threads=16)
    out, st = run_gpu(x, inputs.F32)
    eo, es = normwise_blocks(out, ro), normwise(host(st), rs)
    print("varlen %d tokens, fp32-out: out %.3g state %.3g" % (w.total_tokens or x["total_tokens"], eo, es))
    assert eo <= 2e-3 and es <= 2e-3
    del out, st
    # bf16 outputs, as the timed configuration writes them
    out_b, st_b = run_gpu(x, inputs.BF16)
    check_bf16_out_blocks(out_b, ro, 2e-3)
    assert normwise(host(st_b), rs) <= 2e-3


def test_prefill_128k_workload_full():
    """T=131072, 32 v-heads over 16 q/k heads, d=128, initial state N(0, 0.02):
    every output of every v-head and the whole final state against the oracle."""
    w = inputs.WORKLOADS["prefill_t131072_hv32_hk16_d128"]
    x = inputs.workload_inputs(w)
    ro, rs = run_oracle(x, threads=16)
    out, st = run_gpu(x, inputs.F32)
    eo, es = normwise_blocks(out, ro), normwise(host(st), rs)
    print("128k fp32-out: out %.3g state %.3g" % (eo, es))
    assert eo <= 2e-3 and es <= 2e-3
    del out, st
    out_b, st_b = run_gpu(x, inputs.BF16)
    check_bf16_out_blocks(out_b, ro, 2e-3)
    assert normwise(host(st_b), rs) <= 2e-3


# ---- row slices of the state ------------------------------------------------------------------

ROW_CASES = [  # (d, io dtype, out dtype, lengths)
    (64, inputs.F32, inputs.F32, [257]),
    (64, inputs.F32, inputs.BF16, [1, 130]),
    (64, inputs.BF16, inputs.F32, [200, 0, 65]),
    (64, inputs.BF16, inputs.BF16, [100, 64, 3]),
    (128, inputs.BF16, inputs.F32, [333]),
    (128, inputs.BF16, inputs.BF16, [64, 190, 1]),
]


@pytest.mark.parametrize("case", range(len(ROW_CASES)))
def test_row_slices_16_and_32_agree(case):
    """The scan splits each state over workgroups of 16 or 32 rows (gdn_prefill_ex's
    scan_rows).  fp32 inputs run the same per-row arithmetic either way, so those results
    agree bitwise.  bf16 inputs take two kernels that sum the key contractions in different
    orders (over the whole key range in one wave with 16 rows, over key halves with 32), so
    those agree to rounding.  Both meet the oracle bound, and the default is 16 rows."""
    d, io, od, lens = ROW_CASES[case]
    x = inputs.prefill_inputs(seed=40 + case, lengths=lens, h_k=2, h_v=4, d=d, io_dtype=io, state_std=0.2)
    res = {rows: run_gpu(x, od, options=gdn.GdnPrefillOptions(rows, 0, 0)) for rows in (16, 32)}
    default = run_gpu(x, od)
    assert torch.equal(res[16][0], default[0]) and torch.equal(res[16][1], default[1])
    if io == inputs.F32:
        assert torch.equal(res[16][0], res[32][0]) and torch.equal(res[16][1], res[32][1])
    ro, rs = run_oracle(x)
    tol = 1e-5 if io == inputs.F32 else 2e-3
    for rows in (16, 32):
        out, st = res[rows]
        if od == inputs.F32:
            assert normwise(host(out), ro) <= tol
        else:
            check_bf16_out(host(out), ro, tol)
        assert normwise(host(st), rs) <= tol


# ---- invariants through the GPU path -------------------------------------------------------

def test_split_run_equals_one_call():
    """Prompt chunking: [0, t) then [t, T) from the handed-off state equals one call."""
    x = inputs.prefill_inputs(seed=3, total_tokens=1000, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16,
                              state_std=0.1)
    out, st = run_gpu(x, inputs.F32)
    t = 448  # block-aligned split keeps the same blocks, so the results match bitwise
    a = {k2: (v2[:t] if isinstance(v2, np.ndarray) and k2 in ("q", "k", "v", "g", "beta") else v2) for k2, v2 in x.items()}
    a["total_tokens"] = t
    o1, s1 = run_gpu(a, inputs.F32)
    b = {k2: (v2[t:] if isinstance(v2, np.ndarray) and k2 in ("q", "k", "v", "g", "beta") else v2) for k2, v2 in x.items()}
    b["total_tokens"] = 1000 - t
    b["state_in"] = host(s1).astype(np.float32)
    o2, s2 = run_gpu(b, inputs.F32)
    assert torch.equal(torch.cat([o1, o2]), out)
    assert torch.equal(s2, st)


def test_varlen_equals_separate_calls_and_zero_length():
    lens = [130, 0, 64, 1, 257]
    x = inputs.prefill_inputs(seed=4, lengths=lens, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16)
    x["state_in"] = (0.1 * np.random.default_rng(0).standard_normal((5, 4, 128, 128))).astype(np.float32)
    out, st = run_gpu(x, inputs.F32)
    cu = x["cu_seqlens"]
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        sub = dict(q=x["q"][sl], k=x["k"][sl], v=x["v"][sl], g=x["g"][sl], beta=x["beta"][sl],
                   state_in=x["state_in"][n:n + 1], cu_seqlens=None)
        if lens[n] == 0:
            assert torch.equal(st[n], dev(x["state_in"][n]))
            continue
        on, sn = run_gpu(sub, inputs.F32)
        assert torch.equal(on, out[sl]), n
        assert torch.equal(sn[0], st[n]), n
    ro, rs = run_oracle(x)
    assert normwise(host(out), ro) <= 2e-3 and normwise(host(st), rs) <= 2e-3


def test_grouped_heads_equal_duplicated_heads():
    x = inputs.prefill_inputs(seed=5, total_tokens=300, h_k=2, h_v=6, d=128, io_dtype=inputs.BF16)
    out, st = run_gpu(x, inputs.BF16)
    y = dict(x)
    y["q"] = np.repeat(x["q"], 3, axis=1)
    y["k"] = np.repeat(x["k"], 3, axis=1)
    y["h_k"] = 6
    out2, st2 = run_gpu(y, inputs.BF16)
    assert torch.equal(out, out2) and torch.equal(st, st2)


def test_deterministic_null_state_and_in_place():
    x = inputs.prefill_inputs(seed=6, total_tokens=500, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16)
    o1, s1 = run_gpu(x, inputs.BF16)
    o2, s2 = run_gpu(x, inputs.BF16)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    y = dict(x)
    y["state_in"] = np.zeros((1, 4, 128, 128), np.float32)
    o3, s3 = run_gpu(y, inputs.BF16)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)
    # in place: state_in is state_out
    st = dev(y["state_in"])
    desc = gdn.make_desc(num_seqs=1, total_tokens=500, h_k=2, h_v=4, d=128, io_dtype=gdn.GDN_BF16,
                         out_dtype=gdn.GDN_BF16)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(desc), dtype=torch.uint8, device=st.device)
    o4 = torch.empty_like(o1)
    gdn.gdn_prefill(desc, dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]), st, o4, st,
                    None, 64, ws, ws.numel())
    assert torch.equal(o4, o1) and torch.equal(st, s1)


def test_beta_zero_and_overwrite_through_gpu():
    d, T = 128, 150
    x = inputs.prefill_inputs(seed=8, total_tokens=T, h_k=1, h_v=1, d=d, io_dtype=inputs.BF16, state_std=0.5)
    x["beta"][:] = 0.0
    out, st = run_gpu(x, inputs.F32)
    cum = np.cumprod(np.exp(x["g"][:, 0].astype(np.float64)))
    np.testing.assert_allclose(host(st)[0, 0], cum[-1] * x["state_in"][0, 0], rtol=1e-5, atol=1e-30)
    # orthogonal keys (Hadamard rows, entries +-1, exact in bf16), normalised in-kernel;
    # alpha = beta = 1: every write overwrites, every read returns the value written
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    order = np.random.default_rng(2).permutation(d)[:100]
    y = inputs.prefill_inputs(seed=9, total_tokens=100, h_k=1, h_v=1, d=d, io_dtype=inputs.BF16)
    y["k"] = inputs.f32_to_bf16_bits(H[order][:, None].astype(np.float32))
    y["q"] = y["k"].copy()
    y["g"][:] = 0.0
    y["beta"][:] = 1.0
    out_b, st_b = run_gpu(y, inputs.F32)
    vb = inputs.bf16_bits_to_f32(y["v"]).astype(np.float64)
    assert normwise(host(out_b)[:, 0], vb[:, 0]) <= 2e-3
    S = host(st_b)[0, 0]
    assert normwise((H[order] / np.sqrt(d)) @ S.T, vb[:, 0]) <= 2e-3


@pytest.mark.parametrize("seg", [256, 320, 2048])
def test_segmented_equals_one_call(seg):
    """gdn_prefill_segmented: segments on block boundaries give the one-call result bit for bit."""
    x = inputs.prefill_inputs(seed=14, total_tokens=1000, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.05)
    out, st = run_gpu(x, inputs.BF16)
    a = [dev(x[n]) for n in ("q", "k", "v", "g", "beta")]
    o2, s2 = gdn.prefill_segmented(*a, segment_tokens=seg, state_in=dev(x["state_in"]), out_dtype=inputs.BF16)
    assert torch.equal(o2, out) and torch.equal(s2, st)
    # no initial state, no final state requested (the carried state lives in the workspace)
    z = dict(x)
    z["state_in"] = None
    o3, _ = run_gpu(z, inputs.BF16, state=False)
    o4, s4 = gdn.prefill_segmented(*a, segment_tokens=seg, out_dtype=inputs.BF16, want_state=False)
    assert s4 is None and torch.equal(o4, o3)


def test_segmented_empty_sequence_passes_state():
    x = inputs.prefill_inputs(seed=15, total_tokens=0, h_k=2, h_v=4, d=64, io_dtype=inputs.BF16, state_std=0.1)
    a = [dev(x[n]) for n in ("q", "k", "v", "g", "beta")]
    o, s = gdn.prefill_segmented(*a, segment_tokens=64, state_in=dev(x["state_in"]))
    assert o.numel() == 0 and torch.equal(s, dev(x["state_in"]))


# ---- two-level scan (one long sequence, few heads) -----------------------------------------

@pytest.mark.parametrize("segments", [2, 5, 64])
def test_two_level_bf16_matches_oracle(segments):
    """gdn_prefill_two_level: segments' transitions and affine parts, composed start
    states, then the scan rerun per segment.  bf16, d = 128, 2381 tokens (37 blocks
    + 13 tokens), a non-zero start state; 64 segments caps at one block each."""
    x = inputs.prefill_inputs(seed=90 + segments, total_tokens=2381, h_k=1, h_v=2, d=128, io_dtype=inputs.BF16,
                              state_std=0.2)
    out, st = gdn.prefill_two_level(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                                    segments=segments, state_in=dev(x["state_in"]), out_dtype=inputs.F32)
    ro, rs = run_oracle(x)
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("two-level %d segments: out %.3g state %.3g" % (segments, eo, es))
    assert eo <= 2e-3 and es <= 2e-3
    # and against the one-level path on the same inputs
    o1, s1 = run_gpu(x, inputs.F32)
    assert normwise(host(out), host(o1)) <= 2e-3 and normwise(host(st), host(s1)) <= 2e-3


def test_two_level_bf16_d64_matches_oracle():
    x = inputs.prefill_inputs(seed=94, total_tokens=777, h_k=2, h_v=4, d=64, io_dtype=inputs.BF16, state_std=0.3)
    out, st = gdn.prefill_two_level(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                                    segments=3, state_in=dev(x["state_in"]), out_dtype=inputs.BF16)
    ro, rs = run_oracle(x)
    check_bf16_out(host(out), ro, 2e-3)
    assert normwise(host(st), rs) <= 2e-3


def test_two_level_fp32_matches_oracle():
    x = inputs.prefill_inputs(seed=95, total_tokens=1000, h_k=1, h_v=2, d=64, io_dtype=inputs.F32, state_std=0.3)
    out, st = gdn.prefill_two_level(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                                    segments=4, state_in=dev(x["state_in"]), out_dtype=inputs.F32)
    ro, rs = run_oracle(x)
    assert normwise(host(out), ro) <= 1e-5 and normwise(host(st), rs) <= 1e-5


@pytest.mark.parametrize("d,io", [(64, inputs.F32), (128, inputs.BF16)])
def test_two_level_extreme_gates(d, io):
    """Two-level scan with no-decay, near-total-forgetting and full-overwrite gates mixed
    in (segment state maps with transition parts near zero)."""
    x = inputs.prefill_inputs(seed=96 + d, total_tokens=900, h_k=1, h_v=2, d=d, io_dtype=io, state_std=0.3)
    rng = np.random.default_rng(97)
    pick = rng.integers(0, 5, x["g"].shape)
    x["g"] = np.where(pick == 0, 0.0, np.where(pick == 1, -30.0, x["g"])).astype(np.float32)
    pick = rng.integers(0, 5, x["beta"].shape)
    x["beta"] = np.where(pick == 0, 1.0, x["beta"]).astype(np.float32)
    out, st = gdn.prefill_two_level(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                                    segments=5, state_in=dev(x["state_in"]), out_dtype=inputs.F32)
    ro, rs = run_oracle(x)
    tol = 1e-5 if io == inputs.F32 else 2e-3
    eo, es = normwise(host(out), ro), normwise(host(st), rs)
    print("two-level extreme gates d=%d: out %.3g state %.3g" % (d, eo, es))
    assert eo <= tol and es <= tol


def test_two_level_one_segment_is_prefill():
    x = inputs.prefill_inputs(seed=96, total_tokens=700, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.1)
    out, st = gdn.prefill_two_level(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                                    segments=1, state_in=dev(x["state_in"]), out_dtype=inputs.BF16)
    o1, s1 = run_gpu(x, inputs.BF16)
    assert torch.equal(out, o1) and torch.equal(st, s1)
