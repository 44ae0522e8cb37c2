"""GPU parity of gdn_prefill_direct (token-by-token prefill, state in registers)
against the fp64 oracle, through the C ABI.

Tolerances as for the other paths, per output tensor (max|x - r| / max|r|):
1e-5 for fp32 inputs, 2e-3 for bf16 inputs on fp32-output runs; bf16-output
runs elementwise within 2e-3*max|r| plus half a bf16 ulp.
"""
import numpy as np
import pytest
import torch

from linear_attention_recurrence_rule_amd import gdn, inputs
from oracle import oracle
from tests.gpu_helpers import check_bf16_out, dev, host, normwise

pytestmark = pytest.mark.gpu


def run_direct(x, out_dtype, **kw):
    return gdn.prefill_direct(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                              state_in=dev(x["state_in"]), cu_seqlens=dev(x["cu_seqlens"]),
                              out_dtype=out_dtype, **kw)


def run_oracle(x, **kw):
    return oracle.scan(x["q"], x["k"], x["v"], x["g"], x["beta"], h_k=x["h_k"], h_v=x["h_v"],
                       state_in=x["state_in"], cu_seqlens=x["cu_seqlens"], **kw)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("io", [inputs.BF16, inputs.F32])
@pytest.mark.parametrize("out_dt", [inputs.F32, inputs.BF16])
def test_direct_varlen_grid(d, io, out_dt):
    lens = [5, 0, 17, 1, 64, 130, 2, 3]  # around and below the four-token input prefetch
    x = inputs.prefill_inputs(seed=40 + d + io, lengths=lens, h_k=2, h_v=4, d=d, io_dtype=io, state_std=0.2)
    out, st = run_direct(x, out_dt)
    ro, rs = run_oracle(x)
    tol = 1e-5 if io == inputs.F32 else 2e-3
    if out_dt == inputs.F32:
        assert normwise(host(out), ro) <= tol, normwise(host(out), ro)
    else:
        check_bf16_out(host(out), ro, tol)
    assert normwise(host(st), rs) <= tol, normwise(host(st), rs)
    # the zero-length sequence passes its state through bit for bit
    assert torch.equal(st[1], dev(x["state_in"][1]))


def test_direct_verify_steps_in_place():
    """64 sequences x 4 tokens (a verify step), 32 v-heads / 16 k-heads, d=128, bf16, state updated in place."""
    N, t = 64, 4
    x = inputs.prefill_inputs(seed=77, lengths=[t] * N, h_k=16, h_v=32, d=128, io_dtype=inputs.BF16,
                              state_std=0.02)
    state = dev(x["state_in"])
    out, st = gdn.prefill_direct(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                                 state_in=state, state_out=state, cu_seqlens=dev(x["cu_seqlens"]),
                                 out_dtype=inputs.F32)
    assert st is state
    ro, rs = run_oracle(x)
    assert normwise(host(out), ro) <= 2e-3
    assert normwise(host(state), rs) <= 2e-3


@pytest.mark.parametrize("io", [inputs.BF16, inputs.F32])
def test_direct_one_token_equals_decode_step(io):
    """One token per sequence, in place: the same arithmetic as gdn_decode_step, bit for bit."""
    N, h_k, h_v, d = 8, 2, 4, 128
    x = inputs.decode_inputs(seed=3, num_seqs=N, steps=1, h_k=h_k, h_v=h_v, d=d, io_dtype=io)
    s_dec = dev(x["state"])
    o_dec = gdn.decode_step(dev(x["q"][0]), dev(x["k"][0]), dev(x["v"][0]), dev(x["g"][0]), dev(x["beta"][0]),
                            s_dec, out_dtype=inputs.F32)
    s_dir = dev(x["state"])
    cu = torch.arange(N + 1, dtype=torch.int32, device=s_dir.device)
    o_dir, _ = gdn.prefill_direct(dev(x["q"][0]), dev(x["k"][0]), dev(x["v"][0]), dev(x["g"][0]),
                                  dev(x["beta"][0]), state_in=s_dir, state_out=s_dir, cu_seqlens=cu,
                                  out_dtype=inputs.F32)
    assert torch.equal(o_dir, o_dec) and torch.equal(s_dir, s_dec)


def test_direct_long_sequence_and_no_norm():
    """T=1000 on 4 v-heads (bf16, d=128); and fp32 inputs at d=128 without the in-kernel norm."""
    x = inputs.prefill_inputs(seed=9, total_tokens=1000, h_k=2, h_v=4, d=128, io_dtype=inputs.BF16,
                              state_std=0.05)
    out, st = run_direct(x, inputs.F32)
    ro, rs = run_oracle(x)
    assert normwise(host(out), ro) <= 2e-3 and normwise(host(st), rs) <= 2e-3
    y = inputs.prefill_inputs(seed=10, total_tokens=90, h_k=1, h_v=2, d=128, io_dtype=inputs.F32, state_std=0.1)
    y["q"] = (0.1 * y["q"]).astype(np.float32)
    y["k"] = (0.1 * y["k"]).astype(np.float32)
    out, st = run_direct(y, inputs.F32, qk_l2norm=False, scale=0.5)
    ro, rs = run_oracle(y, qk_l2norm=False, scale=0.5)
    assert normwise(host(out), ro) <= 1e-5 and normwise(host(st), rs) <= 1e-5


def test_direct_matches_chunked_and_edge_cases():
    x = inputs.prefill_inputs(seed=11, lengths=[70, 3, 129], h_k=2, h_v=4, d=128, io_dtype=inputs.BF16,
                              state_std=0.05)
    o_dir, s_dir = run_direct(x, inputs.F32)
    o_chk, s_chk = gdn.prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]), dev(x["beta"]),
                               state_in=dev(x["state_in"]), cu_seqlens=dev(x["cu_seqlens"]), out_dtype=inputs.F32)
    # two evaluations of the same recurrence: they agree to the bf16-input tolerance
    assert normwise(host(o_dir), host(o_chk)) <= 2e-3 and normwise(host(s_dir), host(s_chk)) <= 2e-3
    # null initial state equals explicit zeros; no state_out requested
    z = dict(x)
    z["state_in"] = None
    o1, s1 = run_direct(z, inputs.BF16)
    z["state_in"] = np.zeros_like(x["state_in"])
    o2, s2 = run_direct(z, inputs.BF16)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o3, s3 = run_direct(z, inputs.BF16, want_state=False)
    assert s3 is None and torch.equal(o3, o1)
    # no tokens at all: the states pass through
    e = inputs.prefill_inputs(seed=12, lengths=[0, 0], h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.1)
    oe, se = run_direct(e, inputs.BF16)
    assert oe.numel() == 0 and torch.equal(se, dev(e["state_in"]))


# ---- gdn_prefill_direct_ex: the decode step's per-token operations, token by token -------------

@pytest.mark.parametrize("fuse", [1, 2, 3])
@pytest.mark.parametrize("d,io,out_dt", [(128, inputs.BF16, inputs.F32), (128, inputs.BF16, inputs.BF16),
                                         (64, inputs.F32, inputs.F32)])
def test_direct_fused_matches_oracle(fuse, d, io, out_dt):
    """Multi-token decode / verify shapes (1, 3, 16 and 40 tokens per sequence) with raw gate
    inputs ~ N(0, 1), the output norm (random channel weights), or both."""
    x = inputs.prefill_inputs(seed=81 + d + fuse, lengths=[1, 3, 16, 40], h_k=2, h_v=4, d=d, io_dtype=io,
                              state_std=0.3)
    rng = np.random.default_rng(90 + fuse)
    if fuse & 1:
        x["g"] = rng.standard_normal(x["g"].shape, dtype=np.float32)
        x["beta"] = rng.standard_normal(x["beta"].shape, dtype=np.float32)
    w = (1.0 + 0.5 * rng.standard_normal(d)).astype(np.float32)
    out, st = run_direct(x, out_dt, raw_gates=bool(fuse & 1), output_norm=bool(fuse & 2), norm_weight=dev(w))
    ro, rs = oracle.scan_ex(x["q"], x["k"], x["v"], x["g"], x["beta"], h_k=x["h_k"], h_v=x["h_v"],
                            state_in=x["state_in"], cu_seqlens=x["cu_seqlens"], raw_gates=bool(fuse & 1),
                            output_norm=bool(fuse & 2), norm_weight=w)
    tol = 2e-3 if io == inputs.BF16 else 1e-5
    if out_dt == inputs.F32:
        assert normwise(host(out), ro) <= tol, normwise(host(out), ro)
    else:
        check_bf16_out(host(out), ro, tol)
    assert normwise(host(st), rs) <= tol


def test_direct_fused_flags_off_and_norm_leave_the_state_bitwise():
    x = inputs.prefill_inputs(seed=95, lengths=[5, 12], h_k=2, h_v=4, d=128, io_dtype=inputs.BF16, state_std=0.3)
    o0, s0 = run_direct(x, inputs.F32)
    d_ = dev
    ref = gdn.gdn_prefill_direct_ex
    desc = gdn.make_desc(num_seqs=2, total_tokens=17, h_k=2, h_v=4, d=128, io_dtype=gdn.GDN_BF16,
                         out_dtype=gdn.GDN_F32)
    q, k, v, g, b = (d_(x[n]) for n in ("q", "k", "v", "g", "beta"))
    s_in, cu = d_(x["state_in"]), d_(x["cu_seqlens"])
    o1, s1 = torch.empty_like(o0), torch.empty_like(s0)
    ref(desc, q, k, v, g, b, s_in, o1, s1, cu, 0, None, 0.0)
    assert torch.equal(o1, o0) and torch.equal(s1, s0)
    o2, s2 = torch.empty_like(o0), torch.empty_like(s0)
    ref(desc, q, k, v, g, b, s_in, o2, s2, cu, gdn.GDN_FUSE_OUTPUT_NORM, None, 1e-6)
    assert torch.equal(s2, s0) and not torch.equal(o2, o0)
