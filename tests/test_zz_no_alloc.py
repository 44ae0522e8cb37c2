"""gdn_prefill_noalloc (the prefill on the library's static workspace) against
gdn_prefill with an allocated workspace: bit-identical outputs and states, on two
calls in a row, the second smaller than the first; and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

from linear_attention_recurrence_rule_amd import gdn, inputs
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _desc(x, out_dtype):
    N = 1 if x["cu_seqlens"] is None else len(x["cu_seqlens"]) - 1
    return gdn.make_desc(num_seqs=N, total_tokens=x["total_tokens"], h_k=x["h_k"], h_v=x["h_v"], d=x["d"],
                         io_dtype=gdn.GDN_BF16 if x["io_dtype"] == inputs.BF16 else gdn.GDN_F32,
                         out_dtype=gdn.GDN_BF16 if out_dtype == inputs.BF16 else gdn.GDN_F32)


def _both(x, out_dtype):
    """(noalloc out, noalloc state), (gdn_prefill out, gdn_prefill state) on the same inputs."""
    desc = _desc(x, out_dtype)
    assert gdn.gdn_prefill_workspace_bytes(desc) <= gdn.GDN_PREFILL_NOALLOC_WORKSPACE_BYTES
    args = [dev(x[n]) for n in ("q", "k", "v", "g", "beta")]
    s_in = dev(x["state_in"])
    cu = dev(x["cu_seqlens"])
    odt = torch.bfloat16 if out_dtype == inputs.BF16 else torch.float32
    T, h_v, d, N = x["total_tokens"], x["h_v"], x["d"], desc.num_seqs
    res = []
    for noalloc in (True, False):
        out = torch.full((T, h_v, d), float("nan"), dtype=odt, device="cuda")
        st = torch.full((N, h_v, d, d), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            gdn.gdn_prefill_noalloc(desc, *args, s_in, out, st, cu, 64)
        else:
            ws = torch.empty(gdn.gdn_prefill_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
            gdn.gdn_prefill(desc, *args, s_in, out, st, cu, 64, ws, ws.numel())
        torch.cuda.synchronize()
        res.append((out, st))
    return res


def test_noalloc_matches_prefill_twice_shrinking():
    big = inputs.workload_inputs(inputs.WORKLOADS["prefill_t4096_hv32_hk16_d128"])
    small = inputs.prefill_inputs(seed=31, lengths=[300, 1, 77, 500], h_k=2, h_v=4, d=128,
                                  io_dtype=inputs.BF16, state_std=0.1)
    for x, od in ((big, inputs.BF16), (small, inputs.F32)):
        (o1, s1), (o2, s2) = _both(x, od)
        assert torch.isfinite(o1.float()).all() and torch.isfinite(s1).all()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_noalloc_rejects_problems_beyond_its_workspace():
    desc = gdn.make_desc(num_seqs=1, total_tokens=8192, h_k=16, h_v=32, d=128, io_dtype=gdn.GDN_BF16,
                         out_dtype=gdn.GDN_BF16)
    assert gdn.gdn_prefill_workspace_bytes(desc) > gdn.GDN_PREFILL_NOALLOC_WORKSPACE_BYTES
    F = 0x10000  # never used: the size check comes first
    st = gdn.lib().gdn_prefill_noalloc(ctypes.byref(desc), F, F + (1 << 32), F + (2 << 32), F + (3 << 32),
                                       F + (4 << 32), None, F + (5 << 32), None, None, 64, None)
    assert st == gdn.GDN_ERR_WORKSPACE and "noalloc" in gdn.last_error()
