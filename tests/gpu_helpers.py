"""Shared helpers of the GPU parity tests (not a test module)."""
import numpy as np
import torch

DEV = "cuda:0"


def dev(x):
    """numpy -> device tensor.  uint16 arrays are bfloat16 bit patterns."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(x, r):
    """max_i |x_i - r_i| / max_i |r_i| (the parity metric)."""
    return float(np.abs(x - r).max() / max(np.abs(r).max(), 1e-300))


def bf16_half_ulp(r):
    a = np.abs(r)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 0.5 * 2.0 ** (e - 7)


def check_bf16_out(x, r, tol):
    """bf16-rounded outputs: |x - r| <= tol * max|r| + half a bf16 ulp of r, elementwise."""
    bound = tol * np.abs(r).max() + bf16_half_ulp(r)
    bad = np.abs(x - r) > bound
    assert not bad.any(), "bf16 output outside tol*max|r| + ulp/2 at %d elements (worst excess %.3g)" % (
        int(bad.sum()), float((np.abs(x - r) - bound).max()))


def gather_units(inp, units, h_k, h_v):
    """Repack the (sequence, v-head) units of a packed prefill problem as separate
    single-head sequences, so the oracle can compute just those units."""
    r = h_v // h_k
    cu = inp["cu_seqlens"]
    T = inp["total_tokens"]
    if cu is None:
        cu = np.array([0, T], dtype=np.int32)
    qs, ks, vs, gs, bs, lens, s0 = [], [], [], [], [], [], []
    for (n, h) in units:
        sl = slice(int(cu[n]), int(cu[n + 1]))
        qs.append(inp["q"][sl, h // r]); ks.append(inp["k"][sl, h // r])
        vs.append(inp["v"][sl, h]); gs.append(inp["g"][sl, h]); bs.append(inp["beta"][sl, h])
        lens.append(sl.stop - sl.start)
        if inp["state_in"] is not None:
            s0.append(inp["state_in"][n, h])
    cat = lambda xs: np.concatenate(xs, axis=0)
    sub = dict(q=cat(qs)[:, None], k=cat(ks)[:, None], v=cat(vs)[:, None], g=cat(gs)[:, None],
               beta=cat(bs)[:, None], cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
               state_in=np.stack(s0)[:, None] if s0 else None)
    return sub


def _slices(n, step):
    for i in range(0, n, step):
        yield slice(i, min(n, i + step))


def normwise_blocks(t, r, step=4096):
    """normwise(host(t), r) over the leading axis in slices, so a large device
    tensor is never widened to float64 on the host in one piece."""
    rmax = max(float(np.abs(r).max()), 1e-300)
    err = 0.0
    for s in _slices(r.shape[0], step):
        err = max(err, float(np.abs(host(t[s]) - r[s]).max()))
    return err / rmax


def check_bf16_out_blocks(t, r, tol, step=4096):
    """check_bf16_out over the leading axis in slices, with the bound taken
    from the whole reference tensor."""
    rmax = float(np.abs(r).max())
    bad_total, worst = 0, 0.0
    for s in _slices(r.shape[0], step):
        x, rs = host(t[s]), r[s]
        bound = tol * rmax + bf16_half_ulp(rs)
        excess = np.abs(x - rs) - bound
        bad_total += int((excess > 0).sum())
        worst = max(worst, float(excess.max()))
    assert bad_total == 0, "bf16 output outside tol*max|r| + ulp/2 at %d elements (worst excess %.3g)" % (
        bad_total, worst)
