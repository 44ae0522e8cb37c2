"""Boundary tests that need no GPU: the library loads, exports every function
include/gdn.h declares, sizes workspaces, and rejects every invalid argument on
the host before anything is enqueued (so no HIP call is reached).

Only argument sets that fail validation are passed here.  As a second guard,
the tests that pass made-up pointers are skipped wherever a GPU is visible, so
a validation bug can never turn into a launch on bad addresses.
"""
import ctypes
import os

import pytest

from linear_attention_recurrence_rule_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="made-up pointers are only passed where no GPU is visible")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdn.LIB_PATH):
        from linear_attention_recurrence_rule_amd import build
        build.build()
    return gdn.lib()


def test_exports_every_declared_function(L):
    names = gdn.declared_functions()
    assert set(names) == {"gdn_prefill_workspace_bytes", "gdn_prefill", "gdn_prefill_ex", "gdn_prefill_status_offset",
                          "gdn_prefill_noalloc",
                          "gdn_prefill_prepare",
                          "gdn_prefill_scan", "gdn_prefill_direct", "gdn_prefill_segmented_workspace_bytes",
                          "gdn_prefill_segmented", "gdn_prefill_two_level_workspace_bytes", "gdn_prefill_two_level",
                          "gdn_decode_step", "gdn_decode_step_slots", "gdn_decode_step_ex", "gdn_prefill_direct_ex",
                          "gdn_status_str", "gdn_last_error"}
    for n in names:
        assert hasattr(L, n), n


def test_desc_layout_matches_header():
    # int32, (pad), int64, 7 x int32, float  -> 48 bytes with 8-byte alignment
    assert ctypes.sizeof(gdn.GdnDesc) == 48
    assert gdn.GdnDesc.total_tokens.offset == 8
    assert gdn.GdnDesc.scale.offset == 44


def test_status_strings(L):
    for s, name in enumerate(["GDN_OK", "GDN_ERR_INVALID_ARGUMENT", "GDN_ERR_UNSUPPORTED",
                              "GDN_ERR_WORKSPACE", "GDN_ERR_HIP"]):
        assert gdn.status_str(s) == name
    assert gdn.status_str(99) == "GDN_UNKNOWN_STATUS"


def desc(**kw):
    base = dict(num_seqs=1, total_tokens=4096, h_k=16, h_v=32, d=128, io_dtype=gdn.GDN_BF16,
                out_dtype=gdn.GDN_BF16, qk_l2norm=True, scale=1.0)
    base.update(kw)
    return gdn.make_desc(**base)


def test_workspace_bytes(L):
    # bf16 inputs, per (block, v-head): the six non-zero 1 KiB fragments of T and
    # of P (fp16) and 1 KiB of per-token factors; per (block, k-head) a key record:
    # the scaled fp16 key and query tiles (64 x 128 each) and 1 KiB of factors.
    # 64 blocks x 32 v-heads / 16 k-heads.
    rec = 2 * 6 * 1024 + 1024
    key = 2 * 64 * 128 * 2 + 1024
    plan = (1280 + 1 * 16 + 64 * 4 + 255) // 256 * 256  # 1 KiB sink, 256 B status word, then the plan
    assert gdn.gdn_prefill_workspace_bytes(desc()) == plan + 64 * (32 * rec + 16 * key)
    # packed sequences: at most T/64 + N blocks in total
    n = gdn.gdn_prefill_workspace_bytes(desc(num_seqs=16, total_tokens=1000))
    slots = (1000 + 16 * 63) // 64
    assert n == (1280 + 16 * 16 + slots * 4 + 255) // 256 * 256 + slots * (32 * rec + 16 * key)
    # fp32 inputs keep fp32 operands
    rec64f = 4 * 64 * 64 * 4 + 512
    key64f = 64 * 64 * 4
    assert gdn.gdn_prefill_workspace_bytes(desc(total_tokens=256, h_k=1, h_v=1, d=64,
                                                io_dtype=gdn.GDN_F32, out_dtype=gdn.GDN_F32)) == \
        1536 + 4 * (rec64f + key64f)
    assert L.gdn_prefill_workspace_bytes(ctypes.byref(desc()), 32) == 0
    assert "chunk" in gdn.last_error()


def test_status_offset(L):
    d = desc()
    assert gdn.gdn_prefill_status_offset(d) == 1024  # after the 1 KiB sink, 4-byte aligned
    assert gdn.gdn_prefill_status_offset(desc(num_seqs=3, total_tokens=10)) == 1024
    assert L.gdn_prefill_status_offset(ctypes.byref(d), 32) == 0
    assert "chunk" in gdn.last_error()
    assert L.gdn_prefill_status_offset(ctypes.byref(desc(d=96)), 64) == 0


FAKE = 0x10000  # never dereferenced: every case below fails validation first


def call_prefill(d, *, q=FAKE, k=FAKE + 1 << 32, v=FAKE + 2 << 32, g=FAKE + 3 << 32, b=FAKE + 4 << 32,
                 s_in=None, out=FAKE + 5 << 32, s_out=None, cu=None, chunk=64, ws=None, ws_bytes=0):
    return gdn.lib().gdn_prefill(ctypes.byref(d), q, k, v, g, b, s_in, out, s_out, cu, chunk, ws,
                                 ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_seqs=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(h_k=0), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(h_v=24, h_k=16), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(d=96), gdn.GDN_ERR_UNSUPPORTED),
    (dict(io_dtype=7), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(out_dtype=-1), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(total_tokens=-5), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(total_tokens=(1 << 30) + 1), gdn.GDN_ERR_UNSUPPORTED),
    (dict(io_dtype=gdn.GDN_F32), gdn.GDN_ERR_UNSUPPORTED),      # fp32 prefill at d=128
    (dict(scale=float("inf")), gdn.GDN_ERR_INVALID_ARGUMENT),
    (dict(num_seqs=3), gdn.GDN_ERR_INVALID_ARGUMENT),           # cu_seqlens NULL with N > 1
])
@fake_pointers
def test_prefill_rejects_bad_descriptor(L, kw, status):
    d = desc(**kw)
    assert call_prefill(d) == status
    assert gdn.last_error() != ""


@fake_pointers
def test_prefill_rejects_bad_pointers_and_sizes(L):
    d = desc()
    need = gdn.gdn_prefill_workspace_bytes(d)
    ws = 0x7 << 40
    assert call_prefill(d, chunk=128, ws=ws, ws_bytes=need) == gdn.GDN_ERR_UNSUPPORTED
    assert call_prefill(d, q=None, ws=ws, ws_bytes=need) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_prefill(d, out=None, ws=ws, ws_bytes=need) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_prefill(d, ws=None, ws_bytes=need) == gdn.GDN_ERR_WORKSPACE
    assert call_prefill(d, ws=ws, ws_bytes=need - 1) == gdn.GDN_ERR_WORKSPACE
    # aliasing: out overlapping v is rejected
    assert call_prefill(d, out=(FAKE + 2 << 32) + 64, ws=ws, ws_bytes=need) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "overlap" in gdn.last_error()
    # workspace overlapping q is rejected
    assert call_prefill(d, ws=FAKE, ws_bytes=need) == gdn.GDN_ERR_INVALID_ARGUMENT
    # misaligned tensors are rejected
    assert call_prefill(d, q=FAKE + 2, ws=ws, ws_bytes=need) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "aligned" in gdn.last_error()
    assert call_prefill(d, ws=ws + 16, ws_bytes=need) == gdn.GDN_ERR_INVALID_ARGUMENT
    # state_out overlapping state_in at a different address is rejected
    s = 0x9 << 40
    assert call_prefill(d, s_in=s, s_out=s + 4, ws=ws, ws_bytes=need) == gdn.GDN_ERR_INVALID_ARGUMENT


@fake_pointers
def test_prefill_phases_reject_bad_arguments(L):
    d = desc()
    need = gdn.gdn_prefill_workspace_bytes(d)
    ws = 0x7 << 40
    lib = gdn.lib()
    by = ctypes.byref
    # prepare: inputs required, workspace checked
    assert lib.gdn_prefill_prepare(by(d), None, FAKE, FAKE + 2 << 32, FAKE + 3 << 32, FAKE + 4 << 32, None,
                                   64, ws, need, None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert lib.gdn_prefill_prepare(by(d), FAKE, FAKE + 1 << 32, FAKE + 2 << 32, FAKE + 3 << 32,
                                   FAKE + 4 << 32, None, 64, ws, need - 1, None) == gdn.GDN_ERR_WORKSPACE
    assert lib.gdn_prefill_prepare(by(desc(d=48)), FAKE, FAKE + 1 << 32, FAKE + 2 << 32, FAKE + 3 << 32,
                                   FAKE + 4 << 32, None, 64, ws, need, None) == gdn.GDN_ERR_UNSUPPORTED
    # scan: q, k, v and out required, aliasing checked
    qkv = (FAKE, FAKE + 1 << 32, FAKE + 2 << 32)
    assert lib.gdn_prefill_scan(by(d), *qkv, None, None, None, None, 64, ws, need, None) == \
        gdn.GDN_ERR_INVALID_ARGUMENT
    assert lib.gdn_prefill_scan(by(d), None, qkv[1], qkv[2], None, FAKE + 5 << 32, None, None, 64, ws, need,
                                None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert lib.gdn_prefill_scan(by(d), *qkv, None, ws + 8, None, None, 64, ws, need, None) == \
        gdn.GDN_ERR_INVALID_ARGUMENT
    assert lib.gdn_prefill_scan(by(desc(num_seqs=2)), *qkv, None, FAKE + 5 << 32, None, None, 64, ws, need,
                                None) == gdn.GDN_ERR_INVALID_ARGUMENT


@fake_pointers
def test_decode_rejects_bad_arguments(L):
    lib = gdn.lib()
    def call(d, **p):
        a = dict(q=FAKE, k=FAKE + 1 << 32, v=FAKE + 2 << 32, g=FAKE + 3 << 32, b=FAKE + 4 << 32,
                 s=FAKE + 5 << 32, o=FAKE + 6 << 32)
        a.update(p)
        return lib.gdn_decode_step(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["b"], a["s"],
                                   a["o"], None)
    assert call(desc(num_seqs=64, h_v=30)) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(num_seqs=64, d=32)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(desc(num_seqs=64), s=None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(num_seqs=64), o=FAKE + 5 << 32) == gdn.GDN_ERR_INVALID_ARGUMENT  # out == state
    assert call(desc(num_seqs=0)) == gdn.GDN_ERR_INVALID_ARGUMENT


@fake_pointers
def test_decode_slots_rejects_bad_arguments(L):
    lib = gdn.lib()
    def call(d, **p):
        a = dict(q=FAKE, k=FAKE + 1 << 32, v=FAKE + 2 << 32, g=FAKE + 3 << 32, b=FAKE + 4 << 32,
                 s=FAKE + 5 << 32, n=8, i=FAKE + 6 << 32, o=FAKE + 7 << 32)
        a.update(p)
        return lib.gdn_decode_step_slots(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["b"], a["s"],
                                         a["n"], a["i"], a["o"], None)
    assert call(desc(num_seqs=4, h_v=30)) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(num_seqs=4, d=32)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(desc(num_seqs=4), s=None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(num_seqs=4), i=None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(num_seqs=4), n=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "num_slots" in gdn.last_error()
    assert call(desc(num_seqs=4), i=FAKE + 6 << 32 | 2) == gdn.GDN_ERR_INVALID_ARGUMENT      # misaligned slots
    assert call(desc(num_seqs=4), i=(FAKE + 5 << 32) + 64) == gdn.GDN_ERR_INVALID_ARGUMENT  # slots inside the pool
    assert "overlap" in gdn.last_error()


@fake_pointers
def test_decode_ex_rejects_bad_arguments(L):
    lib = gdn.lib()
    def call(d, **p):
        a = dict(q=FAKE, k=FAKE + 1 << 32, v=FAKE + 2 << 32, g=FAKE + 3 << 32, b=FAKE + 4 << 32,
                 s=FAKE + 5 << 32, o=FAKE + 6 << 32, f=3, w=FAKE + 7 << 32, e=1e-6)
        a.update(p)
        return lib.gdn_decode_step_ex(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["b"], a["s"], a["o"],
                                      a["f"], a["w"], a["e"], None)
    assert call(desc(num_seqs=8, h_v=30)) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(num_seqs=8, d=32)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(desc(num_seqs=8), s=None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(num_seqs=8), f=8) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "flags" in gdn.last_error()
    # one workgroup of 2 d threads per unit: 2^19 x 32 units x 256 reaches 2^32 work-items
    assert call(desc(num_seqs=1 << 19), f=gdn.GDN_STREAM_STATE) == gdn.GDN_ERR_UNSUPPORTED
    assert "units" in gdn.last_error()
    for eps in (0.0, -1e-6, float("nan"), float("inf")):
        assert call(desc(num_seqs=8), e=eps) == gdn.GDN_ERR_INVALID_ARGUMENT
        assert "norm_eps" in gdn.last_error()
    assert call(desc(num_seqs=8), w=(FAKE + 7 << 32) | 2) == gdn.GDN_ERR_INVALID_ARGUMENT    # misaligned weight
    assert call(desc(num_seqs=8), w=(FAKE + 5 << 32) + 256) == gdn.GDN_ERR_INVALID_ARGUMENT  # weight inside state
    assert "overlap" in gdn.last_error()


@fake_pointers
def test_direct_ex_rejects_bad_arguments(L):
    lib = gdn.lib()
    def call(d, **p):
        a = dict(q=FAKE, k=FAKE + 1 << 32, v=FAKE + 2 << 32, g=FAKE + 3 << 32, b=FAKE + 4 << 32,
                 si=FAKE + 5 << 32, o=FAKE + 6 << 32, so=FAKE + 5 << 32, cu=None, f=3, w=FAKE + 7 << 32, e=1e-6)
        a.update(p)
        return lib.gdn_prefill_direct_ex(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["b"], a["si"], a["o"],
                                         a["so"], a["cu"], a["f"], a["w"], a["e"], None)
    assert call(desc(total_tokens=16, h_v=30)) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(total_tokens=16), f=8) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "flags" in gdn.last_error()
    assert call(desc(total_tokens=16), f=gdn.GDN_STREAM_STATE) == gdn.GDN_ERR_INVALID_ARGUMENT  # decode only
    assert call(desc(total_tokens=16), e=0.0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(total_tokens=16), e=float("nan")) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(total_tokens=16), w=(FAKE + 6 << 32) + 64) == gdn.GDN_ERR_INVALID_ARGUMENT  # weight in out
    assert "overlap" in gdn.last_error()
    assert call(desc(total_tokens=16, num_seqs=2)) == gdn.GDN_ERR_INVALID_ARGUMENT  # no cu_seqlens


def test_two_level_workspace_bytes(L):
    one = gdn.gdn_prefill_workspace_bytes(desc(total_tokens=4096))
    assert gdn.gdn_prefill_two_level_workspace_bytes(desc(total_tokens=4096), 1) == one
    # 64 blocks in 8 segments of 8: single-sequence records, a 256-byte segment table, then
    # R and B for 7 segments and start and end states for 8 (32 v-heads, d = 128, fp32)
    rec = 2 * 6 * 1024 + 1024
    key = 2 * 64 * 128 * 2 + 1024
    base = 1280 + 64 * (32 * rec + 16 * key)
    st = 32 * 128 * 128 * 4
    assert gdn.gdn_prefill_two_level_workspace_bytes(desc(total_tokens=4096), 8) == base + 256 + (7 + 7 + 8 + 8) * st
    # more segments than blocks: one segment per block
    assert gdn.gdn_prefill_two_level_workspace_bytes(desc(total_tokens=200), 99) == \
        gdn.gdn_prefill_two_level_workspace_bytes(desc(total_tokens=200), 4)
    assert L.gdn_prefill_two_level_workspace_bytes(ctypes.byref(desc(num_seqs=2)), 64, 4) == 0
    assert "one sequence" in gdn.last_error()
    assert L.gdn_prefill_two_level_workspace_bytes(ctypes.byref(desc()), 64, 0) == 0
    assert "segments" in gdn.last_error()


@fake_pointers
def test_two_level_rejects_bad_arguments(L):
    lib = gdn.lib()
    d0 = desc(total_tokens=4096)
    need = gdn.gdn_prefill_two_level_workspace_bytes(d0, 4)
    ws = FAKE + 9 << 32
    def call(d, **p):
        a = dict(q=FAKE, k=FAKE + 1 << 32, v=FAKE + 2 << 32, g=FAKE + 3 << 32, b=FAKE + 4 << 32,
                 si=None, o=FAKE + 5 << 32, so=None, seg=4, ws=ws, n=need)
        a.update(p)
        return lib.gdn_prefill_two_level(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["b"], a["si"], a["o"],
                                         a["so"], 64, a["seg"], a["ws"], a["n"], None)
    assert call(desc(total_tokens=4096, num_seqs=2)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(d0, seg=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(d0, n=need - 1) == gdn.GDN_ERR_WORKSPACE
    assert call(d0, ws=None) == gdn.GDN_ERR_WORKSPACE
    assert call(d0, o=None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(d0, o=ws + 4096) == gdn.GDN_ERR_INVALID_ARGUMENT   # out inside the workspace
    assert "overlap" in gdn.last_error()


@fake_pointers
def test_direct_prefill_rejects_bad_arguments(L):
    lib = gdn.lib()
    def call(d, **p):
        a = dict(q=FAKE, k=FAKE + 1 << 32, v=FAKE + 2 << 32, g=FAKE + 3 << 32, b=FAKE + 4 << 32,
                 si=None, o=FAKE + 5 << 32, so=None, cu=None)
        a.update(p)
        return lib.gdn_prefill_direct(ctypes.byref(d), a["q"], a["k"], a["v"], a["g"], a["b"], a["si"],
                                      a["o"], a["so"], a["cu"], None)
    assert call(desc(h_v=30)) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(d=32)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(desc(total_tokens=-1)) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(num_seqs=2)) == gdn.GDN_ERR_INVALID_ARGUMENT           # cu_seqlens NULL with 2 sequences
    assert call(desc(), o=None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(desc(), q=FAKE + 2) == gdn.GDN_ERR_INVALID_ARGUMENT         # misaligned
    assert call(desc(), o=FAKE + 4 << 32) == gdn.GDN_ERR_INVALID_ARGUMENT   # out overlaps beta
    s = FAKE + 7 << 32
    assert call(desc(), si=s, so=s + 256) == gdn.GDN_ERR_INVALID_ARGUMENT  # partial state overlap
    assert "overlap" in gdn.last_error()


def test_segmented_workspace_bytes(L):
    full = gdn.gdn_prefill_workspace_bytes(desc(total_tokens=1 << 17))
    seg = gdn.gdn_prefill_segmented_workspace_bytes(desc(total_tokens=1 << 17), 4096)
    one = gdn.gdn_prefill_workspace_bytes(desc(total_tokens=4096))
    # one segment's workspace (aligned) plus one fp32 state of 32 heads x 128 x 128
    assert seg == (one + 255) // 256 * 256 + 32 * 128 * 128 * 4
    assert seg < full // 20
    for bad in (0, 100, -64):
        assert L.gdn_prefill_segmented_workspace_bytes(ctypes.byref(desc()), 64, bad) == 0
        assert "segment_tokens" in gdn.last_error()
    assert L.gdn_prefill_segmented_workspace_bytes(ctypes.byref(desc(num_seqs=2)), 64, 256) == 0
    assert L.gdn_prefill_segmented_workspace_bytes(ctypes.byref(desc()), 32, 256) == 0


@fake_pointers
def test_segmented_rejects_bad_arguments(L):
    lib = gdn.lib()
    d = desc()
    need = gdn.gdn_prefill_segmented_workspace_bytes(d, 1024)
    ws = FAKE + 9 << 32
    def call(dd, seg=1024, wsb=need, **p):
        a = dict(q=FAKE, k=FAKE + 1 << 32, v=FAKE + 2 << 32, g=FAKE + 3 << 32, b=FAKE + 4 << 32,
                 si=None, o=FAKE + 5 << 32, so=None, ws=ws)
        a.update(p)
        return lib.gdn_prefill_segmented(ctypes.byref(dd), a["q"], a["k"], a["v"], a["g"], a["b"], a["si"], a["o"],
                                          a["so"], 64, seg, a["ws"], wsb, None)
    assert call(d, seg=1000) == gdn.GDN_ERR_UNSUPPORTED
    assert call(desc(num_seqs=3)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(d, wsb=need - 1) == gdn.GDN_ERR_WORKSPACE
    assert call(d, ws=None) == gdn.GDN_ERR_WORKSPACE
    assert call(d, o=None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(d, o=FAKE + 3 << 32) == gdn.GDN_ERR_INVALID_ARGUMENT  # out overlaps g


@fake_pointers
def test_null_descriptor(L):
    assert gdn.lib().gdn_prefill(None, None, None, None, None, None, None, None, None, None, 64,
                                 None, 0, None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert gdn.lib().gdn_decode_step(None, None, None, None, None, None, None, None, None) == \
        gdn.GDN_ERR_INVALID_ARGUMENT
    assert gdn.lib().gdn_prefill_direct(None, None, None, None, None, None, None, None, None, None, None) == \
        gdn.GDN_ERR_INVALID_ARGUMENT


def test_calibration_library_loads_and_rejects_bad_arguments():
    """libgdn_calibrate.so (the measured-ceiling kernels bench.py reports) loads and checks its
    arguments on the host; no launch is reached."""
    from linear_attention_recurrence_rule_amd import build
    path = build.CAL_LIB
    if not os.path.exists(path):
        build.build()
    C = ctypes.CDLL(path)
    for name in ("gdn_calib_mfma_f16", "gdn_calib_mfma_f16_flops", "gdn_calib_rmw_f32"):
        assert hasattr(C, name), name
    C.gdn_calib_mfma_f16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    C.gdn_calib_mfma_f16_flops.restype = ctypes.c_double
    assert C.gdn_calib_mfma_f16_flops(10, 3) == 2.0 * 16 * 128 * 128 * 10 * 3 * 4
    C.gdn_calib_mfma_f16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    C.gdn_calib_rmw_f32.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    assert C.gdn_calib_mfma_f16(0, 8, None, None) != 0        # no iterations, no sink
    assert C.gdn_calib_rmw_f32(None, 1024, 8, None) != 0      # no buffer


def test_header_is_plain_c(tmp_path):
    """include/gdn.h is a C header: it compiles as strict C99 (and as C++) with every
    declaration, the flag enum included."""
    import shutil
    import subprocess
    src = tmp_path / "use_gdn.c"
    src.write_text('#include "gdn.h"\n'
                   "int main(void) {\n"
                   "    gdn_fuse_flag f = GDN_FUSE_GATE_ACTIVATIONS;\n"
                   "    gdn_desc d;\n"
                   "    (void)f; (void)d;\n"
                   "    (void)gdn_decode_step_ex; (void)gdn_prefill_direct_ex; (void)gdn_prefill;\n"
                   "    return 0;\n"
                   "}\n")
    inc = os.path.join(ROOT, "include")
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        if shutil.which(cc) is None:
            pytest.skip("%s not available" % cc)
        lang = ["-x", "c++"] if cc == "g++" else []
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-I", inc] + lang +
                           [str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def call_prefill_ex(d, opt, *, cu=None):
    F = 0x10000
    return gdn.lib().gdn_prefill_ex(ctypes.byref(d), F, F + (1 << 32), F + (2 << 32), F + (3 << 32),
                                    F + (4 << 32), None, F + (5 << 32), None, cu, 64,
                                    ctypes.byref(opt) if opt is not None else None, None, 0, None)


@pytest.mark.parametrize("opt,status,msg", [
    ((8, 0, 0), gdn.GDN_ERR_INVALID_ARGUMENT, "scan_rows"),
    ((48, 0, 0), gdn.GDN_ERR_INVALID_ARGUMENT, "scan_rows"),
    ((16, 1, 0), gdn.GDN_ERR_INVALID_ARGUMENT, "reserved"),
    ((0, 0, -2), gdn.GDN_ERR_INVALID_ARGUMENT, "segment_tokens"),
    ((0, 0, 100), gdn.GDN_ERR_UNSUPPORTED, "multiple"),
])
def test_prefill_ex_rejects_bad_options(L, opt, status, msg):
    """Options are checked before anything else (the fake pointers are never used)."""
    assert call_prefill_ex(desc(), gdn.GdnPrefillOptions(*opt)) == status
    assert msg in gdn.last_error()


def test_prefill_ex_segments_need_one_sequence(L):
    st = call_prefill_ex(desc(num_seqs=2, total_tokens=256), gdn.GdnPrefillOptions(0, 0, 128), cu=0x20000)
    assert st == gdn.GDN_ERR_UNSUPPORTED and "one sequence" in gdn.last_error()


def test_prefill_ex_defaults_validate_like_prefill(L):
    """NULL options or explicit defaults reach the gdn_prefill checks (here: no workspace)."""
    for opt in (None, gdn.GdnPrefillOptions(0, 0, 0), gdn.GdnPrefillOptions(32, 0, -1)):
        assert call_prefill_ex(desc(), opt) == gdn.GDN_ERR_WORKSPACE


def test_no_environment_tuning():
    """The library reads no environment variables: tuning goes through gdn_prefill_ex."""
    import glob, os
    csrc = os.path.join(os.path.dirname(gdn.__file__), "csrc")
    for f in glob.glob(os.path.join(csrc, "*")):
        assert "getenv" not in open(f).read(), f
