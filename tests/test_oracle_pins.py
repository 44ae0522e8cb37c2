"""Pins for the fp64 CPU oracle, each independent of the oracle's own code.

The pages ("Optimizing on-device inference for Apple Silicon", section "Qwen
creates three distinct workload shapes") describe the gated delta rule
qualitatively and print no worked example.  So the oracle is pinned by:
  * hand-worked examples (tests/golden/hand_examples.json);
  * closed forms: beta = 0 gives pure geometric decay of the initial state;
    alpha = beta = 1 with orthonormal keys gives exact overwrite-retrieval;
  * brute force on T <= 8: explicit products of the per-token transition
    matrices M_t = alpha_t (I - beta_t k_t k_t^T);
  * invariants: the blocked form equals the token scan (the page's two
    evaluation strategies compute the same thing), linearity in
    (state, values), the contraction bound, grouped-head sharing equal to
    duplicated heads, and packed sequences equal to separate calls;
  * a mutation check: plausible mistakes planted in a copy of the oracle's C
    source must each fail at least one of the pins above;
  * for the per-token ops beside the decode step (gate activations, output
    normalisation): closed forms (softplus(0) = ln 2, exp(-softplus(x)) =
    1 / (1 + e^x), a hand-worked norm), identities and invariants, each also
    shown to fail for planted mistakes.
"""
import json
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rand_case(rng, T, h_k, h_v, d, s0=True, unit_qk=False):
    q = rng.standard_normal((T, h_k, d))
    k = rng.standard_normal((T, h_k, d))
    if unit_qk:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, h_v, d))
    g = -np.logaddexp(0.0, rng.standard_normal((T, h_v)))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, h_v))))
    S0 = 0.3 * rng.standard_normal((1, h_v, d, d)) if s0 else None
    return q, k, v, g, b, S0


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# --- hand-worked examples ------------------------------------------------------------------

@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    T, d = len(case["q"]), case["d"]
    q = np.array(case["q"], float).reshape(T, 1, d)
    k = np.array(case["k"], float).reshape(T, 1, d)
    v = np.array(case["v"], float).reshape(T, 1, d)
    g = np.log(np.array(case["alpha"], float)).reshape(T, 1)
    b = np.array(case["beta"], float).reshape(T, 1)
    s0 = np.array(case["state_in"], float).reshape(1, 1, d, d)
    for fn in (oracle.scan, lambda *a, **kw: oracle.chunked(*a, chunk=1, **kw)):
        out, st = fn(q, k, v, g, b, h_k=1, h_v=1, state_in=s0, qk_l2norm=case["qk_l2norm"],
                     scale=case["scale"])
        np.testing.assert_allclose(out.reshape(T, d), np.array(case["out"]), atol=case["tol"], rtol=0)
        np.testing.assert_allclose(st.reshape(d, d), np.array(case["state_out"]), atol=case["tol"], rtol=0)


# --- closed forms --------------------------------------------------------------------------

def test_beta_zero_is_geometric_decay():
    rng = np.random.default_rng(11)
    T, d = 37, 16
    q, k, v, g, b, S0 = rand_case(rng, T, 1, 1, d, unit_qk=True)
    b[:] = 0.0
    out, st = oracle.scan(q, k, v, g, b, h_k=1, h_v=1, state_in=S0, qk_l2norm=False)
    cum = np.cumprod(np.exp(g[:, 0]))
    np.testing.assert_allclose(st[0, 0], cum[-1] * S0[0, 0], rtol=1e-12, atol=1e-14)
    expect = cum[:, None] * (S0[0, 0] @ q[:, 0, :].T).T
    np.testing.assert_allclose(out[:, 0, :], expect, rtol=1e-12, atol=1e-14)


def hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("l2norm", [False, True])
def test_overwrite_retrieval_orthonormal_keys(l2norm):
    d = 64
    keys = hadamard(d) / 8.0            # orthonormal rows, exact in bf16 as well
    rng = np.random.default_rng(5)
    order = rng.permutation(d)[:20]
    T = len(order) + 1
    k = np.zeros((T, 1, d)); q = np.zeros((T, 1, d)); v = rng.standard_normal((T, 1, d))
    for t, i in enumerate(order):
        k[t, 0] = keys[i]
        q[t, 0] = keys[i]
    # last token rewrites the first key with a new value
    k[-1, 0] = keys[order[0]]; q[-1, 0] = keys[order[0]]
    g = np.zeros((T, 1)); b = np.ones((T, 1))
    out, st = oracle.scan(q, k, v, g, b, h_k=1, h_v=1, qk_l2norm=l2norm)
    tol = 1e-6 if l2norm else 1e-13   # the 1e-6 epsilon shortens unit keys by ~5e-7
    # reading with the key just written returns exactly the value just written
    np.testing.assert_allclose(out[:, 0], v[:, 0], atol=tol * 10, rtol=0)
    S = st[0, 0]
    for t, i in enumerate(order[1:], start=1):
        np.testing.assert_allclose(S @ keys[i], v[t, 0], atol=tol * 10, rtol=0)
    np.testing.assert_allclose(S @ keys[order[0]], v[-1, 0], atol=tol * 10, rtol=0)


# --- brute force -------------------------------------------------------------------------

def brute_force(q, k, v, g, b, S0, l2norm=True, scale=1.0):
    """S_t = S_0 M_1...M_t + sum_{j<=t} beta_j v_j k_j^T M_{j+1}...M_t with the
    transition matrices M_j = alpha_j (I - beta_j k_j k_j^T) formed explicitly."""
    T, d = q.shape[0], q.shape[-1]
    def prep(x):
        return x / np.sqrt((x * x).sum() + 1e-6) if l2norm else x
    K = np.array([prep(k[t]) for t in range(T)])
    Q = np.array([prep(q[t]) * scale for t in range(T)])
    M = [np.exp(g[t]) * (np.eye(d) - b[t] * np.outer(K[t], K[t])) for t in range(T)]
    outs, St = [], None
    for t in range(T):
        prod = np.eye(d)
        for j in range(t + 1):
            prod = prod @ M[j]
        St = S0 @ prod
        for j in range(t + 1):
            tail = np.eye(d)
            for m in range(j + 1, t + 1):
                tail = tail @ M[m]
            St = St + b[j] * np.outer(v[j], K[j]) @ tail
        outs.append(St @ Q[t])
    return np.array(outs), St


@pytest.mark.parametrize("T", [1, 2, 5, 8])
@pytest.mark.parametrize("l2norm", [True, False])
def test_brute_force_products(T, l2norm):
    rng = np.random.default_rng(100 + T)
    d = 6
    q, k, v, g, b, S0 = rand_case(rng, T, 1, 1, d)
    out, st = oracle.scan(q, k, v, g, b, h_k=1, h_v=1, state_in=S0, qk_l2norm=l2norm, scale=0.7)
    bo, bs = brute_force(q[:, 0], k[:, 0], v[:, 0], g[:, 0], b[:, 0], S0[0, 0], l2norm, 0.7)
    assert rel(out[:, 0], bo) < 1e-12
    assert rel(st[0, 0], bs) < 1e-12


# --- invariants ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,C", [(1, 64), (63, 64), (64, 64), (65, 64), (200, 64), (200, 1),
                                 (200, 4), (200, 16), (200, 200), (257, 16)])
def test_chunked_equals_scan(T, C):
    rng = np.random.default_rng(T * 7 + C)
    q, k, v, g, b, S0 = rand_case(rng, T, 2, 4, 16)
    o1, s1 = oracle.scan(q, k, v, g, b, h_k=2, h_v=4, state_in=S0)
    o2, s2 = oracle.chunked(q, k, v, g, b, h_k=2, h_v=4, state_in=S0, chunk=C)
    assert rel(o2, o1) < 1e-12
    assert rel(s2, s1) < 1e-12


def test_chunked_equals_scan_long_memory_varlen():
    rng = np.random.default_rng(3)
    lens = [0, 130, 64, 1, 77]
    T = sum(lens)
    q, k, v, g, b, _ = rand_case(rng, T, 1, 2, 32)
    g = -np.logaddexp(0.0, rng.standard_normal(g.shape) - 4.0)   # alpha close to 1
    S0 = 0.1 * rng.standard_normal((len(lens), 2, 32, 32))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o1, s1 = oracle.scan(q, k, v, g, b, h_k=1, h_v=2, state_in=S0, cu_seqlens=cu)
    o2, s2 = oracle.chunked(q, k, v, g, b, h_k=1, h_v=2, state_in=S0, cu_seqlens=cu, chunk=64)
    assert rel(o2, o1) < 1e-11
    assert rel(s2, s1) < 1e-11
    # a zero-length sequence passes its state through unchanged
    np.testing.assert_array_equal(s1[0], S0[0])


def test_linear_in_state_and_values():
    rng = np.random.default_rng(8)
    T, d = 50, 8
    q, k, v, g, b, S0 = rand_case(rng, T, 1, 1, d)
    _, _, v2, _, _, S02 = rand_case(rng, T, 1, 1, d)
    a1, a2 = 0.7, -1.3
    o1, s1 = oracle.scan(q, k, v, g, b, h_k=1, h_v=1, state_in=S0)
    o2, s2 = oracle.scan(q, k, v2, g, b, h_k=1, h_v=1, state_in=S02)
    o3, s3 = oracle.scan(q, k, a1 * v + a2 * v2, g, b, h_k=1, h_v=1, state_in=a1 * S0 + a2 * S02)
    assert rel(o3, a1 * o1 + a2 * o2) < 1e-12
    assert rel(s3, a1 * s1 + a2 * s2) < 1e-12


def test_contraction_bound():
    rng = np.random.default_rng(9)
    T, d = 40, 8
    q, k, v, g, b, S0 = rand_case(rng, T, 1, 1, d)
    prev = np.linalg.norm(S0[0, 0], 2)
    for t in range(1, T + 1):
        _, st = oracle.scan(q[:t], k[:t], v[:t], g[:t], b[:t], h_k=1, h_v=1, state_in=S0)
        cur = np.linalg.norm(st[0, 0], 2)
        bound = np.exp(g[t - 1, 0]) * prev + b[t - 1, 0] * np.linalg.norm(v[t - 1, 0])
        assert cur <= bound * (1 + 1e-12)
        prev = cur


def test_grouped_heads_equal_duplicated_heads():
    rng = np.random.default_rng(10)
    T, d = 70, 16
    q, k, v, g, b, S0 = rand_case(rng, T, 2, 6, d)
    o1, s1 = oracle.scan(q, k, v, g, b, h_k=2, h_v=6, state_in=S0)
    qd = np.repeat(q, 3, axis=1); kd = np.repeat(k, 3, axis=1)   # v-head h reads k-head h // 3
    o2, s2 = oracle.scan(qd, kd, v, g, b, h_k=6, h_v=6, state_in=S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_packed_equals_separate_and_decode_equals_scan():
    rng = np.random.default_rng(12)
    lens = [5, 0, 9, 1]
    T, d = sum(lens), 8
    q, k, v, g, b, _ = rand_case(rng, T, 1, 2, d)
    S0 = rng.standard_normal((len(lens), 2, d, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, s = oracle.scan(q, k, v, g, b, h_k=1, h_v=2, state_in=S0, cu_seqlens=cu)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        on, sn = oracle.scan(q[sl], k[sl], v[sl], g[sl], b[sl], h_k=1, h_v=2, state_in=S0[n:n + 1])
        np.testing.assert_array_equal(o[sl], on)
        np.testing.assert_array_equal(s[n], sn[0])
    # decode: one token per sequence, state carried step to step
    N = 3
    st = rng.standard_normal((N, 2, d, d))
    qs, ks, vs, gs, bs, _ = rand_case(rng, 4 * N, 1, 2, d)
    ref = st.copy()
    for step in range(4):
        sl = slice(step * N, (step + 1) * N)
        od, st = oracle.decode_step(qs[sl], ks[sl], vs[sl], gs[sl], bs[sl], st, h_k=1, h_v=2)
        for n in range(N):
            on, ref_n = oracle.scan(qs[sl][n:n + 1], ks[sl][n:n + 1], vs[sl][n:n + 1],
                                    gs[sl][n:n + 1], bs[sl][n:n + 1], h_k=1, h_v=2,
                                    state_in=ref[n:n + 1])
            np.testing.assert_array_equal(od[n], on[0])
            ref[n] = ref_n[0]
    np.testing.assert_array_equal(st, ref)


# --- the pins catch planted mistakes -------------------------------------------------------

MUTATIONS = {
    # drop alpha from the erase term
    "no_alpha_on_erase": ("*s = alpha * *s - alpha * bt * Sk[i] * kh[j]", "*s = alpha * *s - bt * Sk[i] * kh[j]"),
    # wrong sign of the written value
    "value_sign": ("+ bt * vt[i] * kh[j];", "- bt * vt[i] * kh[j];"),
    # transposed state access in S k
    "transposed_Sk": ("acc += S[(size_t)i * d_k + j] * kh[j];\n                Sk[i] = acc;",
                      "acc += S[(size_t)j * d_k + i] * kh[j];\n                Sk[i] = acc;"),
    # v-heads mapped to the wrong k-head
    "wrong_kv_head": ("hk = h / r;", "hk = h % h_k;"),
    # output read with the key instead of the query
    "query_vs_key": ("acc += S[(size_t)i * d_k + j] * qh[j];", "acc += S[(size_t)i * d_k + j] * kh[j];"),
    "no_eps_sqrt": ("1.0 / sqrt(ss + GDN_EPS)", "1.0 / (ss + GDN_EPS)"),
    "decay_after": ("const double alpha = exp(g[(size_t)t * h_v + h]);",
                    "const double alpha = exp(g[(size_t)t * h_v + h]) * 0.999;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTATIONS[name]
    assert old in src, name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           str(mutated), "-o", str(lib), "-lm"])
    env = dict(os.environ, GDN_ORACLE_LIB=str(lib))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    # run the pins (not this test) against the mutated library in a child process
    r = subprocess.run(["python", "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.abspath(__file__), "-k", "not planted"],
                       cwd=root, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "mutation %s survived every pin:\n%s" % (name, r.stdout[-2000:])


# ---- the per-token ops beside the decode step ---------------------------------------------
# gate_activations and output_rms_norm are pinned by closed forms and identities of the
# two functions, written independently of the oracle's code; each pin helper returns the
# names of the pins an implementation fails, so planted mistakes can be checked too.

def gate_pin_failures(fn):
    fails = []
    g, b = fn(np.array([0.0]), np.array([0.0]))
    # softplus(0) = ln 2 and the logistic function at 0 is 1/2
    if abs(g[0] + 0.6931471805599453) > 1e-15 or abs(b[0] - 0.5) > 1e-15:
        fails.append("values at zero")
    x = np.linspace(-30.0, 30.0, 121)
    g, b = fn(x, x)
    _, b_neg = fn(x, -x)
    # exp(-softplus(x)) = 1 / (1 + e^x): the decay of input x is the write strength of input -x
    if not np.allclose(np.exp(g), b_neg, rtol=1e-13, atol=0.0):
        fails.append("alpha is the logistic function of -x")
    g_neg, _ = fn(-x, x)
    # softplus(x) - softplus(-x) = x
    if not np.allclose(g_neg - g, x, rtol=0.0, atol=1e-12):
        fails.append("odd part of softplus")
    if not (np.all(np.diff(g) < 0.0) and np.all(np.diff(b) > 0.0) and np.all(g < 0.0)):
        fails.append("monotone, g < 0")
    g, b = fn(np.array([-800.0, 800.0]), np.array([-800.0, 800.0]))
    if not (np.all(np.isfinite(g)) and g[0] == 0.0 and g[1] == -800.0 and b[0] == 0.0 and b[1] == 1.0):
        fails.append("finite at the ends")
    return fails


def norm_pin_failures(fn):
    fails = []
    # hand-worked: o = (3, 4) has mean square 12.5; 3/sqrt(12.5) and 2*4/sqrt(12.5)
    out = fn(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    if not np.allclose(out, [[0.8485281374238570, 2.2627416997969525]], rtol=1e-15, atol=0.0):
        fails.append("hand-worked (3, 4)")
    # eps inside the root: eps = 12.5 doubles the mean square, o / 5
    out = fn(np.array([[3.0, 4.0]]), None, 12.5)
    if not np.allclose(out, [[0.6, 0.8]], rtol=1e-15, atol=0.0):
        fails.append("eps inside the square root")
    rng = np.random.default_rng(5)
    o = 7.0 * rng.standard_normal((4, 3, 16))
    out = fn(o, None, 0.0)
    if not np.allclose(np.sqrt(np.mean(out * out, axis=-1)), 1.0, rtol=1e-14, atol=0.0):
        fails.append("unit root-mean-square per head")
    o2 = o.copy()
    o2[1, 2] *= 3.0
    o2[0, 1] += 1.0
    out2 = fn(o2, None, 0.0)
    # each head on its own: scaling a head leaves it unchanged, other heads never move
    same = np.ones((4, 3), dtype=bool)
    same[0, 1] = False
    if not (np.allclose(out2[same], out[same], rtol=1e-14, atol=0.0) and
            not np.allclose(out2[0, 1], out[0, 1])):
        fails.append("heads independent, scale invariant")
    w = rng.standard_normal(16)
    if not np.allclose(fn(o, w, 0.0), out * w, rtol=1e-14, atol=0.0):
        fails.append("channel-wise weight")
    if not np.all(fn(np.zeros((2, 8)), None, 1e-6) == 0.0):
        fails.append("zero output stays zero")
    return fails


def test_gate_activations_pins():
    assert gate_pin_failures(oracle.gate_activations) == []


def test_output_rms_norm_pins():
    assert norm_pin_failures(oracle.output_rms_norm) == []


def _planted_gates():
    def sign(x, y):
        g, b = oracle.gate_activations(x, y)
        return -g, b
    def argument(x, y):
        return oracle.gate_activations(-np.asarray(x), y)
    def beta_flip(x, y):
        return oracle.gate_activations(x, -np.asarray(y))
    def naive(x, y):
        x = np.asarray(x, dtype=np.float64)
        y = np.asarray(y, dtype=np.float64)
        with np.errstate(over="ignore"):
            return -np.log1p(np.exp(x)), 1.0 / (1.0 + np.exp(-y))
    return {"sign": sign, "argument": argument, "beta_flip": beta_flip, "naive_overflow": naive}


def _planted_norms():
    def mean_not_rms(o, w, eps):
        o = np.asarray(o, dtype=np.float64)
        out = o / (np.mean(o * o, axis=-1, keepdims=True) + eps)
        return out if w is None else out * w
    def eps_outside(o, w, eps):
        o = np.asarray(o, dtype=np.float64)
        out = o / (np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) + eps)
        return out if w is None else out * w
    def wrong_axis(o, w, eps):
        o = np.asarray(o, dtype=np.float64)
        out = o / np.sqrt(np.mean(o * o, axis=0, keepdims=True) + eps)
        return out if w is None else out * w
    def weight_divides(o, w, eps):
        out = oracle.output_rms_norm(o, None, eps)
        return out if w is None else out / w
    def sum_not_mean(o, w, eps):
        o = np.asarray(o, dtype=np.float64)
        out = o / np.sqrt(np.sum(o * o, axis=-1, keepdims=True) + eps)
        return out if w is None else out * w
    return {"mean_not_rms": mean_not_rms, "eps_outside": eps_outside, "wrong_axis": wrong_axis,
            "weight_divides": weight_divides, "sum_not_mean": sum_not_mean}


@pytest.mark.parametrize("name", sorted(_planted_gates()))
def test_gate_pins_catch_planted_mistake(name):
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        assert gate_pin_failures(_planted_gates()[name]) != []


@pytest.mark.parametrize("name", sorted(_planted_norms()))
def test_norm_pins_catch_planted_mistake(name):
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        assert norm_pin_failures(_planted_norms()[name]) != []


def test_decode_step_ex_composes_the_pinned_parts():
    """Both options off is decode_step; raw gate inputs of 0 are g = -ln 2, beta = 1/2;
    the output norm leaves the state alone and gives each head unit root-mean-square."""
    rng = np.random.default_rng(6)
    N, h_k, h_v, d = 3, 2, 4, 16
    q = rng.standard_normal((N, h_k, d))
    k = rng.standard_normal((N, h_k, d))
    v = rng.standard_normal((N, h_v, d))
    xg = rng.standard_normal((N, h_v))
    xb = rng.standard_normal((N, h_v))
    S = 0.2 * rng.standard_normal((N, h_v, d, d))
    o0, s0 = oracle.decode_step(q, k, v, xg, xb, S, h_k=h_k, h_v=h_v)
    o1, s1 = oracle.decode_step_ex(q, k, v, xg, xb, S, h_k=h_k, h_v=h_v)
    assert np.array_equal(o0, o1) and np.array_equal(s0, s1)
    z = np.zeros((N, h_v))
    o2, s2 = oracle.decode_step_ex(q, k, v, z, z, S, h_k=h_k, h_v=h_v, raw_gates=True)
    o3, s3 = oracle.decode_step(q, k, v, np.full((N, h_v), -np.log(2.0)), np.full((N, h_v), 0.5), S,
                                h_k=h_k, h_v=h_v)
    assert np.allclose(o2, o3, rtol=1e-14, atol=1e-15) and np.allclose(s2, s3, rtol=1e-14, atol=1e-15)
    o4, s4 = oracle.decode_step_ex(q, k, v, xg, xb, S, h_k=h_k, h_v=h_v, output_norm=True, norm_eps=0.0)
    assert np.array_equal(s4, s0)
    assert np.allclose(np.sqrt(np.mean(o4 * o4, axis=-1)), 1.0, rtol=1e-14)
    assert np.allclose(o4 * np.sqrt(np.mean(o0 * o0, axis=-1, keepdims=True)), o0, rtol=1e-13)


def test_scan_ex_is_decode_step_ex_token_by_token():
    """Two tokens through scan_ex equal two decode_step_ex calls; no options is scan."""
    rng = np.random.default_rng(8)
    h_k, h_v, d = 1, 2, 8
    q, k, v = rng.standard_normal((2, h_k, d)), rng.standard_normal((2, h_k, d)), rng.standard_normal((2, h_v, d))
    xg, xb = rng.standard_normal((2, h_v)), rng.standard_normal((2, h_v))
    S0 = 0.3 * rng.standard_normal((1, h_v, d, d))
    w = rng.standard_normal(d)
    o, s = oracle.scan_ex(q, k, v, xg, xb, h_k=h_k, h_v=h_v, state_in=S0, raw_gates=True, output_norm=True,
                          norm_weight=w)
    st = S0
    for t in range(2):
        ot, st = oracle.decode_step_ex(q[t:t + 1], k[t:t + 1], v[t:t + 1], xg[t:t + 1], xb[t:t + 1], st, h_k=h_k,
                                       h_v=h_v, raw_gates=True, output_norm=True, norm_weight=w)
        assert np.allclose(o[t], ot[0], rtol=1e-13, atol=1e-14)
    assert np.allclose(s, st, rtol=1e-13, atol=1e-14)
    o0, s0 = oracle.scan(q, k, v, xg, xb, h_k=h_k, h_v=h_v, state_in=S0)
    o1, s1 = oracle.scan_ex(q, k, v, xg, xb, h_k=h_k, h_v=h_v, state_in=S0)
    assert np.array_equal(o0, o1) and np.array_equal(s0, s1)
