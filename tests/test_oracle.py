"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: the literal
matrix form of the gated delta rule, exact rational arithmetic, a hand-worked
fixture, the delta-rule invariant, closed forms, and the independently derived
block form.  The recurrence is the one Perplexity's "Optimizing on-device
inference for Apple Silicon" describes in prose (section "Qwen creates three
distinct workload shapes"); the carried-state property is from section
"Bounding scratch memory by chunking the prompt".

The last tests plant plausible mistakes in copies of the oracle's token loop
and check that at least one pin fails for each.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (decode_attention, dequantize_q4, gated_delta_chunk_form, gated_delta_decode_fused,
                    gated_delta_decode_step, gated_delta_recurrence, grouped_gemm_q4, qk_head_of, round_bf16, sigmoid, softplus)
from gated_deltanet_linear_delta_amd.workloads import make_prefill, round_to_bf16, tiny_fp32_prefill

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(x, r):
    return np.linalg.norm(np.ravel(x - r)) / max(np.linalg.norm(np.ravel(r)), 1e-300)


def rand_problem(seed, T, h_qk, h_v, d_k, d_v, unit_k=True, gate_shift=0.0, state=True, N=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, h_qk, d_k))
    k = rng.standard_normal((T, h_qk, d_k))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, h_v, d_v))
    g = -np.logaddexp(0, rng.standard_normal((T, h_v)) + gate_shift)
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, h_v))))
    n = 1 if N is None else N
    s0 = rng.standard_normal((n, h_v, d_v, d_k)) * 0.5 if state else None
    return q, k, v, g, beta, s0


# ---------------------------------------------------------------- P1 brute force
def literal_matrix_form(q, k, v, g, beta, s0):
    """S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T with explicit d_k x d_k
    transition matrices; one sequence."""
    T, h_qk, d_k = q.shape
    h_v = v.shape[1]
    grp = h_v // h_qk
    o = np.zeros(v.shape)
    S_all = s0[0].copy()
    for h in range(h_v):
        S = S_all[h]
        for t in range(T):
            kk = k[t, h // grp][:, None]
            P = math.exp(g[t, h]) * (np.eye(d_k) - beta[t, h] * (kk @ kk.T))
            S = S @ P + beta[t, h] * (v[t, h][:, None] @ kk.T)
            o[t, h] = S @ q[t, h // grp]
        S_all[h] = S
    return o, S_all[None]


@pytest.mark.parametrize("seed", range(4))
def test_p1_brute_force_literal_form(seed):
    args = rand_problem(seed, 12, 2, 4, 5, 3, unit_k=(seed % 2 == 0))
    o_ref, s_ref = literal_matrix_form(*args)
    o, s = gated_delta_recurrence(*args[:5], state_in=args[5])
    assert rel(o, o_ref) < 1e-13 and rel(s, s_ref) < 1e-13


# ---------------------------------------------------------------- P2 exact rationals
def fraction_recurrence(q, k, v, alpha, beta, s0):
    """Exact rational evaluation of the literal matrix form (one head)."""
    T, d_k = len(k), len(k[0])
    d_v = len(v[0])
    S = [row[:] for row in s0]
    outs = []
    for t in range(T):
        P = [[alpha[t] * ((1 if i == j else 0) - beta[t] * k[t][i] * k[t][j]) for j in range(d_k)]
             for i in range(d_k)]
        S = [[sum(S[a][i] * P[i][j] for i in range(d_k)) + beta[t] * v[t][a] * k[t][j]
              for j in range(d_k)] for a in range(d_v)]
        outs.append([sum(S[a][j] * q[t][j] for j in range(d_k)) for a in range(d_v)])
    return outs, S


def test_p2_exact_rationals():
    rng = np.random.default_rng(7)
    T, d_k, d_v = 6, 3, 2
    fr = lambda lo, hi: Fraction(int(rng.integers(lo, hi)), int(rng.integers(1, 9)))
    q = [[fr(-9, 10) for _ in range(d_k)] for _ in range(T)]
    k = [[fr(-9, 10) for _ in range(d_k)] for _ in range(T)]  # not unit norm
    v = [[fr(-9, 10) for _ in range(d_v)] for _ in range(T)]
    alpha = [Fraction(int(rng.integers(1, 8)), 8) for _ in range(T)]
    beta = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    s0 = [[fr(-5, 6) for _ in range(d_k)] for _ in range(d_v)]
    o_ex, s_ex = fraction_recurrence(q, k, v, alpha, beta, s0)
    f = lambda x: np.array(x, dtype=np.float64)
    o, s = gated_delta_recurrence(f(q)[:, None], f(k)[:, None], f(v)[:, None],
                                  np.log(f(alpha))[:, None], f(beta)[:, None],
                                  state_in=f(s0)[None, None])
    assert rel(o[:, 0], f(o_ex)) < 1e-13
    assert rel(s[0, 0], f(s_ex)) < 1e-13


# ---------------------------------------------------------------- golden fixture
def load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rhs = (x.strip() for x in line.split("=", 1))
            vals[key] = np.array([float(Fraction(x.strip())) for x in rhs.split(",")])
    return vals


def test_golden_hand_worked_T2():
    gv = load_golden("hand_worked_T2.txt")
    q = gv["q"].reshape(2, 1, 2)
    k = gv["k"].reshape(2, 1, 2)
    v = gv["v"].reshape(2, 1, 2)
    g = np.log(gv["alpha"]).reshape(2, 1)
    beta = gv["beta"].reshape(2, 1)
    s0 = gv["S0"].reshape(1, 1, 2, 2)
    o, s = gated_delta_recurrence(q, k, v, g, beta, state_in=s0)
    np.testing.assert_allclose(o.reshape(-1), gv["o"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(s.reshape(-1), gv["S2"], rtol=1e-14, atol=1e-14)
    # the block form must reproduce the same fixture for every block size
    for C in (1, 2, 3):
        o2, s2 = gated_delta_chunk_form(q, k, v, g, beta, C, state_in=s0)
        np.testing.assert_allclose(o2.reshape(-1), gv["o"], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(s2.reshape(-1), gv["S2"], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- P3 delta invariant
def test_p3_delta_invariant():
    """beta = 1 and unit k: the update writes v exactly at key k, so
    S_t k_t = v_t; with q = k the output is v."""
    q, k, v, g, beta, s0 = rand_problem(3, 20, 2, 2, 8, 5)
    beta = np.ones_like(beta)
    o, _ = gated_delta_recurrence(k, k, v, g, beta, state_in=s0)
    assert np.max(np.abs(o - v)) < 1e-13
    # and the state after every prefix satisfies S_t k_t = v_t
    for t in (0, 7, 19):
        _, s = gated_delta_recurrence(q[:t + 1], k[:t + 1], v[:t + 1], g[:t + 1], beta[:t + 1], state_in=s0)
        for h in range(2):
            assert np.max(np.abs(s[0, h] @ k[t, h] - v[t, h])) < 1e-13


# ---------------------------------------------------------------- P4 / P5 closed forms
def test_p4_constancy():
    q, k, v, g, beta, s0 = rand_problem(4, 16, 2, 4, 6, 3)
    o, s = gated_delta_recurrence(q, k, v, np.zeros_like(g), np.zeros_like(beta), state_in=s0)
    grp = 2
    expect = np.einsum("hij,thj->thi", s0[0], np.repeat(q, grp, axis=1))
    assert np.array_equal(s, s0)
    assert np.max(np.abs(o - expect)) < 1e-14


def test_p5_pure_decay():
    q, k, v, g, beta, s0 = rand_problem(5, 16, 2, 2, 6, 3, gate_shift=-1.0)
    o, s = gated_delta_recurrence(q, k, v, g, np.zeros_like(beta), state_in=s0)
    cum = np.exp(np.cumsum(g, axis=0))  # [T, H_v]
    assert rel(s[0], cum[-1][:, None, None] * s0[0]) < 1e-14
    expect = cum[:, :, None] * np.einsum("hij,thj->thi", s0[0], q)
    assert rel(o, expect) < 1e-14


# ---------------------------------------------------------------- P6 orthonormal keys
def test_p6_orthonormal_keys():
    """k_t = e_{pi(t)}: column pi(t) becomes alpha(1-beta) col + beta v, every
    other column is scaled by alpha."""
    rng = np.random.default_rng(6)
    d_k, d_v, T = 6, 3, 6
    perm = rng.permutation(d_k)
    k = np.eye(d_k)[perm][:, None]
    q = rng.standard_normal((T, 1, d_k))
    v = rng.standard_normal((T, 1, d_v))
    g = -rng.uniform(0.1, 2, (T, 1))
    beta = rng.uniform(0, 1, (T, 1))
    s0 = rng.standard_normal((1, 1, d_v, d_k))
    S = s0[0, 0].copy()
    for t in range(T):
        a, b, j = math.exp(g[t, 0]), beta[t, 0], perm[t]
        S = a * S
        S[:, j] = (1 - b) * S[:, j] + b * v[t, 0]
    _, s = gated_delta_recurrence(q, k, v, g, beta, state_in=s0)
    assert rel(s[0, 0], S) < 1e-14


# ---------------------------------------------------------------- P7 two forms agree
@pytest.mark.parametrize("C", [1, 2, 3, 16, 64, 200])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 67])
def test_p7_scan_equals_chunk_form(C, T):
    q, k, v, g, beta, s0 = rand_problem(100 + T + C, T, 2, 4, 8, 5, gate_shift=2.0)
    o1, s1 = gated_delta_recurrence(q, k, v, g, beta, state_in=s0)
    o2, s2 = gated_delta_chunk_form(q, k, v, g, beta, C, state_in=s0)
    assert rel(o2, o1) < 1e-12 and rel(s2, s1) < 1e-12


def test_p7_long_strong_gate():
    q, k, v, g, beta, s0 = rand_problem(77, 1000, 1, 2, 16, 8, gate_shift=2.0)
    o1, s1 = gated_delta_recurrence(q, k, v, g, beta, state_in=s0)
    o2, s2 = gated_delta_chunk_form(q, k, v, g, beta, 64, state_in=s0)
    assert rel(o2, o1) < 1e-12 and rel(s2, s1) < 1e-12


# ---------------------------------------------------------------- P8 linearity
def test_p8_linearity():
    q, k, v, g, beta, s0 = rand_problem(8, 24, 2, 2, 6, 4)
    rng = np.random.default_rng(88)
    v2, s02 = rng.standard_normal(v.shape), rng.standard_normal(s0.shape)
    a, b = 0.7, -1.3
    o1, s1 = gated_delta_recurrence(q, k, v, g, beta, state_in=s0)
    o2, s2 = gated_delta_recurrence(q, k, v2, g, beta, state_in=s02)
    o3, s3 = gated_delta_recurrence(q, k, a * v + b * v2, g, beta, state_in=a * s0 + b * s02)
    assert rel(o3, a * o1 + b * o2) < 1e-12 and rel(s3, a * s1 + b * s2) < 1e-12
    o4, s4 = gated_delta_recurrence(2.5 * q, k, v, g, beta, state_in=s0)
    assert rel(o4, 2.5 * o1) < 1e-14 and rel(s4, s1) == 0.0


# ---------------------------------------------------------------- P9 split / carry
@pytest.mark.parametrize("split", [0, 1, 13, 40])
def test_p9_split_carry(split):
    q, k, v, g, beta, s0 = rand_problem(9, 40, 2, 4, 6, 4)
    o, s = gated_delta_recurrence(q, k, v, g, beta, state_in=s0)
    oa, sa = gated_delta_recurrence(q[:split], k[:split], v[:split], g[:split], beta[:split], state_in=s0)
    ob, sb = gated_delta_recurrence(q[split:], k[split:], v[split:], g[split:], beta[split:], state_in=sa)
    assert rel(np.concatenate([oa, ob]), o) < 1e-13 and rel(sb, s) < 1e-13


# ---------------------------------------------------------------- P10 ragged batch
def test_p10_ragged_equals_independent():
    lens = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, g, beta, s0 = rand_problem(10, T, 2, 4, 6, 3, N=len(lens))
    o, s = gated_delta_recurrence(q, k, v, g, beta, cu_seqlens=cu, state_in=s0)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, sn = gated_delta_recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], state_in=s0[n:n + 1])
        assert np.array_equal(o[a:b], on) and np.array_equal(s[n], sn[0])
    assert np.array_equal(s[1], s0[1])  # zero-length sequence passes its state through
    oc, sc = gated_delta_chunk_form(q, k, v, g, beta, 4, cu_seqlens=cu, state_in=s0)
    assert rel(oc, o) < 1e-12 and rel(sc, s) < 1e-12


# ---------------------------------------------------------------- P11 head sharing
def test_p11_gqa_mapping():
    q, k, v, g, beta, s0 = rand_problem(11, 10, 2, 6, 5, 3)
    o, s = gated_delta_recurrence(q, k, v, g, beta, state_in=s0)
    qr, kr = np.repeat(q, 3, axis=1), np.repeat(k, 3, axis=1)
    o2, s2 = gated_delta_recurrence(qr, kr, v, g, beta, state_in=s0)
    assert np.array_equal(o, o2) and np.array_equal(s, s2)
    assert list(qk_head_of(6, 2)) == [0, 0, 0, 1, 1, 1]


# ---------------------------------------------------------------- P12 decode == prefill
def test_p12_decode_equals_prefill():
    q, k, v, g, beta, s0 = rand_problem(12, 7, 2, 4, 6, 3)
    o, s = gated_delta_recurrence(q, k, v, g, beta, state_in=s0)
    S = s0
    for t in range(7):
        ot, S = gated_delta_decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], S)
        assert rel(ot[0], o[t]) < 1e-13
    assert rel(S, s) < 1e-13
    # batched decode: B sequences at once == each alone
    B = 3
    qb, kb, vb, gb, bb, sb = rand_problem(13, B, 2, 4, 6, 3, N=B)
    ob, snew = gated_delta_decode_step(qb, kb, vb, gb, bb, sb)
    for i in range(B):
        oi, si = gated_delta_recurrence(qb[i:i + 1], kb[i:i + 1], vb[i:i + 1], gb[i:i + 1], bb[i:i + 1],
                                        state_in=sb[i:i + 1])
        assert np.array_equal(ob[i], oi[0]) and np.array_equal(snew[i], si[0])


# ---------------------------------------------------------------- P13 rounding floor
def test_p13_bf16_rounding_floor():
    """Rounding the fp64 output to bf16 costs ~1e-3 relative (per head,
    Frobenius), so a 3e-3 bound on bf16 outputs is attainable."""
    inp = make_prefill([256], 2, 4, 32, 32, "bf16", 2.0, None, seed=3)
    o, _ = gated_delta_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta)
    ob = round_to_bf16(o.astype(np.float32)).astype(np.float64)
    worst = max(rel(ob[:, h], o[:, h]) for h in range(4))
    assert 5e-4 < worst < 2e-3


def test_round_to_bf16_ties_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-39], dtype=np.float32)
    r = round_to_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0 + 4 * 2 ** -8) and r[3] == -2.5
    bits = r.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_tiny_fp32_shapes_and_distributions():
    inp = tiny_fp32_prefill()
    assert inp.q.shape == (64, 2, 16) and inp.v.shape == (64, 2, 16) and inp.chunk_size == 16
    assert np.allclose(np.linalg.norm(inp.q, axis=-1), 1, atol=1e-6)
    assert np.all(inp.g < 0) and np.all((inp.beta > 0) & (inp.beta < 1))
    o1, s1 = gated_delta_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta)
    o2, s2 = gated_delta_chunk_form(inp.q, inp.k, inp.v, inp.g, inp.beta, 16)
    assert rel(o2, o1) < 1e-12 and rel(s2, s1) < 1e-12


# ---------------------------------------------------------------- planted mistakes
def _mutant(kind):
    """A copy of the token loop with one plausible mistake planted in it."""
    def run(q, k, v, g, beta, cu_seqlens=None, state_in=None):
        T, h_qk, d_k = q.shape
        h_v, d_v = v.shape[1], v.shape[2]
        qmap = np.arange(h_v) // (h_v // h_qk)
        if kind == "interleaved_heads":
            qmap = np.arange(h_v) % h_qk
        S = np.zeros((h_v, d_v, d_k)) if state_in is None else np.array(state_in[0], dtype=float)
        o = np.zeros((T, h_v, d_v))
        for t in range(T):
            kt, qt = k[t, qmap], q[t, qmap]
            a = np.exp(g[t])
            p = np.einsum("hij,hj->hi", S, kt)
            if kind == "alpha_after_delta":
                u = beta[t][:, None] * (v[t] - p)
            elif kind == "sign":
                u = beta[t][:, None] * (v[t] + a[:, None] * p)
            elif kind == "transposed_state":
                p = np.einsum("hji,hj->hi", S, kt) if d_v == d_k else p
                u = beta[t][:, None] * (v[t] - a[:, None] * p)
            else:
                u = beta[t][:, None] * (v[t] - a[:, None] * p)
            Sn = a[:, None, None] * S + u[:, :, None] * kt[:, None, :]
            if kind == "no_decay":
                Sn = S + u[:, :, None] * kt[:, None, :]
            o[t] = np.einsum("hij,hj->hi", S if kind == "pre_update_output" else Sn, qt)
            S = Sn
        return o, S[None]
    return run


@pytest.mark.parametrize("kind", ["alpha_after_delta", "sign", "transposed_state", "no_decay",
                                  "pre_update_output", "interleaved_heads"])
def test_pins_catch_planted_mistakes(kind):
    fn = _mutant(kind)
    failures = 0
    # golden fixture
    gv = load_golden("hand_worked_T2.txt")
    o, s = fn(gv["q"].reshape(2, 1, 2), gv["k"].reshape(2, 1, 2), gv["v"].reshape(2, 1, 2),
              np.log(gv["alpha"]).reshape(2, 1), gv["beta"].reshape(2, 1), state_in=gv["S0"].reshape(1, 1, 2, 2))
    failures += not (np.allclose(o.reshape(-1), gv["o"]) and np.allclose(s.reshape(-1), gv["S2"]))
    # brute force on the literal form with shared heads
    args = rand_problem(1, 12, 2, 4, 5, 5)
    o_ref, s_ref = literal_matrix_form(*args)
    o, s = fn(*args[:5], state_in=args[5])
    failures += not (rel(o, o_ref) < 1e-12 and rel(s, s_ref) < 1e-12)
    assert failures >= 1


# ---------------------------------------------------------------- fused decode step
# The decode path fuses the preparation of queries and keys and the recurrent
# update with its normalisation (section "Reduce state and intermediate
# traffic"); gated_delta_decode_fused takes the raw inputs.  Pinned by a
# hand-worked fixture, closed forms of the activations and scale invariances.
def load_golden_cases(name):
    """{case: {key: fp64 array}} from 'CASE.key = a, b, ...' lines; a value is
    a fraction or ln(fraction)."""
    cases = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rhs = (x.strip() for x in line.split("=", 1))
            case, key = key.split(".", 1)
            vals = []
            for x in rhs.split(","):
                x = x.strip()
                vals.append(math.log(Fraction(x[3:-1])) if x.startswith("ln(") else float(Fraction(x)))
            cases.setdefault(case, {})[key] = np.array(vals)
    return cases


def _run_fused_case(c, fn=gated_delta_decode_fused):
    return fn(c["q_raw"].reshape(1, 1, 2), c["k_raw"].reshape(1, 1, 2), c["v"].reshape(1, 1, 2),
              c["g_raw"].reshape(1, 1), c["b_raw"].reshape(1, 1), c["S0"].reshape(1, 1, 2, 2),
              gate_bias=c["gate_bias"], gate_scale=c["gate_scale"], norm_weight=c["w"],
              qk_eps=float(c["qk_eps"][0]), norm_eps=float(c["norm_eps"][0]))


@pytest.mark.parametrize("case", ["A", "B", "C"])
def test_golden_decode_fused(case):
    c = load_golden_cases("hand_worked_decode_fused.txt")[case]
    out, s1 = _run_fused_case(c)
    np.testing.assert_allclose(out.reshape(-1), c["out"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(s1.reshape(-1), c["S1"], rtol=1e-14, atol=1e-14)


def test_activation_closed_forms():
    # softplus(0) = ln 2, softplus(ln(e - 1)) = 1, softplus(x) - softplus(-x) = x
    assert abs(softplus(0.0) - math.log(2.0)) < 1e-16
    assert abs(softplus(math.log(math.e - 1.0)) - 1.0) < 1e-15
    x = np.linspace(-40, 40, 81)
    np.testing.assert_allclose(softplus(x) - softplus(-x), x, rtol=0, atol=1e-13)
    assert softplus(800.0) == 800.0 and 0.0 < softplus(-700.0) < 1e-300 and softplus(-800.0) == 0.0
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(x) + sigmoid(-x) = 1, no overflow at the ends
    assert sigmoid(0.0) == 0.5
    assert abs(sigmoid(math.log(3.0)) - 0.75) < 1e-15
    np.testing.assert_allclose(sigmoid(x) + sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert sigmoid(800.0) == 1.0 and sigmoid(-800.0) == 0.0


def _fused_problem(seed, B=3, h_qk=2, h_v=4, d_k=8, d_v=6):
    rng = np.random.default_rng(seed)
    return dict(q_raw=rng.normal(size=(B, h_qk, d_k)), k_raw=rng.normal(size=(B, h_qk, d_k)),
                v=rng.normal(size=(B, h_v, d_v)), g_raw=rng.normal(size=(B, h_v)),
                beta_raw=rng.normal(size=(B, h_v)), state=rng.normal(size=(B, h_v, d_v, d_k)),
                gate_bias=rng.normal(size=h_v), gate_scale=rng.uniform(0.5, 2.0, size=h_v),
                norm_weight=rng.normal(size=d_v))


def test_fused_scale_invariances():
    p = _fused_problem(0)
    out, s = gated_delta_decode_fused(**p, qk_eps=0.0, norm_eps=0.0)
    # q and k enter only through their directions
    p2 = dict(p, q_raw=p["q_raw"] * 3.7, k_raw=p["k_raw"] * 0.21)
    out2, s2 = gated_delta_decode_fused(**p2, qk_eps=0.0, norm_eps=0.0)
    assert rel(out2, out) < 1e-13 and rel(s2, s) < 1e-13
    # (v, state) -> c (v, state) scales the state by c and leaves the normalised output alone
    p3 = dict(p, v=p["v"] * 5.0, state=p["state"] * 5.0)
    out3, s3 = gated_delta_decode_fused(**p3, qk_eps=0.0, norm_eps=0.0)
    assert rel(out3, out) < 1e-13 and rel(s3, 5.0 * s) < 1e-13
    # the output's RMS over d_v is |norm_weight|'s when norm_eps = 0 and the weight is one
    out4, _ = gated_delta_decode_fused(**dict(p, norm_weight=None), qk_eps=0.0, norm_eps=0.0)
    np.testing.assert_allclose(np.mean(out4 ** 2, axis=-1), 1.0, rtol=1e-13)


def test_fused_prepared_inputs_match_decode_step():
    # With unit q, k, g_raw = softplus^-1(-g) and beta_raw = logit(beta), the
    # fused step's state equals the plain step's, and its output is the plain
    # output normalised.
    p = _fused_problem(1)
    q = p["q_raw"] / np.linalg.norm(p["q_raw"], axis=-1, keepdims=True)
    k = p["k_raw"] / np.linalg.norm(p["k_raw"], axis=-1, keepdims=True)
    g = -np.abs(p["g_raw"]) - 0.05
    beta = 1.0 / (1.0 + np.exp(-p["beta_raw"]))
    o, s = gated_delta_decode_step(q, k, p["v"], g, beta, p["state"])
    g_raw = np.log(np.expm1(-g))  # softplus(g_raw) = -g
    out, s_f = gated_delta_decode_fused(q, k, p["v"], g_raw, p["beta_raw"], p["state"], qk_eps=0.0, norm_eps=0.0)
    assert rel(s_f, s) < 1e-13
    assert rel(out, o / np.sqrt(np.mean(o ** 2, axis=-1, keepdims=True))) < 1e-13


def _fused_mutant(kind):
    """A copy of the fused step with one plausible mistake planted in it."""
    def run(q_raw, k_raw, v, g_raw, beta_raw, state, gate_bias=None, gate_scale=None, norm_weight=None,
            qk_eps=1e-6, norm_eps=1e-6):
        h_v, d_v = v.shape[1], v.shape[2]
        bias = np.zeros(h_v) if gate_bias is None else gate_bias
        scale = np.ones(h_v) if gate_scale is None else gate_scale
        w = np.ones(d_v) if norm_weight is None else norm_weight
        nq = np.sum(q_raw * q_raw, axis=-1, keepdims=True) + qk_eps
        nk = np.sum(k_raw * k_raw, axis=-1, keepdims=True) + qk_eps
        q = q_raw / (nq if kind == "qk_no_sqrt" else np.sqrt(nq))
        k = k_raw / np.sqrt(nk)
        sp = np.logaddexp(0.0, g_raw + (0.0 if kind == "no_bias" else bias))
        g = (scale * sp) if kind == "gate_sign" else -scale * sp
        beta = np.logaddexp(0.0, beta_raw) if kind == "beta_softplus" else 1.0 / (1.0 + np.exp(-beta_raw))
        o, s = gated_delta_decode_step(q, k, v, g, beta, state)
        if kind == "norm_eps_outside":
            out = o / (np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) + norm_eps) * w
        elif kind == "norm_over_heads":
            out = o / np.sqrt(np.mean(o * o, axis=-2, keepdims=True) + norm_eps) * w
        elif kind == "weight_before_norm":
            ow = o * w
            out = ow / np.sqrt(np.mean(ow * ow, axis=-1, keepdims=True) + norm_eps)
        else:
            out = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + norm_eps) * w
        return out, s
    return run


@pytest.mark.parametrize("kind", ["qk_no_sqrt", "no_bias", "gate_sign", "beta_softplus", "norm_eps_outside",
                                  "norm_over_heads", "weight_before_norm"])
def test_fused_pins_catch_planted_mistakes(kind):
    fn = _fused_mutant(kind)
    cases = load_golden_cases("hand_worked_decode_fused.txt")
    failures = 0
    for c in cases.values():
        out, s1 = _run_fused_case(c, fn)
        failures += not (np.allclose(out.reshape(-1), c["out"]) and np.allclose(s1.reshape(-1), c["S1"]))
    # the invariance pin with several heads
    p = _fused_problem(0)
    out, _ = fn(**dict(p, norm_weight=None), qk_eps=0.0, norm_eps=0.0)
    failures += not np.allclose(np.mean(out ** 2, axis=-1), 1.0, rtol=1e-12)
    assert failures >= 1


# ---------------------------------------------------------------- grouped GEMM on 4-bit weights
# Section "Dequantize the weights during the matrix multiplication": 4-bit
# codes, a bf16 scale and bias per group of 64 weights, weights rebuilt in bf16
# before the multiplication.  Pinned by a hand-worked fixture (which also fixes
# the bf16 rounding and the nibble order), an independent brute-force loop,
# closed forms and planted mistakes.
def _expand(tok):
    """'v*n', '[a;b]*n' or a plain token -> list of strings."""
    tok = tok.strip()
    if "*" in tok:
        body, n = tok.rsplit("*", 1)
        items = body[1:-1].split(";") if body.startswith("[") else [body]
        return [t.strip() for t in items] * int(n)
    return [tok]


def load_q4_fixture():
    vals = {}
    with open(os.path.join(GOLDEN, "hand_worked_q4_gemm.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rhs = (x.strip() for x in line.split("=", 1))
            toks = [t for part in rhs.split(",") for t in _expand(part)]
            if key.startswith("codes"):
                vals[key] = np.array([int(t, 16) for t in toks], dtype=np.uint8)
            else:
                vals[key] = np.array([float(Fraction(t)) for t in toks])
    codes = np.stack([np.stack([vals["codes_e0_n0"], vals["codes_e0_n1"]]),
                      np.stack([vals["codes_e1_n0"], vals["codes_e1_n1"]])])  # [2, 2, 64]
    x = np.stack([vals["x_row0"], vals["x_row1"], vals["x_row2"]])
    return dict(x=x, codes=codes, scales=vals["scales"].reshape(2, 2, 2), biases=vals["biases"].reshape(2, 2, 2),
                offsets=vals["offsets"].astype(np.int64), y=vals["y"].reshape(3, 2))


def test_golden_q4_gemm():
    f = load_q4_fixture()
    assert f["codes"].shape == (2, 2, 64) and f["x"].shape == (3, 128)
    y = grouped_gemm_q4(f["x"], f["codes"], f["scales"], f["biases"], f["offsets"])
    np.testing.assert_array_equal(y, f["y"])  # every value and partial sum is exact in fp64


def test_round_bf16_definition():
    # bf16 keeps 8 significant bits: values on the grid stay, midpoints go to the even neighbour
    assert round_bf16(1.0) == 1.0 and round_bf16(-3.03125) == -3.03125
    assert round_bf16(1 + 2.0 ** -8) == 1.0                       # tie: 1.0 is even
    assert round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6          # tie: up to the even neighbour
    assert round_bf16(1 + 2.0 ** -8 + 2.0 ** -20) == 1 + 2.0 ** -7  # past the tie: up
    assert round_bf16(387 / 128) == 3.03125
    x = np.random.default_rng(3).normal(size=2000).astype(np.float32).astype(np.float64)
    r = round_bf16(x)
    # on the bf16 grid (low 16 bits zero) and within half a unit in the last place
    assert np.all((r.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(x))) - 7)
    assert np.all(np.abs(r - x) <= ulp / 2)


def _q4_problem(seed, E=4, N=8, K=128, rows=(3, 0, 5, 1)):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    scales = round_bf16(rng.uniform(0.001, 0.1, size=(E, N, K // 64)).astype(np.float32).astype(np.float64))
    biases = round_bf16(rng.uniform(-0.5, 0.5, size=(E, N, K // 64)).astype(np.float32).astype(np.float64))
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    x = rng.normal(size=(int(off[-1]), K))
    return x, codes, scales, biases, off


def _brute_q4(x, codes, scales, biases, off):
    """Triple loop over rows, columns and k, with the nibble taken by divmod."""
    E, N, half = codes.shape
    y = np.zeros((x.shape[0], N))
    for e in range(E):
        for r in range(int(off[e]), int(off[e + 1])):
            for n in range(N):
                acc = 0.0
                for i in range(half):
                    hi, lo = divmod(int(codes[e, n, i]), 16)
                    for k, c in ((2 * i, lo), (2 * i + 1, hi)):
                        w = float(round_bf16(scales[e, n, k // 64] * c + biases[e, n, k // 64]))
                        acc += x[r, k] * w
                y[r, n] = acc
    return y


def test_q4_gemm_brute_force_and_empty_experts():
    x, codes, scales, biases, off = _q4_problem(5)
    y = grouped_gemm_q4(x, codes, scales, biases, off)
    np.testing.assert_allclose(y, _brute_q4(x, codes, scales, biases, off), rtol=1e-12, atol=1e-12)
    assert y.shape == (9, 8)


def test_q4_closed_forms():
    E, N, K = 2, 3, 128
    codes = np.full((E, N, K // 2), 0x77, dtype=np.uint8)  # every code 7
    scales = np.full((E, N, 2), 0.25)
    biases = np.full((E, N, 2), -1.0)
    x = np.random.default_rng(1).normal(size=(5, K))
    off = np.array([0, 2, 5])
    # constant weight 7/4 - 1 = 3/4: y = 3/4 * row sum
    np.testing.assert_allclose(grouped_gemm_q4(x, codes, scales, biases, off),
                               0.75 * np.repeat(x.sum(axis=1, keepdims=True), N, axis=1), rtol=1e-13)
    # one-hot rows read one rebuilt weight: x = e_k gives y[n] = w[e, n, k]
    c2 = np.random.default_rng(2).integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    w = dequantize_q4(c2, scales, biases)
    eye = np.eye(K)[[0, 1, 64, 127]]
    y = grouped_gemm_q4(eye, c2, scales, biases, np.array([0, 4, 4]))
    np.testing.assert_array_equal(y, w[0][:, [0, 1, 64, 127]].T)
    # a zero scale leaves the bias
    np.testing.assert_array_equal(dequantize_q4(c2, np.zeros((E, N, 2)), biases), np.full((E, N, K), -1.0))


def _q4_mutant(kind):
    def run(x, codes, scales, biases, off, group=64):
        codes = np.asarray(codes)
        lo, hi = (codes & 0x0F).astype(float), (codes >> 4).astype(float)
        if kind == "nibble_swap":
            lo, hi = hi, lo
        q = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], -1)
        g = 32 if kind == "group_32" else group
        s = np.repeat(scales, g, axis=-1)[..., :q.shape[-1]]
        b = np.repeat(biases, g, axis=-1)[..., :q.shape[-1]]
        if s.shape[-1] < q.shape[-1]:
            s = np.concatenate([s, s[..., -1:].repeat(q.shape[-1] - s.shape[-1], -1)], -1)
            b = np.concatenate([b, b[..., -1:].repeat(q.shape[-1] - b.shape[-1], -1)], -1)
        if kind == "scale_bias_swap":
            s, b = b, s
        w = s * q + b
        if kind != "no_rounding":
            w = round_bf16(w)
        off2 = np.array(off)
        if kind == "offsets_shift":
            off2 = np.concatenate([[0], off2[1:-1] + 1, [off2[-1]]])
        y = np.zeros((x.shape[0], w.shape[1]))
        for e in range(w.shape[0]):
            a, c = int(off2[e]), int(off2[e + 1])
            y[a:c] = x[a:c] @ w[e].T
        return y
    return run


@pytest.mark.parametrize("kind", ["nibble_swap", "group_32", "scale_bias_swap", "no_rounding", "offsets_shift"])
def test_q4_pins_catch_planted_mistakes(kind):
    f = load_q4_fixture()
    y = _q4_mutant(kind)(f["x"], f["codes"], f["scales"], f["biases"], f["offsets"])
    assert not np.allclose(y, f["y"])


# ---------------------------------------------------------------- decode attention
# Sections "Pack query heads to reuse KV rows" and "Switch attention layouts at
# long contexts": grouped-query softmax attention over a KV cache.  Pinned by a
# hand-worked fixture with rational answers, closed forms (uniform scores give
# the mean value, a dominant key its own value, two keys a logistic weight from
# scipy), invariance to shifting every score and to permuting the cached
# positions, the contiguous head grouping, and planted mistakes.
def load_attention_fixture():
    vals = {}
    with open(os.path.join(GOLDEN, "hand_worked_decode_attention.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rhs = (x.strip() for x in line.split("=", 1))
            toks = [t.strip() for t in rhs.split(",")]
            vals[key] = np.array([np.log(float(Fraction(t[3:-1]))) if t.startswith("ln(") else float(Fraction(t))
                                  for t in toks])
    return dict(q=vals["q"].reshape(2, 4, 2), k=vals["k"].reshape(2, 2, 3, 2), v=vals["v"].reshape(2, 2, 3, 2),
                lens=vals["context_lens"].astype(np.int64), scale=float(vals["scale"][0]),
                out=vals["out"].reshape(2, 4, 2))


def test_golden_decode_attention():
    f = load_attention_fixture()
    o = decode_attention(f["q"], f["k"], f["v"], f["lens"], f["scale"])
    np.testing.assert_allclose(o, f["out"], rtol=1e-13, atol=1e-13)


def _attn_problem(seed, B=2, h_q=8, h_kv=2, T=20, d=6):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(B, h_q, d)), rng.normal(size=(B, h_kv, T, d)), rng.normal(size=(B, h_kv, T, d)),
            rng.integers(1, T + 1, size=B))


def test_attention_closed_forms():
    from scipy.special import expit
    q, k, v, lens = _attn_problem(1)
    # scale 0 (or q = 0): every position weighs the same -> the mean of the cached values
    o = decode_attention(q, k, v, lens, 0.0)
    for b in range(2):
        for h in range(8):
            np.testing.assert_allclose(o[b, h], v[b, h // 4, :lens[b]].mean(axis=0), rtol=1e-12, atol=1e-14)
    # one key far above the rest takes all the weight, even past fp64's exp range
    k2 = k.copy()
    k2[:, :, 3] = 0.0
    q2 = np.zeros_like(q)
    q2[..., 0] = 1.0
    k2[:, :, 3, 0] = 900.0
    o = decode_attention(q2, k2, v, np.array([20, 20]), 1.0)
    for h in range(8):
        np.testing.assert_allclose(o[:, h], v[:, h // 4, 3], rtol=1e-12)
    # two positions: o = sigmoid(s1 - s2) v1 + (1 - sigmoid(s1 - s2)) v2
    o = decode_attention(q, k, v, np.array([2, 2]), 0.7)
    for b in range(2):
        for h in range(8):
            j = h // 4
            w = expit(0.7 * (q[b, h] @ k[b, j, 0] - q[b, h] @ k[b, j, 1]))
            np.testing.assert_allclose(o[b, h], w * v[b, j, 0] + (1 - w) * v[b, j, 1], rtol=1e-12, atol=1e-14)
    # an empty context gives zeros; the value of a one-position context is returned as is
    o = decode_attention(q, k, v, np.array([0, 1]), 1.0)
    np.testing.assert_array_equal(o[0], 0.0)
    np.testing.assert_allclose(o[1], np.repeat(v[1, :, 0], 4, axis=0), rtol=1e-15)


def test_attention_invariances():
    q, k, v, lens = _attn_problem(2, d=5)
    base = decode_attention(q, k, v, lens, 0.4)
    # shifting every score of a head by c: an extra coordinate with k = 1 and q = c / scale
    c = np.random.default_rng(3).normal(size=(2, 8)) * 1000.0
    q_ext = np.concatenate([q, (c / 0.4)[..., None]], axis=-1)
    k_ext = np.concatenate([k, np.ones(k.shape[:-1] + (1,))], axis=-1)
    v_ext = np.concatenate([v, np.zeros(v.shape[:-1] + (1,))], axis=-1)
    np.testing.assert_allclose(decode_attention(q_ext, k_ext, v_ext, lens, 0.4)[..., :5], base, rtol=1e-9, atol=1e-12)
    # permuting the cached positions (keys and values together) changes nothing
    T = k.shape[2]
    lens_full = np.array([T, T])
    full = decode_attention(q, k, v, lens_full, 0.4)
    perm = np.random.default_rng(4).permutation(T)
    np.testing.assert_allclose(decode_attention(q, k[:, :, perm], v[:, :, perm], lens_full, 0.4), full,
                               rtol=1e-12, atol=1e-14)
    # positions past the context are never read, whatever they hold
    k_nan, v_nan = k.copy(), v.copy()
    for b in range(2):
        k_nan[b, :, lens[b]:] = np.nan
        v_nan[b, :, lens[b]:] = np.inf
    np.testing.assert_array_equal(decode_attention(q, k_nan, v_nan, lens, 0.4), base)
    # contiguous head groups: sharing 2 KV heads equals 8 KV heads repeated in blocks of 4
    np.testing.assert_array_equal(decode_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), lens, 0.4),
                                  base)
    # scale folds into q
    np.testing.assert_allclose(decode_attention(0.4 * q, k, v, lens, 1.0), base, rtol=1e-12, atol=1e-14)


def _attn_mutant(kind):
    def run(q, k, v, lens, scale):
        B, h_q, d = q.shape
        h_kv = k.shape[1]
        o = np.zeros((B, h_q, d))
        for b in range(B):
            n = int(lens[b]) + (1 if kind == "one_past_context" else 0)
            for h in range(h_q):
                j = h % h_kv if kind == "interleaved_heads" else h // (h_q // h_kv)
                kk, vv = (v, k) if kind == "keys_values_swapped" else (k, v)
                sc = 1.0 / np.sqrt(d) if kind == "fixed_scale" else scale
                s = sc * (kk[b, j, :n] @ q[b, h])
                if kind == "no_max_shift":
                    w = np.exp(s)
                else:
                    w = np.exp(s - s.max())
                if kind == "unnormalised":
                    o[b, h] = w @ vv[b, j, :n]
                else:
                    o[b, h] = (w / w.sum()) @ vv[b, j, :n]
        return o
    return run


@pytest.mark.parametrize("kind", ["one_past_context", "interleaved_heads", "keys_values_swapped", "fixed_scale",
                                  "unnormalised", "no_max_shift"])
def test_attention_pins_catch_planted_mistakes(kind):
    fn = _attn_mutant(kind)
    f = load_attention_fixture()
    caught = False
    with np.errstate(all="ignore"):
        o = fn(f["q"], f["k"], f["v"], f["lens"], f["scale"])
        caught |= not np.allclose(o, f["out"])
        q, k, v, lens = _attn_problem(1)
        caught |= not np.allclose(fn(q, k, v, lens, 0.0)[0, 0], v[0, 0, :lens[0]].mean(axis=0))
        k2, q2 = np.zeros_like(k), np.zeros_like(q)
        q2[..., 0] = 1.0
        k2[:, :, 3, 0] = 900.0
        o2 = fn(q2, k2, v, np.array([20, 20]), 1.0)
        caught |= not np.allclose(o2[:, 0], v[:, 0, 3])
    assert caught
