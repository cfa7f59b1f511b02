"""The parity measures can see one wrong token in a long sequence (CPU).

An oracle output of one 131072-token sequence (one value head, d = 16, so
that the fp64 token loop finishes in seconds) is rounded to bf16, the best a
bf16 kernel can return.  Rounding alone passes all three measures.  One token
planted wrong fails the per-token measure in every way tried (zeroed,
negated, replaced by another token, halved), while its share of the slice's
Frobenius norm is only about 1/sqrt(131072): a token halved stays within the
Frobenius tolerance, and a zeroed one lands just past it (the 2.8e-3 of the
token adds in quadrature to the 1.5e-3 of the rounding).  A large error on
one element fails the max-norm measure.
"""
import numpy as np
import pytest

from gated_deltanet_linear_delta_amd.workloads import make_prefill, round_to_bf16
from metrics import TOL, TOL_MAX, TOL_TOK, out_errors, seq_errors, state_errors
from oracle import gated_delta_recurrence

T_LONG = 131072


def round_bf16(x):
    # what a bf16 kernel returns at best: fp32, then bf16 to nearest even
    return round_to_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


@pytest.fixture(scope="module")
def long_output():
    inp = make_prefill([T_LONG], 1, 1, 16, 16, "bf16", 2.0, 0.0, seed=131)
    o, s = gated_delta_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta)
    return o, s


def test_rounding_alone_passes(long_output):
    o, s = long_output
    e = out_errors(round_bf16(o), o, [0, T_LONG])
    es = state_errors(s.astype(np.float32).astype(np.float64), s)
    print(f"bf16 rounding of the oracle output: {e}; fp32 state: {es}")
    assert e.ok("bf16") and es.ok("f32")


@pytest.mark.parametrize("how", ["zero", "negate", "other_token", "halve"])
def test_one_wrong_token_is_caught(long_output, how):
    o, _ = long_output
    x = round_bf16(o).copy()
    rms = np.sqrt(np.mean(np.sum(o[:, 0] ** 2, axis=1)))
    norms = np.linalg.norm(o[:, 0], axis=1)
    t = int(np.argmin(np.abs(norms - rms)))  # a token of typical size
    if how == "zero":
        x[t] = 0.0
    elif how == "negate":
        x[t] = -x[t]
    elif how == "other_token":
        x[t] = x[(t + 1000) % T_LONG]
    else:
        x[t] = 0.5 * x[t]
    e = out_errors(x, o, [0, T_LONG])
    print(f"token {t} {how}: {e}")
    if how == "halve":
        assert e.frob <= TOL["bf16"], "half a token's error hides inside the Frobenius measure"
    assert e.tok > TOL_TOK["bf16"], "the per-token measure must catch it"
    assert not e.ok("bf16")


def test_one_wrong_element_fails_max_norm(long_output):
    o, _ = long_output
    x = round_bf16(o).copy()
    i = np.unravel_index(np.argmax(np.abs(o)), o.shape)
    x[i] += 0.05 * np.max(np.abs(o))
    e = out_errors(x, o, [0, T_LONG])
    print(f"one element off by 5% of the slice maximum: {e}")
    assert e.frob <= TOL["bf16"] and e.maxn > TOL_MAX["bf16"]


def test_measures_on_small_cases():
    r = np.zeros((4, 2, 3))
    r[:, 0] = 1.0
    r[:, 1] = [[1.0, 2.0, 2.0]] * 4  # row norm 3
    x = r.copy()
    x[2, 1, 0] += 0.3
    e = seq_errors(x, r)
    # head 1: Frobenius 0.3 / 6, max 0.3 / 2, token 0.3 / max(3, 3)
    assert e.frob == pytest.approx(0.05)
    assert e.maxn == pytest.approx(0.15)
    assert e.tok == pytest.approx(0.1)
    # an all-zero reference slice compares absolute errors
    z = seq_errors(np.full((2, 1, 2), 1e-3), np.zeros((2, 1, 2)))
    assert z.frob == pytest.approx(2e-3) and z.maxn == pytest.approx(1e-3)
    # empty sequences contribute nothing
    assert out_errors(np.zeros((0, 1, 2)), np.zeros((0, 1, 2)), [0, 0]).frob == 0.0
