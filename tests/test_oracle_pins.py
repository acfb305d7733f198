"""Pins of the CPU oracle against things other than itself.

Each test fixes the oracle to a value the mathematics determines: the
hand-worked example in tests/golden/, the closed form written out as a triple
sum, library matmuls of the masked matrices, special cases with a closed form
(gamma = 0, a constant key direction, d = 1), invariants the pages state
(causality, exactness of the chunk-parallel scan), algebraic properties of the
combine, and planted mistakes that the pins must catch.
"""

import inspect
import json
import os

import numpy as np
import pytest

import oracle
from oracle import hla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(U, T, d, dv, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((U, T, d)), rng.standard_normal((U, T, d)),
            rng.standard_normal((U, T, dv)))


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


GAMMAS = [None, 0.93, np.array([0.8, 0.97, 1.0])]


# --- hand-worked example ------------------------------------------------------

def test_hand_example_exact():
    with open(os.path.join(GOLDEN, "hand_example_d1.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"]).reshape(1, -1, 1)
    k = np.array(ex["k"]).reshape(1, -1, 1)
    v = np.array(ex["v"]).reshape(1, -1, 1)
    for case in ex["cases"]:
        g = case["gamma"]
        want_num = np.array(case["num"])
        want_den = np.array(case["den"])
        num, den, _ = O.serial(q, k, v, g)
        assert np.array_equal(num[0, :, 0], want_num), (g, num)
        assert np.array_equal(den[0], want_den), (g, den)
        bn, bd = O.brute(q, k, v, g)
        assert np.array_equal(bn[0, :, 0], want_num) and np.array_equal(bd[0], want_den)
        for c in (1, 3):
            cn, cd, _, _ = O.chunk_scan_forward(q, k, v, c, g)
            assert np.allclose(cn[0, :, 0], want_num, rtol=0, atol=1e-12)
            assert np.allclose(cd[0], want_den, rtol=0, atol=1e-12)


# --- closed form --------------------------------------------------------------

def _golden_normalise_cases():
    from fractions import Fraction
    with open(os.path.join(GOLDEN, "hand_example_d1.json")) as f:
        ex = json.load(f)
    by_gamma = {c["gamma"]: c for c in ex["cases"]}
    for c in ex["normalise"]["cases"]:
        base = by_gamma[c["gamma"]]
        want = np.array([float(Fraction(x)) for x in c["o"]])
        yield np.array(base["num"]), np.array(base["den"]), c["eps"], want


def test_normalise_hand_example():
    """o = num / (den + eps) on the hand-worked example, eps != 0 and one
    negative denominator (gamma = 1, t = 3: den = -5)."""
    seen_negative = False
    for num, den, eps, want in _golden_normalise_cases():
        got = O.normalise(num[None, :, None], den[None, :], eps)[0, :, 0]
        assert rel(got, want) < 1e-15, (eps, got, want)
        seen_negative |= bool(np.any(den < 0))
    assert seen_negative


NORMALISE_MUTANTS = [
    ("/ (_f64(den)[..., None] + float(eps))", "/ (np.abs(_f64(den))[..., None] + float(eps))"),
    ("/ (_f64(den)[..., None] + float(eps))", "/ (_f64(den)[..., None] - float(eps))"),
    ("return _f64(num) / (_f64(den)[..., None] + float(eps))",
     "return (_f64(num) + float(eps)) / _f64(den)[..., None]"),
    ("return _f64(num) / (_f64(den)[..., None] + float(eps))",
     "return _f64(num) / _f64(den)[..., None] + float(eps)"),
]


@pytest.mark.parametrize("old,new", NORMALISE_MUTANTS)
def test_normalise_pin_catches_planted_mistakes(old, new):
    bad = _mutant(O.normalise, old, new)
    caught = False
    for num, den, eps, want in _golden_normalise_cases():
        got = bad(num[None, :, None], den[None, :], eps)[0, :, 0]
        caught |= rel(got, want) > 1e-9
    assert caught


@pytest.mark.parametrize("gamma", GAMMAS)
def test_serial_matches_brute_triple_sum(gamma):
    q, k, v = rnd(3, 18, 4, 3, seed=1)
    num, den, _ = O.serial(q, k, v, gamma)
    bn, bd = O.brute(q, k, v, gamma)
    assert rel(num, bn) < 1e-12
    assert rel(den, bd) < 1e-12


@pytest.mark.parametrize("gamma", GAMMAS)
def test_serial_matches_matrix_form(gamma):
    q, k, v = rnd(3, 160, 8, 5, seed=2)
    num, den, _ = O.serial(q, k, v, gamma)
    mn, md = O.matrix_form(q, k, v, gamma)
    assert rel(num, mn) < 1e-11
    assert rel(den, md) < 1e-11


def test_gamma_zero_keeps_only_the_diagonal():
    # gamma = 0: only i = j = t survives: o_t = (q_t.k_t)^2 v_t.
    q, k, v = rnd(2, 12, 5, 4, seed=3)
    num, den, _ = O.serial(q, k, v, 0.0)
    s = np.sum(q * k, axis=-1)
    assert rel(num, (s * s)[..., None] * v) < 1e-13
    assert rel(den, s * s) < 1e-13


def test_constant_key_direction_counts_i_le_j():
    # k_i = kappa * e for all i: (q_t.k_i)(q_j.k_i) = kappa^2 (q_t.e)(q_j.e) and
    # there are exactly j keys with i <= j, so
    # num_t = kappa^2 (q_t.e) sum_{j<=t} j (q_j.e) v_j  (gamma = 1).
    U, T, d, dv = 2, 30, 6, 3
    q, _, v = rnd(U, T, d, dv, seed=4)
    e = np.zeros(d)
    e[2] = 1.0
    kappa = 1.5
    k = np.broadcast_to(kappa * e, (U, T, d)).copy()
    num, den, _ = O.serial(q, k, v)
    qe = q[..., 2]
    j = np.arange(1, T + 1)
    want = kappa ** 2 * qe[..., None] * np.cumsum((j * qe)[..., None] * v, axis=1)
    want_den = kappa ** 2 * qe * np.cumsum(j * qe, axis=1)
    assert rel(num, want) < 1e-12
    assert rel(den, want_den) < 1e-12


def test_d1_cumsum_form():
    # d = 1, gamma = 1: o_t = q_t sum_{j<=t} q_j v_j sum_{i<=j} k_i^2.
    q, k, v = rnd(2, 40, 1, 3, seed=5)
    num, den, _ = O.serial(q, k, v)
    K = np.cumsum(k[..., 0] ** 2, axis=1)
    want = q[..., 0:1] * np.cumsum((q[..., 0] * K)[..., None] * v, axis=1)
    assert rel(num, want) < 1e-12
    assert rel(den, q[..., 0] * np.cumsum(q[..., 0] * K, axis=1)) < 1e-12


# --- invariants the pages state ----------------------------------------------

@pytest.mark.parametrize("gamma", [None, 0.9])
def test_causality(gamma):
    q, k, v = rnd(2, 40, 4, 3, seed=6)
    num, den, _ = O.serial(q, k, v, gamma)
    t0 = 17
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    rng = np.random.default_rng(9)
    q2[:, t0 + 1:] = rng.standard_normal(q2[:, t0 + 1:].shape)
    k2[:, t0 + 1:] *= -3.0
    v2[:, t0 + 1:] = 7.0
    num2, den2, _ = O.serial(q2, k2, v2, gamma)
    assert np.array_equal(num[:, :t0 + 1], num2[:, :t0 + 1])
    assert np.array_equal(den[:, :t0 + 1], den2[:, :t0 + 1])
    assert not np.allclose(num[:, t0 + 1:], num2[:, t0 + 1:])


def test_linear_in_v_and_scaling():
    q, k, v = rnd(2, 25, 4, 3, seed=7)
    num, den, _ = O.serial(q, k, v, 0.95)
    _, _, v2 = rnd(2, 25, 4, 3, seed=8)
    n2, _, _ = O.serial(q, k, v2, 0.95)
    n12, d12, _ = O.serial(q, k, 2.0 * v - 3.0 * v2, 0.95)
    assert rel(n12, 2.0 * num - 3.0 * n2) < 1e-12
    assert rel(d12, den) < 1e-14
    # q appears twice and k twice in every term: num, den scale as a^2 b^2,
    # and the ratio-normalised output (eps = 0) is invariant.
    na, da, _ = O.serial(1.7 * q, 0.6 * k, v, 0.95)
    assert rel(na, (1.7 * 0.6) ** 2 * num) < 1e-12
    assert rel(da, (1.7 * 0.6) ** 2 * den) < 1e-12
    assert rel(O.normalise(na, da, 0.0), O.normalise(num, den, 0.0)) < 1e-10


def test_den_is_num_with_unit_values():
    q, k, _ = rnd(2, 30, 5, 1, seed=10)
    ones = np.ones((2, 30, 1))
    num, den, _ = O.serial(q, k, ones, 0.9)
    assert rel(num[..., 0], den) < 1e-13


# --- segment summaries, combine, Blelloch scan --------------------------------

@pytest.mark.parametrize("gamma", GAMMAS)
def test_summary_sums_match_recurrence(gamma):
    q, k, v = rnd(3, 37, 5, 4, seed=11)
    a = O.segment_summary(q, k, v, gamma)
    b = O.segment_summary_sums(q, k, v, gamma)
    for key in "SCmGh":
        assert rel(a[key], b[key]) < 1e-12, key


@pytest.mark.parametrize("gamma", GAMMAS)
def test_combine_associative_with_identity(gamma):
    q, k, v = rnd(3, 30, 4, 3, seed=12)
    A = O.segment_summary(q[:, :7], k[:, :7], v[:, :7], gamma)
    B = O.segment_summary(q[:, 7:19], k[:, 7:19], v[:, 7:19], gamma)
    C = O.segment_summary(q[:, 19:], k[:, 19:], v[:, 19:], gamma)
    left = O.combine(O.combine(A, B, gamma), C, gamma)
    right = O.combine(A, O.combine(B, C, gamma), gamma)
    whole = O.segment_summary(q, k, v, gamma)
    e = O.identity_summary(3, 4, 3)
    for key in "SCmGh":
        assert rel(left[key], right[key]) < 1e-13
        assert rel(left[key], whole[key]) < 1e-12
        assert np.array_equal(O.combine(e, A, gamma)[key], A[key])
        assert np.array_equal(O.combine(A, e, gamma)[key], A[key])


@pytest.mark.parametrize("gamma", GAMMAS)
@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 6, 8, 12, 24])
def test_exclusive_scan_reproduces_serial(gamma, chunk):
    # The pages' exactness claim: chunk summaries + exclusive Blelloch scan
    # give the serial activations (n = 24/chunk includes 3, 6, 12, 24).
    q, k, v = rnd(3, 24, 4, 3, seed=13)
    num, den, st = O.serial(q, k, v, gamma)
    cn, cd, pre, total = O.chunk_scan_forward(q, k, v, chunk, gamma)
    assert rel(cn, num) < 1e-12
    assert rel(cd, den) < 1e-12
    # exclusive prefix i = serial state after i*chunk tokens; total = final state
    for i in range(0, 24 // chunk, max(1, 24 // chunk // 3)):
        _, _, sti = O.serial(q[:, :i * chunk], k[:, :i * chunk], v[:, :i * chunk], gamma)
        for key in "SCmGh":
            assert rel(pre[i][key] + 1e-300, sti[key] + 1e-300) < 1e-12 or \
                np.max(np.abs(pre[i][key] - sti[key])) < 1e-12
    for key in "SCmGh":
        assert rel(total[key], st[key]) < 1e-12


def test_decode_continues_the_recurrence():
    q, k, v = rnd(4, 50, 6, 5, seed=14)
    g = np.array([0.9, 1.0, 0.99, 0.5])
    num, den, _ = O.serial(q, k, v, g)
    _, _, st = O.serial(q[:, :40], k[:, :40], v[:, :40], g)
    for t in range(40, 50):
        n1, d1, st = O.decode_step(st, q[:, t], k[:, t], v[:, t], g)
        assert rel(n1, num[:, t]) < 1e-12
        assert rel(d1, den[:, t]) < 1e-12


@pytest.mark.parametrize("gamma", [None, 0.9])
def test_chained_single_sum_identity(gamma):
    # S_t C_t - G_t = sum_{j<=t} g^(2(t-j)) S_j q_j v_j^T: the masked numerator
    # is a first-order linear attention over p_j = S_j q_j.  Checked from the
    # oracle's own states, token by token.
    q, k, v = rnd(2, 20, 4, 3, seed=15)
    g = 1.0 if gamma is None else gamma
    st = O.zero_state(2, 4, 3)
    M = np.zeros((2, 4, 3))
    for t in range(20):
        _, _, st = O.serial(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], gamma, st)
        p = np.matmul(st["S"], q[:, t, :, None])[..., 0]
        M = g * g * M + p[:, :, None] * v[:, t, None, :]
        assert rel(np.matmul(st["S"], st["C"]) - st["G"], M) < 1e-12


# --- planted mistakes ---------------------------------------------------------

def _mutant(func, old, new):
    src = inspect.getsource(func)
    assert old in src, old
    ns = dict(vars(O))
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    return ns[func.__name__]


SERIAL_MUTANTS = [
    # G update reads C after token t was added (drops/duplicates the diagonal)
    ("kC = np.matmul(kt[:, None, :], C)[:, 0, :]",
     "kC = np.matmul(kt[:, None, :], g1[:, :, None] * C + qt[:, :, None] * vt[:, None, :])[:, 0, :]"),
    # wrong sign of the cross summary
    ("- np.matmul(qt[:, None, :], G)[:, 0, :])", "+ np.matmul(qt[:, None, :], G)[:, 0, :])"),
    # decay on G applied once instead of twice
    ("G = g2[:, :, None] * G", "G = g1[:, :, None] * G"),
    # h built from k.q instead of k.m
    ("km = np.sum(kt * m, axis=1)", "km = np.sum(kt * qt, axis=1)"),
    # decay dropped from the new cross term
    ("+ g1[:, :, None] * kt[:, :, None] * kC[:, None, :]", "+ kt[:, :, None] * kC[:, None, :]"),
]


@pytest.mark.parametrize("old,new", SERIAL_MUTANTS)
def test_pins_catch_planted_mistakes_in_serial(old, new):
    bad = _mutant(O.serial, old, new)
    q, k, v = rnd(2, 10, 3, 2, seed=16)
    caught = False
    for gamma in (None, 0.8):
        n_bad, d_bad, _ = bad(q, k, v, gamma)
        bn, bd = O.brute(q, k, v, gamma)
        if rel(n_bad, bn) > 1e-9 or rel(d_bad, bd) > 1e-9:
            caught = True
    assert caught


COMBINE_MUTANTS = [
    ("a3 * np.matmul(B[\"S\"], A[\"C\"])", "a3 * np.matmul(A[\"S\"], B[\"C\"])"),   # cross term swapped
    ("a3 * a3 * A[\"G\"]", "a3 * A[\"G\"]"),                                        # decay power
    ("\"m\": a1 * A[\"m\"] + B[\"m\"]", "\"m\": A[\"m\"] + B[\"m\"]"),              # m not decayed
]


@pytest.mark.parametrize("old,new", COMBINE_MUTANTS)
def test_pins_catch_planted_mistakes_in_combine(old, new):
    bad_combine = _mutant(O.combine, old, new)
    q, k, v = rnd(2, 12, 3, 2, seed=17)
    caught = False
    for gamma in (None, 0.8):
        A = O.segment_summary(q[:, :5], k[:, :5], v[:, :5], gamma)
        B = O.segment_summary(q[:, 5:], k[:, 5:], v[:, 5:], gamma)
        whole = O.segment_summary(q, k, v, gamma)
        got = bad_combine(A, B, gamma)
        if any(rel(got[x], whole[x]) > 1e-9 for x in "SCmGh"):
            caught = True
    assert caught


def test_oracle_module_exports():
    for name in oracle.__all__ if hasattr(oracle, "__all__") else O.__all__:
        assert callable(getattr(O, name))
