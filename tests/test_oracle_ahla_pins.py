"""Pins of the oracle's asymmetric variant AHLA (masked A A V, A = Q K^T).

The serial recurrence over the summaries P^KV, m^K, E, n is fixed against the
closed form written out as a triple sum, against two chained masked matmuls
(library products), against gamma = 0 and d = 1 closed forms, causality, the
algebra of its segment combine, exactness of the chunk-parallel form, and
planted mistakes.
"""

import inspect

import numpy as np
import pytest

from oracle import hla_oracle as O


def rnd(U, T, d, dv, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((U, T, d)), rng.standard_normal((U, T, d)),
            rng.standard_normal((U, T, dv)))


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


GAMMAS = [None, 0.93, np.array([0.8, 0.97, 1.0])]


@pytest.mark.parametrize("gamma", GAMMAS)
def test_serial_matches_brute_triple_sum(gamma):
    q, k, v = rnd(3, 16, 4, 3, seed=51)
    num, den, _ = O.serial_ahla(q, k, v, gamma)
    bn, bd = O.brute_ahla(q, k, v, gamma)
    assert rel(num, bn) < 1e-12
    assert rel(den, bd) < 1e-12


@pytest.mark.parametrize("gamma", [None, 0.85])
def test_serial_matches_two_masked_matmuls(gamma):
    # A_L = L o (Q K^T), L[t, i] = g^(t-i) (i <= t): num = A_L (A_L V), den = A_L (A_L 1)
    q, k, v = rnd(2, 64, 6, 4, seed=52)
    T = q.shape[1]
    g = 1.0 if gamma is None else gamma
    t = np.arange(T)
    L = np.where(t[:, None] >= t[None, :], g ** np.maximum(t[:, None] - t[None, :], 0), 0.0)
    num, den, _ = O.serial_ahla(q, k, v, gamma)
    for u in range(q.shape[0]):
        A = L * (q[u] @ k[u].T)
        assert rel(num[u], A @ (A @ v[u])) < 1e-12
        assert rel(den[u], A @ (A @ np.ones(T))) < 1e-12


def test_gamma_zero_keeps_only_the_current_token():
    q, k, v = rnd(2, 12, 4, 3, seed=53)
    num, den, _ = O.serial_ahla(q, k, v, 0.0)
    qk = np.sum(q * k, axis=2)
    assert rel(num, qk[..., None] ** 2 * v) < 1e-12
    assert rel(den, qk ** 2) < 1e-12


@pytest.mark.parametrize("gamma", [None, 0.9])
def test_d1_nested_running_sums(gamma):
    # d = 1: r_i = q_i sum_{j<=i} g^(i-j) k_j v_j, o_t = q_t sum_{i<=t} g^(t-i) k_i r_i
    q, k, v = rnd(2, 40, 1, 3, seed=54)
    g = 1.0 if gamma is None else gamma
    T = q.shape[1]
    inner, outer = np.zeros((2, 3)), np.zeros((2, 3))
    want = np.zeros((2, T, 3))
    for t in range(T):
        inner = g * inner + k[:, t, 0:1] * v[:, t]
        r = q[:, t, 0:1] * inner
        outer = g * outer + k[:, t, 0:1] * r
        want[:, t] = q[:, t, 0:1] * outer
    num, _, _ = O.serial_ahla(q, k, v, gamma)
    assert rel(num, want) < 1e-12


def test_differs_from_the_symmetric_operator():
    q, k, v = rnd(1, 10, 3, 2, seed=55)
    na, _, _ = O.serial_ahla(q, k, v)
    nh, _, _ = O.serial(q, k, v)
    assert rel(na, nh) > 1e-2


@pytest.mark.parametrize("gamma", [None, 0.9])
def test_causality(gamma):
    q, k, v = rnd(2, 30, 4, 3, seed=56)
    num, den, _ = O.serial_ahla(q, k, v, gamma)
    t0 = 13
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, t0 + 1:] *= -2.0
    k2[:, t0 + 1:] += 1.0
    v2[:, t0 + 1:] = 5.0
    n2, d2, _ = O.serial_ahla(q2, k2, v2, gamma)
    assert np.array_equal(num[:, :t0 + 1], n2[:, :t0 + 1])
    assert np.array_equal(den[:, :t0 + 1], d2[:, :t0 + 1])


@pytest.mark.parametrize("gamma", [None, 0.93])
def test_combine_associative_identity_and_halves(gamma):
    q, k, v = rnd(2, 15, 3, 2, seed=57)
    a, b, c = (O.ahla_segment_summary(q[:, s:e], k[:, s:e], v[:, s:e], gamma)
               for s, e in ((0, 4), (4, 11), (11, 15)))
    left = O.combine_ahla(O.combine_ahla(a, b, gamma), c, gamma)
    right = O.combine_ahla(a, O.combine_ahla(b, c, gamma), gamma)
    whole = O.ahla_segment_summary(q, k, v, gamma)
    for x in ("P", "m", "E", "n", "X"):
        assert rel(left[x], right[x]) < 1e-12, x
        assert rel(left[x], whole[x]) < 1e-12, x
    e = O.ahla_identity(2, 3, 2)
    for x in ("P", "m", "E", "n", "X"):
        assert rel(O.combine_ahla(e, a, gamma)[x], a[x]) < 1e-15
        assert rel(O.combine_ahla(a, e, gamma)[x], a[x]) < 1e-15


@pytest.mark.parametrize("gamma", [None, 0.93])
@pytest.mark.parametrize("chunk", [1, 3, 4, 8, 24])
def test_chunk_form_reproduces_serial(gamma, chunk):
    q, k, v = rnd(2, 24, 3, 2, seed=58)
    num, den, _ = O.serial_ahla(q, k, v, gamma)
    cn, cd, _ = O.ahla_chunk_forward(q, k, v, chunk, gamma)
    assert rel(cn, num) < 1e-12
    assert rel(cd, den) < 1e-12


def _mutant(func, old, new):
    src = inspect.getsource(func)
    assert old in src, old
    ns = dict(vars(O))
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    return ns[func.__name__]


SERIAL_MUTANTS = [
    # r read from P before token t is added (j < i instead of j <= i)
    ("r = np.matmul(qt[:, None, :], P)[:, 0, :]",
     "r = np.matmul(qt[:, None, :], P - kt[:, :, None] * vt[:, None, :])[:, 0, :]"),
    # E not decayed
    ("E = g1[:, :, None] * E + kt", "E = E + kt"),
    # denominator from q.m instead of q.n
    ("den[:, t] = np.sum(qt * n, axis=1)", "den[:, t] = np.sum(qt * m, axis=1)"),
]


@pytest.mark.parametrize("old,new", SERIAL_MUTANTS)
def test_pins_catch_planted_mistakes_in_serial(old, new):
    bad = _mutant(O.serial_ahla, old, new)
    q, k, v = rnd(2, 10, 3, 2, seed=59)
    caught = False
    for gamma in (None, 0.8):
        n_bad, d_bad, _ = bad(q, k, v, gamma)
        bn, bd = O.brute_ahla(q, k, v, gamma)
        if rel(n_bad, bn) > 1e-9 or rel(d_bad, bd) > 1e-9:
            caught = True
    assert caught


COMBINE_MUTANTS = [
    ('a3 * np.matmul(B["X"], A["P"])', 'np.matmul(B["X"], A["P"])'),        # cross term not decayed
    ('a3 * np.matmul(B["X"], A["P"])', 'a3 * np.matmul(A["X"], A["P"])'),   # X of the wrong side
    ('"m": a1 * A["m"] + B["m"]', '"m": A["m"] + B["m"]'),                  # m not decayed
]


@pytest.mark.parametrize("old,new", COMBINE_MUTANTS)
def test_pins_catch_planted_mistakes_in_combine(old, new):
    bad = _mutant(O.combine_ahla, old, new)
    q, k, v = rnd(2, 12, 3, 2, seed=60)
    A = O.ahla_segment_summary(q[:, :5], k[:, :5], v[:, :5], 0.8)
    B = O.ahla_segment_summary(q[:, 5:], k[:, 5:], v[:, 5:], 0.8)
    whole = O.ahla_segment_summary(q, k, v, 0.8)
    got = bad(A, B, 0.8)
    assert any(rel(got[x], whole[x]) > 1e-9 for x in ("P", "m", "E", "n"))
