"""Pins of the oracle's unmasked second-order variant (o_t = q_t^T S_t C_t).

The unmasked recurrence is fixed against its closed form written out as a
triple sum, against the prefix sums written out with library products,
against library matmuls of the masked-matrix form, against special cases
with a closed form (gamma = 0, d = 1), against causality and against the
exactness of its chunk-parallel scan; planted mistakes must be caught.
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
    q, k, v = rnd(3, 16, 4, 3, seed=31)
    num, den, _ = O.serial_unmasked(q, k, v, gamma)
    bn, bd = O.brute_unmasked(q, k, v, gamma)
    assert rel(num, bn) < 1e-12
    assert rel(den, bd) < 1e-12


@pytest.mark.parametrize("gamma", [None, 0.9])
def test_serial_matches_prefix_sums_written_out(gamma):
    # S_t = sum_{i<=t} g^(t-i) k_i k_i^T, C_t likewise, m_t likewise, each
    # built for every t at once with einsum; num_t = q_t^T S_t C_t.
    q, k, v = rnd(2, 30, 5, 3, seed=32)
    U, T, _ = q.shape
    g = 1.0 if gamma is None else gamma
    t = np.arange(T)
    W = np.where(t[:, None] >= t[None, :], g ** np.maximum(t[:, None] - t[None, :], 0), 0.0)
    S = np.einsum("ti,uia,uib->utab", W, k, k)
    C = np.einsum("tj,uja,ujb->utab", W, q, v)
    m = np.einsum("tj,uja->uta", W, q)
    want = np.einsum("uta,utab,utbc->utc", q, S, C)
    want_den = np.einsum("uta,utab,utb->ut", q, S, m)
    num, den, _ = O.serial_unmasked(q, k, v, gamma)
    assert rel(num, want) < 1e-12
    assert rel(den, want_den) < 1e-12


@pytest.mark.parametrize("gamma", [None, 0.85])
def test_serial_matches_matrix_form(gamma):
    # P = (L o Q K^T) K  (row t: S_t q_t), num = (L o P Q^T) V, den = (L o P Q^T) 1,
    # L[t, i] = g^(t-i) for i <= t: two masked first-order products.
    q, k, v = rnd(2, 64, 6, 4, seed=33)
    T = q.shape[1]
    g = 1.0 if gamma is None else gamma
    t = np.arange(T)
    L = np.where(t[:, None] >= t[None, :], g ** np.maximum(t[:, None] - t[None, :], 0), 0.0)
    num, den, _ = O.serial_unmasked(q, k, v, gamma)
    for u in range(q.shape[0]):
        P = (L * (q[u] @ k[u].T)) @ k[u]
        Wm = L * (P @ q[u].T)
        assert rel(num[u], Wm @ v[u]) < 1e-12
        assert rel(den[u], Wm.sum(axis=1)) < 1e-12


def test_gamma_zero_keeps_only_the_current_token():
    q, k, v = rnd(2, 12, 4, 3, seed=34)
    num, den, _ = O.serial_unmasked(q, k, v, 0.0)
    qk = np.sum(q * k, axis=2)
    assert rel(num, qk[..., None] ** 2 * v) < 1e-12
    assert rel(den, qk ** 2) < 1e-12          # (q_t^T k_t k_t^T) q_t


@pytest.mark.parametrize("gamma", [None, 0.9])
def test_d1_product_of_two_running_sums(gamma):
    # d = 1: o_t = q_t (sum_{i<=t} g^(t-i) k_i^2) (sum_{j<=t} g^(t-j) q_j v_j)
    q, k, v = rnd(2, 40, 1, 3, seed=35)
    g = 1.0 if gamma is None else gamma
    T = q.shape[1]
    Ks = np.zeros((2, T))
    Cs = np.zeros((2, T, 3))
    Ms = np.zeros((2, T))
    ak, ac, am = np.zeros(2), np.zeros((2, 3)), np.zeros(2)
    for t in range(T):
        ak = g * ak + k[:, t, 0] ** 2
        ac = g * ac + q[:, t, 0:1] * v[:, t]
        am = g * am + q[:, t, 0]
        Ks[:, t], Cs[:, t], Ms[:, t] = ak, ac, am
    num, den, _ = O.serial_unmasked(q, k, v, gamma)
    assert rel(num, q[..., 0:1] * Ks[..., None] * Cs) < 1e-12
    assert rel(den, q[..., 0] * Ks * Ms) < 1e-12


def test_differs_from_the_masked_operator_by_the_future_terms():
    # unmasked - masked = sum over key index i after value index j (j < i <= t)
    q, k, v = rnd(1, 9, 3, 2, seed=36)
    nu, _, _ = O.serial_unmasked(q, k, v)
    nm, _, _ = O.serial(q, k, v)
    want = np.zeros_like(nu)
    for t in range(9):
        for j in range(t + 1):
            for i in range(j + 1, t + 1):
                want[0, t] += (q[0, t] @ k[0, i]) * (k[0, i] @ q[0, j]) * v[0, j]
    assert rel(nu - nm, want) < 1e-12
    assert np.max(np.abs(want)) > 1e-3


@pytest.mark.parametrize("gamma", [None, 0.9])
def test_causality(gamma):
    q, k, v = rnd(2, 30, 4, 3, seed=37)
    num, den, _ = O.serial_unmasked(q, k, v, gamma)
    t0 = 11
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, t0 + 1:] *= -2.0
    k2[:, t0 + 1:] += 1.0
    v2[:, t0 + 1:] = 5.0
    n2, d2, _ = O.serial_unmasked(q2, k2, v2, gamma)
    assert np.array_equal(num[:, :t0 + 1], n2[:, :t0 + 1])
    assert np.array_equal(den[:, :t0 + 1], d2[:, :t0 + 1])


@pytest.mark.parametrize("gamma", [None, 0.93])
def test_combine_associative_with_identity(gamma):
    q, k, v = rnd(2, 15, 3, 2, seed=38)
    parts = []
    for s, e in ((0, 4), (4, 11), (11, 15)):
        _, _, st = O.serial_unmasked(q[:, s:e], k[:, s:e], v[:, s:e], gamma)
        st["G"], st["h"] = np.zeros((2, 3, 2)), np.zeros((2, 3))
        st["L"] = np.full(2, e - s, dtype=np.int64)
        parts.append(st)
    a, b, c = parts
    left = O.combine_unmasked(O.combine_unmasked(a, b, gamma), c, gamma)
    right = O.combine_unmasked(a, O.combine_unmasked(b, c, gamma), gamma)
    _, _, whole = O.serial_unmasked(q, k, v, gamma)
    for x in "SCm":
        assert rel(left[x], right[x]) < 1e-12
        assert rel(left[x], whole[x]) < 1e-12
    e = O.identity_summary(2, 3, 2)
    for x in "SCm":
        assert rel(O.combine_unmasked(e, a, gamma)[x], a[x]) < 1e-15
        assert rel(O.combine_unmasked(a, e, gamma)[x], a[x]) < 1e-15


@pytest.mark.parametrize("gamma", [None, 0.93])
@pytest.mark.parametrize("chunk", [1, 3, 4, 8, 24])
def test_exclusive_scan_reproduces_serial(gamma, chunk):
    q, k, v = rnd(2, 24, 3, 2, seed=39)
    num, den, _ = O.serial_unmasked(q, k, v, gamma)
    cn, cd, _ = O.unmasked_chunk_forward(q, k, v, chunk, gamma)
    assert rel(cn, num) < 1e-12
    assert rel(cd, den) < 1e-12


def _mutant(func, old, new):
    src = inspect.getsource(func)
    assert old in src, old
    ns = dict(vars(O))
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    return ns[func.__name__]


SERIAL_MUTANTS = [
    # decay dropped from C
    ("C = g1[:, :, None] * C + qt", "C = C + qt"),
    # output read before this token's k k^T is in S
    ("qS = np.matmul(qt[:, None, :], S)[:, 0, :]",
     "qS = np.matmul(qt[:, None, :], S - kt[:, :, None] * kt[:, None, :])[:, 0, :]"),
    # denominator from q.m instead of (q^T S) m
    ("den[:, t] = np.sum(qS * m, axis=1)", "den[:, t] = np.sum(qt * m, axis=1)"),
]


@pytest.mark.parametrize("old,new", SERIAL_MUTANTS)
def test_pins_catch_planted_mistakes_in_serial(old, new):
    bad = _mutant(O.serial_unmasked, old, new)
    q, k, v = rnd(2, 10, 3, 2, seed=40)
    caught = False
    for gamma in (None, 0.8):
        n_bad, d_bad, _ = bad(q, k, v, gamma)
        bn, bd = O.brute_unmasked(q, k, v, gamma)
        if rel(n_bad, bn) > 1e-9 or rel(d_bad, bd) > 1e-9:
            caught = True
    assert caught


COMBINE_MUTANTS = [
    ("\"m\": a[:, None] * A[\"m\"] + B[\"m\"]", "\"m\": A[\"m\"] + B[\"m\"]"),          # m not decayed
    ("\"S\": a[:, None, None] * A[\"S\"] + B[\"S\"]",
     "\"S\": A[\"S\"] + a[:, None, None] * B[\"S\"]"),                                  # decay on B
]


@pytest.mark.parametrize("old,new", COMBINE_MUTANTS)
def test_pins_catch_planted_mistakes_in_combine(old, new):
    bad = _mutant(O.combine_unmasked, old, new)
    q, k, v = rnd(2, 12, 3, 2, seed=41)
    _, _, A = O.serial_unmasked(q[:, :5], k[:, :5], v[:, :5], 0.8)
    _, _, B = O.serial_unmasked(q[:, 5:], k[:, 5:], v[:, 5:], 0.8)
    _, _, whole = O.serial_unmasked(q, k, v, 0.8)
    for st, L in ((A, 5), (B, 7)):
        st["G"], st["h"] = np.zeros((2, 3, 2)), np.zeros((2, 3))
        st["L"] = np.full(2, L, dtype=np.int64)
    got = bad(A, B, 0.8)
    assert any(rel(got[x], whole[x]) > 1e-9 for x in "SCm")
