"""Pins of the third-order HLA oracle against things other than itself:
the hand-worked example in tests/golden/, the closed form written out as a
quadruple sum, each cross summary against its class of terms summed one by
one, library matmuls of the masked matrices, special cases with a closed form
(gamma = 0, d = 1), causality, the algebra of the segment combine
(associativity, identity, parts = whole), the exactness of the chunk-parallel
scan, and planted mistakes that the pins must catch."""

import inspect
import json
import os

import numpy as np
import pytest

from oracle import hla3_oracle as O3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(U, T, d, dv, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((U, T, d)), rng.standard_normal((U, T, d)),
            rng.standard_normal((U, T, dv)))


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


GAMMAS = [None, 0.9, np.array([0.7, 0.95, 1.0])]


def test_hand_example_exact():
    with open(os.path.join(GOLDEN, "hand_example_hla3_d1.json")) as f:
        ex = json.load(f)
    q, k, v = (np.array(ex[x]).reshape(1, -1, 1) for x in ("q", "k", "v"))
    for case in ex["cases"]:
        g = case["gamma"]
        wn, wd = np.array(case["num"]), np.array(case["den"])
        for form in (O3.serial3, lambda *a: O3.serial3_r(*a)[:2], O3.brute3, O3.matrix_form3):
            n, dn = form(q, k, v, g)[:2]
            assert np.allclose(n[0, :, 0], wn, rtol=0, atol=1e-12), (g, n)
            assert np.allclose(dn[0], wd, rtol=0, atol=1e-12), (g, dn)
        n, dn, _ = O3.serial3_r(q, k, v, g)
        assert np.array_equal(n[0, :, 0], wn) and np.array_equal(dn[0], wd)   # dyadic: exact


@pytest.mark.parametrize("gamma", GAMMAS)
def test_forms_match_brute_quadruple_sum(gamma):
    q, k, v = rnd(3, 9, 3, 2, seed=1)
    bn, bd = O3.brute3(q, k, v, gamma)
    for n, dn in (O3.serial3(q, k, v, gamma), O3.serial3_r(q, k, v, gamma)[:2],
                  O3.matrix_form3(q, k, v, gamma)):
        assert rel(n, bn) < 1e-12 and rel(dn, bd) < 1e-12


@pytest.mark.parametrize("gamma", [None, 0.85])
def test_cross_summaries_are_the_forbidden_classes(gamma):
    """num = q^T (F - G1 - G2 - G3) with each G its class of terms; checked
    on the products q_t^T X_t that the output sees, class by class."""
    q, k, v = rnd(2, 7, 3, 2, seed=2)
    F, G1, G2, G3 = O3.brute3_classes(q, k, v, gamma)
    bn, _ = O3.brute3(q, k, v, gamma)
    proj = lambda X: np.einsum("utd,utde->ute", q, X)
    assert rel(proj(F - G1 - G2 - G3), bn) < 1e-12
    # the serial form's running cross summaries, class by class: rebuild them
    # with planted zeros in the other two and compare the outputs
    src = inspect.getsource(O3.serial3)
    ns = dict(vars(O3))
    for keep, G in ((1, G1), (2, G2), (3, G3)):
        mod = src.replace("num[:, t] = _vm(SqQ, P) - _vm(qt, G1 + G2 + G3)",
                          f"num[:, t] = _vm(qt, G{keep})")
        exec(compile(mod, "<class>", "exec"), ns)
        n, _ = ns["serial3"](q, k, v, gamma)
        assert rel(n, proj(G)) < 1e-11, keep


def test_gamma_zero_keeps_only_the_diagonal():
    q, k, v = rnd(2, 10, 4, 3, seed=3)
    s = np.sum(q * k, axis=-1)
    for form in (O3.serial3, lambda *a: O3.serial3_r(*a)[:2], O3.matrix_form3):
        n, dn = form(q, k, v, 0.0)[:2]
        assert rel(n, (s ** 3)[..., None] * v) < 1e-12 and rel(dn, s ** 3) < 1e-12


def test_d1_closed_form():
    q, k, v = rnd(2, 30, 1, 3, seed=4)
    n, dn, _ = O3.serial3_r(q, k, v)
    K = np.cumsum(k[..., 0] ** 2, axis=1)
    Uv = np.cumsum(k * v, axis=1)
    M = np.cumsum(k[..., 0], axis=1)
    qq = q[..., 0]
    want = qq[..., None] * np.cumsum((qq ** 2 * K)[..., None] * Uv, axis=1)
    assert rel(n, want) < 1e-12
    assert rel(dn, qq * np.cumsum(qq ** 2 * K * M, axis=1)) < 1e-12
    n2, d2 = O3.serial3(q, k, v)
    assert rel(n2, want) < 1e-11


@pytest.mark.parametrize("gamma", [None, 0.9])
def test_causality(gamma):
    q, k, v = rnd(2, 30, 3, 2, seed=5)
    n, d, _ = O3.serial3_r(q, k, v, gamma)
    t0 = 13
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, t0 + 1:] *= -2.0
    k2[:, t0 + 1:] += 1.0
    v2[:, t0 + 1:] = 5.0
    n2, d2, _ = O3.serial3_r(q2, k2, v2, gamma)
    assert np.array_equal(n[:, :t0 + 1], n2[:, :t0 + 1]) and np.array_equal(d[:, :t0 + 1], d2[:, :t0 + 1])
    assert not np.allclose(n[:, t0 + 1:], n2[:, t0 + 1:])


def test_den_is_num_with_unit_values_and_scaling():
    q, k, _ = rnd(2, 20, 4, 1, seed=6)
    n, d, _ = O3.serial3_r(q, k, np.ones((2, 20, 1)), 0.9)
    assert rel(n[..., 0], d) < 1e-13
    # q appears three times, k three times in every term
    _, v = None, rnd(2, 20, 4, 2, seed=7)[2]
    n1, d1, _ = O3.serial3_r(q, k, v, 0.9)
    na, da, _ = O3.serial3_r(1.3 * q, 0.7 * k, v, 0.9)
    assert rel(na, (1.3 * 0.7) ** 3 * n1) < 1e-12 and rel(da, (1.3 * 0.7) ** 3 * d1) < 1e-12


SUMMARY_KEYS = ("S", "Q", "P", "m", "V", "Z", "z", "R", "r", "a")


@pytest.mark.parametrize("gamma", GAMMAS)
def test_combine_associative_identity_and_parts_equal_whole(gamma):
    q, k, v = rnd(3, 14, 3, 2, seed=8)
    A = O3.segment_summary3(q[:, :4], k[:, :4], v[:, :4], gamma)
    B = O3.segment_summary3(q[:, 4:9], k[:, 4:9], v[:, 4:9], gamma)
    C = O3.segment_summary3(q[:, 9:], k[:, 9:], v[:, 9:], gamma)
    whole = O3.segment_summary3(q, k, v, gamma)
    left = O3.combine3(O3.combine3(A, B), C)
    right = O3.combine3(A, O3.combine3(B, C))
    I = O3.identity3(3, 3, 2)
    for x in SUMMARY_KEYS:
        assert rel(left[x], right[x]) < 1e-13, x
        assert rel(left[x], whole[x]) < 1e-12, x
        assert rel(O3.combine3(I, A)[x], A[x]) < 1e-15 and rel(O3.combine3(A, I)[x], A[x]) < 1e-15


@pytest.mark.parametrize("gamma", [None, 0.93])
@pytest.mark.parametrize("chunk", [1, 3, 4, 8, 24])
def test_exclusive_scan_reproduces_serial(gamma, chunk):
    q, k, v = rnd(2, 24, 3, 2, seed=9)
    n, d, st = O3.serial3_r(q, k, v, gamma)
    cn, cd, tot = O3.chunk_forward3(q, k, v, chunk, gamma)
    assert rel(cn, n) < 1e-11 and rel(cd, d) < 1e-11
    for x in ("S", "P", "m", "R", "r"):
        assert rel(tot[x], st[x]) < 1e-11, x


def test_decode_continues_the_recurrence():
    q, k, v = rnd(2, 20, 3, 2, seed=10)
    n, d, _ = O3.serial3_r(q, k, v, 0.9)
    _, _, st = O3.serial3_r(q[:, :15], k[:, :15], v[:, :15], 0.9)
    for t in range(15, 20):
        nt, dt, st = O3.decode_step3(st, q[:, t], k[:, t], v[:, t], 0.9)
        assert rel(nt, n[:, t]) < 1e-12 and rel(dt, d[:, t]) < 1e-12


def _mutant(func, old, new):
    src = inspect.getsource(func)
    assert old in src, old
    ns = dict(vars(O3))
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), ns)
    return ns[func.__name__]


SERIAL3_MUTANTS = [
    ("g2[:, :, None] * _outer(kt, kZ)", "g2[:, :, None] * _outer(kt, _vm(kt, P))"),   # G1 from P, not Z
    ("G2 = g3[:, :, None] * G2", "G2 = g2[:, :, None] * G2"),                          # decay power
    ("+ (g1 * kQk[:, None])[:, :, None] * _outer(kt, vt))", ")"),                      # drops the i = l term
    ("- _vm(qt, G1 + G2 + G3)", "- _vm(qt, G1 + G2)"),                                  # one class missing
    ("V = g2[:, :, None] * V + _outer(Sq, qt)", "V = g2[:, :, None] * V + _outer(qt, Sq)"),  # V transposed
]


@pytest.mark.parametrize("old,new", SERIAL3_MUTANTS)
def test_pins_catch_planted_mistakes_in_serial3(old, new):
    """Either the output or one of the cross summaries (projected on q_t, as
    in test_cross_summaries_are_the_forbidden_classes) departs from its brute
    sum.  (V enters G2 and G3 with opposite signs, so a mistake in V shows
    in the classes but cancels in the output.)"""
    src = inspect.getsource(O3.serial3)
    assert old in src
    bad_src = src.replace(old, new, 1)
    q, k, v = rnd(2, 8, 3, 2, seed=11)
    proj = lambda X: np.einsum("utd,utde->ute", q, X)
    caught = False
    for gamma in (None, 0.8):
        ns = dict(vars(O3))
        exec(compile(bad_src, "<mutant>", "exec"), ns)
        n, d = ns["serial3"](q, k, v, gamma)
        bn, bd = O3.brute3(q, k, v, gamma)
        caught |= rel(n, bn) > 1e-9 or rel(d, bd) > 1e-9
        _, G1, G2, G3 = O3.brute3_classes(q, k, v, gamma)
        for keep, G in ((1, G1), (2, G2), (3, G3)):
            ns = dict(vars(O3))
            exec(compile(bad_src.replace("num[:, t] = _vm(SqQ, P) - _vm(qt, G1 + G2 + G3)",
                                         f"num[:, t] = _vm(qt, G{keep})"), "<mutant>", "exec"), ns)
            caught |= rel(ns["serial3"](q, k, v, gamma)[0], proj(G)) > 1e-9
    assert caught


COMBINE3_MUTANTS = [
    ("A1 * np.matmul(A[\"S\"], B[\"Z\"])", "A1 * np.matmul(B[\"S\"], A[\"Z\"])"),   # sides swapped
    ("MKQ = A2 * SAQB + A1 * B[\"V\"]", "MKQ = A1 * SAQB + A1 * B[\"V\"]"),              # map decay
    ("A1 * np.matmul(B[\"Q\"], A[\"P\"])", "A1 * np.matmul(A[\"Q\"], B[\"P\"])"),          # Z cross order
    ("\"R\": A3 * A[\"R\"]", "\"R\": A2 * A[\"R\"]"),                                       # R decay
]


@pytest.mark.parametrize("old,new", COMBINE3_MUTANTS)
def test_pins_catch_planted_mistakes_in_combine3(old, new):
    bad = _mutant(O3.combine3, old, new)
    q, k, v = rnd(2, 11, 3, 2, seed=12)
    caught = False
    for gamma in (None, 0.8):
        A = O3.segment_summary3(q[:, :5], k[:, :5], v[:, :5], gamma)
        B = O3.segment_summary3(q[:, 5:], k[:, 5:], v[:, 5:], gamma)
        whole = O3.segment_summary3(q, k, v, gamma)
        got = bad(A, B)
        caught |= any(rel(got[x], whole[x]) > 1e-9 for x in SUMMARY_KEYS)
    assert caught
