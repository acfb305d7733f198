"""Pins of the backward oracle (gradients of the masked second-order forward).

Both backward forms (float64 autograd through the masked matrix form, and the
serial forward/reverse state recurrences) are fixed against central finite
differences of the oracle's serial forward recurrence (a third, independent
code path), against the gamma = 0 closed form, and against causality: the
gradient at token s depends only on upstream gradients at tokens t >= s.
"""

import numpy as np
import pytest

from oracle import hla_oracle as O
from oracle import hla_backward_oracle as BO


def rnd(U, T, d, dv, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((U, T, d)), rng.standard_normal((U, T, d)),
            rng.standard_normal((U, T, dv)), rng.standard_normal((U, T, dv)))


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def loss(q, k, v, do, gamma, normalize, eps):
    num, den, _ = O.serial(q, k, v, gamma)
    o = num / (den + eps)[..., None] if normalize else num
    return float(np.sum(o * do))


GAMMAS = [None, 0.9, np.array([0.75, 1.0])]


@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("gamma", GAMMAS)
def test_autograd_matches_finite_differences_of_serial(gamma, normalize):
    q, k, v, do = rnd(2, 7, 3, 2, seed=71)
    eps = 1e-6
    if normalize:
        # keep the denominator away from zero so the quotient is smooth
        k = np.abs(k)
        q = np.abs(q)
        _, den, _ = O.serial(q, k, v, gamma)
        assert np.min(np.abs(den + eps)) > 1e-2
    grads = BO.grad_autograd(q, k, v, do, gamma, normalize, eps)
    rng = np.random.default_rng(5)
    h = 1e-5
    for which in range(3):
        dirs = [np.zeros_like(x) for x in (q, k, v)]
        dirs[which] = rng.standard_normal(dirs[which].shape)
        plus = [x + h * e for x, e in zip((q, k, v), dirs)]
        minus = [x - h * e for x, e in zip((q, k, v), dirs)]
        fd = (loss(*plus, do, gamma, normalize, eps) - loss(*minus, do, gamma, normalize, eps)) / (2 * h)
        an = float(np.sum(grads[which] * dirs[which]))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("gamma", GAMMAS)
def test_states_match_finite_differences_of_serial(gamma):
    q, k, v, do = rnd(2, 6, 3, 4, seed=72)
    grads = BO.grad_states(q, k, v, do, gamma)
    rng = np.random.default_rng(6)
    h = 1e-5
    for which in range(3):
        dirs = [np.zeros_like(x) for x in (q, k, v)]
        dirs[which] = rng.standard_normal(dirs[which].shape)
        plus = [x + h * e for x, e in zip((q, k, v), dirs)]
        minus = [x - h * e for x, e in zip((q, k, v), dirs)]
        fd = (loss(*plus, do, gamma, False, 0.0) - loss(*minus, do, gamma, False, 0.0)) / (2 * h)
        an = float(np.sum(grads[which] * dirs[which]))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("shape", [(3, 20, 4, 3), (2, 33, 8, 8), (1, 5, 1, 1)])
@pytest.mark.parametrize("gamma", GAMMAS)
def test_states_match_autograd(shape, gamma):
    U = shape[0]
    g = gamma if not isinstance(gamma, np.ndarray) else np.resize(gamma, U)
    q, k, v, do = rnd(*shape, seed=73)
    a = BO.grad_autograd(q, k, v, do, g)
    s = BO.grad_states(q, k, v, do, g)
    for x, y in zip(s, a):
        assert rel(x, y) < 1e-11


def test_gamma_zero_closed_form():
    # gamma = 0 keeps only i = j = t: o_t = (q_t.k_t)^2 v_t
    q, k, v, do = rnd(2, 9, 4, 3, seed=74)
    qk = np.sum(q * k, axis=2)
    dov = np.sum(do * v, axis=2)
    want_dv = (qk ** 2)[..., None] * do
    want_dq = (2 * qk * dov)[..., None] * k
    want_dk = (2 * qk * dov)[..., None] * q
    for got in (BO.grad_autograd(q, k, v, do, 0.0), BO.grad_states(q, k, v, do, 0.0)):
        assert rel(got[0], want_dq) < 1e-12
        assert rel(got[1], want_dk) < 1e-12
        assert rel(got[2], want_dv) < 1e-12


@pytest.mark.parametrize("gamma", [None, 0.9])
def test_gradient_is_causal(gamma):
    q, k, v, do = rnd(2, 12, 3, 2, seed=75)
    s0 = 7
    do[:, s0:] = 0.0
    for got in (BO.grad_autograd(q, k, v, do, gamma), BO.grad_states(q, k, v, do, gamma)):
        for x in got:
            assert np.all(x[:, s0:] == 0.0)
            assert np.max(np.abs(x[:, :s0])) > 0.0


def test_single_token_closed_form():
    # T = 1: o = (q.k)^2 v for any gamma
    q, k, v, do = rnd(3, 1, 5, 2, seed=76)
    qk = np.sum(q * k, axis=2)
    dov = np.sum(do * v, axis=2)
    got = BO.grad_states(q, k, v, do, 0.6)
    assert rel(got[2], (qk ** 2)[..., None] * do) < 1e-12
    assert rel(got[0], (2 * qk * dov)[..., None] * k) < 1e-12
    assert rel(got[1], (2 * qk * dov)[..., None] * q) < 1e-12
