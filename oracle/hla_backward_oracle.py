"""CPU oracle for the backward pass of the masked second-order HLA forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests use it.  It shares no code with the HIP
path.

Sources: the method section on parallel training by associative scans
("Higher-order Linear Attention", gist.science summaries) motivates a
backward pass but gives no formula for it.  The backward is therefore the
plain gradient of the forward's closed form,

    num_t = sum_{j<=t} sum_{i<=j} g^((t-i)+(t-j)) (q_t.k_i)(q_j.k_i) v_j,

(the masked A A^T V structure of the method section on second-order HLA,
with the decay reading gamma^((t-i)+(t-j)) of the forward oracle), taken with
respect to q, k and v for an upstream gradient dO = dL/d num.  gamma is not
differentiated.

Two independent forms live here:

  * `grad_autograd`: float64 PyTorch autograd through the masked matrix form
    (W = L o ((A o L)(A o 1)^T), num = W V).  This is the definition, and the
    parity target of the GPU backward.
  * `grad_states`: the same gradient from serial recurrences over the tokens,
    forward then reverse.  With p_t = S_t q_t (S_t the decayed sum of
    k_i k_i^T), the forward is o_t = sum_{j<=t} g^(2(t-j)) (q_t.p_j) v_j, a
    linear attention over keys p_j, and the chain rule gives
        dp_j = sum_{t>=j} g^(2(t-j)) (v_j.dO_t) q_t
        dv_j = sum_{t>=j} g^(2(t-j)) (p_j.q_t) dO_t
        dq_t = sum_{j<=t} g^(2(t-j)) (dO_t.v_j) p_j + S_t dp_t
        dk_i = sum_{t>=i} g^(t-i) [(k_i.q_t) dp_t + (k_i.dp_t) q_t].
    Each sum is a decayed running state (forward for dq, reverse for the
    others), walked one token at a time.  The HIP backward computes exactly
    these seven first-order sums.

The tests pin both against central finite differences of the serial forward
recurrence (`hla_oracle.serial`), the gamma = 0 closed form and causality.
"""

import numpy as np
import torch

__all__ = ["grad_autograd", "grad_states"]

_F = np.float64


def _gamma(gamma, U):
    if gamma is None:
        return np.ones(U, dtype=_F)
    g = np.asarray(gamma, dtype=_F).reshape(-1)
    if g.size == 1:
        g = np.full(U, g[0], dtype=_F)
    assert g.shape == (U,)
    return g


def _forward_torch(q, k, v, g, normalize, eps):
    """Masked matrix form of the forward in float64 torch ops, per unit."""
    U, T, _ = q.shape
    idx = torch.arange(T, dtype=torch.float64)
    diff = idx[:, None] - idx[None, :]
    lower = (diff >= 0).to(torch.float64)
    outs = []
    for u in range(U):
        gu = float(g[u])
        if gu == 0.0:
            L = torch.eye(T, dtype=torch.float64)
        else:
            L = lower * torch.pow(torch.tensor(gu, dtype=torch.float64), diff.clamp(min=0))
        A = q[u] @ k[u].T
        W = L * ((A * L) @ (A * lower).T)
        num = W @ v[u]
        if normalize:
            den = W.sum(dim=1)
            num = num / (den + eps)[:, None]
        outs.append(num)
    return torch.stack(outs)


def grad_autograd(q, k, v, dout, gamma=None, normalize=False, eps=1e-6):
    """dL/dq, dL/dk, dL/dv for L = sum_t dout_t . o_t, by float64 autograd.

    o is the unnormalised numerator, or num / (den + eps) when `normalize`.
    q, k: [U, T, d]; v, dout: [U, T, dv]; gamma: [U] or None (gamma = 1).
    Returns three float64 NumPy arrays shaped like q, k, v.
    """
    q = torch.tensor(np.asarray(q, dtype=_F), requires_grad=True)
    k = torch.tensor(np.asarray(k, dtype=_F), requires_grad=True)
    v = torch.tensor(np.asarray(v, dtype=_F), requires_grad=True)
    g = _gamma(gamma, q.shape[0])
    o = _forward_torch(q, k, v, g, normalize, eps)
    (o * torch.tensor(np.asarray(dout, dtype=_F))).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def grad_states(q, k, v, dout, gamma=None):
    """The unnormalised gradient from serial forward and reverse states.

    Forward walk (t = 1..T): S <- g S + k_t k_t^T, p_t = S q_t,
    M <- g^2 M + p_t v_t^T, dq_t = M dO_t (the first dq term; M dO_t equals
    sum_{j<=t} g^(2(t-j)) (dO_t.v_j) p_j).
    Reverse walk (t = T..1): U <- g^2 U + q_t dO_t^T, dp_t = U v_t,
    dv_t = U^T p_t; R <- g R + dp_t q_t^T + q_t dp_t^T, dk_t = R k_t.
    A second forward walk adds S_t dp_t to dq_t.
    """
    q, k, v, do = (np.asarray(x, dtype=_F) for x in (q, k, v, dout))
    U, T, d = q.shape
    dv_ = v.shape[2]
    g = _gamma(gamma, U)
    g1 = g[:, None, None]
    g2 = (g * g)[:, None, None]
    S = np.zeros((U, d, d))
    M = np.zeros((U, d, dv_))
    p = np.empty((U, T, d))
    dq = np.empty((U, T, d))
    for t in range(T):
        S = g1 * S + k[:, t, :, None] * k[:, t, None, :]
        p[:, t] = np.einsum("uab,ub->ua", S, q[:, t])
        M = g2 * M + p[:, t, :, None] * v[:, t, None, :]
        dq[:, t] = np.einsum("uae,ue->ua", M, do[:, t])
    Ur = np.zeros((U, d, dv_))
    R = np.zeros((U, d, d))
    dp = np.empty((U, T, d))
    dk = np.empty((U, T, d))
    dv = np.empty((U, T, dv_))
    for t in range(T - 1, -1, -1):
        Ur = g2 * Ur + q[:, t, :, None] * do[:, t, None, :]
        dp[:, t] = np.einsum("uae,ue->ua", Ur, v[:, t])
        dv[:, t] = np.einsum("uae,ua->ue", Ur, p[:, t])
        R = (g1 * R + dp[:, t, :, None] * q[:, t, None, :]
             + q[:, t, :, None] * dp[:, t, None, :])
        dk[:, t] = np.einsum("uab,ub->ua", R, k[:, t])
    S = np.zeros((U, d, d))
    for t in range(T):
        S = g1 * S + k[:, t, :, None] * k[:, t, None, :]
        dq[:, t] += np.einsum("uab,ub->ua", S, dp[:, t])
    return dq, dk, dv

