"""CPU oracle for the masked second-order HLA forward, its decode step, the
unmasked variant and the asymmetric variant AHLA.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP path.

Everything is plain NumPy in float64.  Inputs are upcast exactly from the
values the GPU receives (bf16 or fp32); arrays are batched over independent
units u = (batch, head): q, k are [U, T, d], v is [U, T, dv], gamma is [U].

Sources (the pages are two summaries of one paper, "Higher-order Linear
Attention", arXiv 2510.27258, on gist.science, in Japanese and French):

  [S1]  method section 1, second-order HLA: the prefix moments
        S^K_t = sum_{i<=t} k_i k_i^T, C^QV_t = sum_{i<=t} q_i v_i^T,
        m^Q_t = sum_{i<=t} q_i; the cross summaries G_t, h_t that remove the
        future terms from S^K_t C^QV_t; the output
        o_t = q_t^T (S^K_t C^QV_t - G_t); a ratio-normalised variant whose
        denominator is a masked term built from the same kind of summaries.
  [S4]  method section 4, parallel training by associative scans: an
        associative (semidirect-product) operator joins token segments and
        carries the cross term S^K_B C^QV_A; an exclusive Blelloch scan of
        segment summaries gives exactly the serial forward activations.
  [C2]  key contributions, item 2: the operators also exist with
        exponential decay.
  [R]   results and claims: O(d^2 + d dv) per token, exact equality of the
        chunk-parallel scheme with the serial recurrence, and causality
        (o_t depends only on tokens j <= t).

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * The G/h updates: G_t = G_{t-1} + k_t k_t^T C_{t-1},
    h_t = h_{t-1} + k_t k_t^T m_{t-1} (C and m BEFORE token t is added), and
    the combine G_AB = G_A + G_B + S_B C_A, h_AB = h_A + h_B + S_B m_A.
    Together they give the closed form
    o_t = sum_{j<=t} sum_{i<=j} (q_t.k_i)(q_j.k_i) v_j, which `brute` writes
    out and the tests pin the recurrence against.
  * Decay: a per-unit gamma multiplies every prefix moment (S, C, m) once per
    token.  For o_t = q_t^T(S_t C_t - G_t) to keep the closed form, G and h
    then take gamma^2 on the old value and gamma on the new cross term; the
    closed-form weight is gamma^((t-i)+(t-j)).  A segment of length L has
    decay a = gamma^L and the combine becomes
    S = a S_A + S_B, C = a C_A + C_B, m = a m_A + m_B,
    G = a^2 G_A + G_B + a S_B C_A, h = a^2 h_A + h_B + a S_B m_A.
  * Denominator: den_t = q_t^T (S_t m_t - h_t) (the same closed form with
    v = 1); the normalised output is num / (den + eps), no abs or clamp.
  * Inclusive sums, zero initial state, no 1/sqrt(d) and no feature map.
"""

import numpy as np

__all__ = [
    "zero_state", "serial", "brute", "matrix_form", "segment_summary",
    "segment_summary_sums",
    "identity_summary", "combine", "blelloch_exclusive_scan",
    "chunk_summaries", "chunk_outputs", "chunk_scan_forward", "decode_step",
    "normalise", "powers",
    "serial_unmasked", "brute_unmasked", "combine_unmasked",
    "unmasked_chunk_forward",
    "serial_ahla", "brute_ahla", "ahla_segment_summary", "ahla_identity", "combine_ahla",
    "ahla_chunk_forward",
]

_F = np.float64


def _f64(x):
    return np.asarray(x, dtype=_F)


def _gamma(gamma, U):
    """Per-unit decay as float64 [U]; None means gamma = 1 (no decay)."""
    if gamma is None:
        return np.ones(U, dtype=_F)
    g = _f64(gamma).reshape(-1)
    if g.size == 1:
        g = np.full(U, g[0], dtype=_F)
    assert g.shape == (U,)
    return g


def powers(gamma, n):
    """gamma**n in float64 with 0**0 = 1 (used for segment decays a = gamma^L)."""
    g = _f64(gamma)
    return np.where(np.asarray(n) == 0, 1.0, g ** np.asarray(n, dtype=_F))


def zero_state(U, d, dv):
    """The empty prefix: S, C, m, G, h all zero ([S1]; sums over no tokens)."""
    return {
        "S": np.zeros((U, d, d), _F), "C": np.zeros((U, d, dv), _F),
        "m": np.zeros((U, d), _F), "G": np.zeros((U, d, dv), _F),
        "h": np.zeros((U, d), _F),
    }


def serial(q, k, v, gamma=None, state=None):
    """Serial token-by-token recurrence ([S1]; decay per [C2] as read above).

    For t = 1..T, in order:
      G <- g^2 G + g k_t (k_t^T C),  h <- g^2 h + g k_t (k_t^T m)   (old C, m)
      S <- g S + k_t k_t^T,  C <- g C + q_t v_t^T,  m <- g m + q_t
      num_t = q_t^T (S C - G),  den_t = q_t^T (S m - h)
    q_t^T (S C) is evaluated as (q_t^T S) C: the same product, associated
    the cheap way, so the cost is O(d^2 + d dv) per token as [R] states.

    Returns (num [U,T,dv], den [U,T], final state dict).  `state` (optional)
    is the state before the first token; it is not modified.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    g1 = g[:, None]
    g2 = (g * g)[:, None]
    st = zero_state(U, d, dv) if state is None else {
        key: _f64(val).copy() for key, val in state.items()}
    S, C, m, G, h = st["S"], st["C"], st["m"], st["G"], st["h"]
    num = np.empty((U, T, dv), _F)
    den = np.empty((U, T), _F)
    for t in range(T):
        qt, kt, vt = q[:, t, :], k[:, t, :], v[:, t, :]
        kC = np.matmul(kt[:, None, :], C)[:, 0, :]          # k_t^T C_{t-1}
        km = np.sum(kt * m, axis=1)                          # k_t^T m_{t-1}
        G = g2[:, :, None] * G + g1[:, :, None] * kt[:, :, None] * kC[:, None, :]
        h = g2 * h + g1 * kt * km[:, None]
        S = g1[:, :, None] * S + kt[:, :, None] * kt[:, None, :]
        C = g1[:, :, None] * C + qt[:, :, None] * vt[:, None, :]
        m = g1 * m + qt
        qS = np.matmul(qt[:, None, :], S)[:, 0, :]            # q_t^T S_t
        num[:, t, :] = (np.matmul(qS[:, None, :], C)[:, 0, :]
                        - np.matmul(qt[:, None, :], G)[:, 0, :])
        den[:, t] = np.sum(qS * m, axis=1) - np.sum(qt * h, axis=1)
    return num, den, {"S": S, "C": C, "m": m, "G": G, "h": h}


def brute(q, k, v, gamma=None):
    """The closed form written out as a triple sum (tiny inputs only).

    num_t = sum_{j<=t} sum_{i<=j} w (q_t.k_i)(q_j.k_i) v_j,
    den_t = the same sum without v_j,  w = gamma^((t-i)+(t-j)).
    This is the masked AA^T V structure of [S1]/[S4] with A = Q K^T; the
    weight is the decay reading stated in the module docstring.
    Pure Python loops: O(T^3 d) per unit.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    num = np.zeros((U, T, dv), _F)
    den = np.zeros((U, T), _F)
    for u in range(U):
        for t in range(T):
            for j in range(t + 1):
                for i in range(j + 1):
                    w = float(g[u]) ** ((t - i) + (t - j))
                    s = w * float(q[u, t] @ k[u, i]) * float(q[u, j] @ k[u, i])
                    num[u, t] += s * v[u, j]
                    den[u, t] += s
    return num, den


def matrix_form(q, k, v, gamma=None):
    """The closed form as masked matrix products (library matmul as a step).

    With A = Q K^T and the decayed causal mask L[t,i] = gamma^(t-i) for i <= t
    (0 above the diagonal):  W = L o ((A o L) (A o 1_{i<=j})^T), num = W V,
    den = W 1.  Entry (t, j) of W is sum_{i<=j} gamma^((t-i)+(t-j))
    (q_t.k_i)(q_j.k_i) for j <= t, i.e. the double sum of `brute`.
    O(T^2 d) time and O(T^2) memory per unit.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    g = _gamma(gamma, U)
    idx = np.arange(T)
    diff = idx[:, None] - idx[None, :]                       # t - i
    lower = diff >= 0
    num = np.empty((U, T, v.shape[2]), _F)
    den = np.empty((U, T), _F)
    for u in range(U):
        L = np.where(lower, powers(g[u], np.maximum(diff, 0)), 0.0)
        A = q[u] @ k[u].T
        W = L * ((A * L) @ (A * lower).T)
        num[u] = W @ v[u]
        den[u] = W.sum(axis=1)
    return num, den


# ----------------------------------------------------------------------------
# Segment summaries, the semidirect-product combine, the exclusive Blelloch
# scan and the chunk-parallel forward ([S4]).
# ----------------------------------------------------------------------------

def segment_summary(q, k, v, gamma=None):
    """Summary of one token segment: the state the serial recurrence reaches
    from the empty prefix after the segment's tokens, plus its length L
    (decay a = gamma^L).  q, k: [U, L, d]; v: [U, L, dv]."""
    _, _, st = serial(q, k, v, gamma)
    st["L"] = np.full(np.shape(q)[0], np.shape(q)[1], dtype=np.int64)
    return st


def segment_summary_sums(q, k, v, gamma=None):
    """The same summary as explicit weighted sums over the segment
    (positions 1..L, weights from the decay reading), with library matmuls:
      S = sum_i g^(L-i) k_i k_i^T,  C = sum_j g^(L-j) q_j v_j^T,
      m = sum_j g^(L-j) q_j,
      G = sum_{j<i} g^((L-i)+(L-j)) k_i (k_i.q_j) v_j^T,  h = the same with v = 1.
    These are the recurrence unrolled; the tests pin one against the other.
    O(L^2 d) per unit, so long prefixes are cheap."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, L, d = q.shape
    g = _gamma(gamma, U)
    pos = np.arange(1, L + 1)
    out = zero_state(U, d, v.shape[2])
    strict = pos[:, None] > pos[None, :]                       # j < i
    for u in range(U):
        w = powers(g[u], L - pos)                               # g^(L-i)
        out["S"][u] = (k[u] * w[:, None]).T @ k[u]
        out["C"][u] = (q[u] * w[:, None]).T @ v[u]
        out["m"][u] = (q[u] * w[:, None]).sum(axis=0)
        X = np.where(strict, (w[:, None] * w[None, :]) * (k[u] @ q[u].T), 0.0)
        out["G"][u] = k[u].T @ (X @ v[u])
        out["h"][u] = k[u].T @ X.sum(axis=1)
    out["L"] = np.full(U, L, dtype=np.int64)
    return out


def identity_summary(U, d, dv):
    """Neutral element of the combine: zero moments, length 0 (a = 1)."""
    st = zero_state(U, d, dv)
    st["L"] = np.zeros(U, dtype=np.int64)
    return st


def combine(A, B, gamma=None):
    """Segment A followed by segment B ([S4]: semidirect product with the
    cross term S_B C_A; decay per [C2] as read in the module docstring).

    a = gamma^(L_B):
      S = a S_A + S_B,  C = a C_A + C_B,  m = a m_A + m_B,
      G = a^2 G_A + G_B + a S_B C_A,  h = a^2 h_A + h_B + a S_B m_A,
      L = L_A + L_B.
    """
    U = A["S"].shape[0]
    g = _gamma(gamma, U)
    a = powers(g, B["L"])
    a1 = a[:, None]
    a3 = a[:, None, None]
    return {
        "S": a3 * A["S"] + B["S"],
        "C": a3 * A["C"] + B["C"],
        "m": a1 * A["m"] + B["m"],
        "G": a3 * a3 * A["G"] + B["G"] + a3 * np.matmul(B["S"], A["C"]),
        "h": a1 * a1 * A["h"] + B["h"] + a1 * np.matmul(B["S"], A["m"][:, :, None])[:, :, 0],
        "L": A["L"] + B["L"],
    }


def blelloch_exclusive_scan(summaries, gamma=None, op=None):
    """Exclusive Blelloch scan ([S4]) of a list of n segment summaries.

    Work-efficient up-sweep then down-sweep over an array padded to a power
    of two with identities.  The operator is not commutative: in the
    down-sweep a right child receives (parent prefix) combined with (left
    sum), in that order.  Returns the list of exclusive prefixes
    P_i = s_0 (+) ... (+) s_{i-1}, P_0 = identity.  `op` is the combine
    (default: the masked one above; combine_unmasked for the unmasked variant).
    """
    op = combine if op is None else op
    n = len(summaries)
    if n == 0:
        return []
    U, d, dv = summaries[0]["C"].shape
    N = 1
    while N < n:
        N *= 2
    x = [dict(s) for s in summaries] + [identity_summary(U, d, dv) for _ in range(N - n)]
    step = 1
    while step < N:                                   # up-sweep
        for j in range(2 * step - 1, N, 2 * step):
            x[j] = op(x[j - step], x[j], gamma)
        step *= 2
    x[N - 1] = identity_summary(U, d, dv)
    step = N // 2
    while step >= 1:                                  # down-sweep
        for j in range(2 * step - 1, N, 2 * step):
            left = x[j - step]
            x[j - step] = x[j]
            x[j] = op(x[j], left, gamma)
        step //= 2
    return x[:n]


def chunk_summaries(q, k, v, chunk, gamma=None):
    """Split [U, T, .] into n = T / chunk segments and summarise each."""
    T = np.shape(q)[1]
    assert chunk > 0 and T % chunk == 0
    return [segment_summary(q[:, s:s + chunk], k[:, s:s + chunk], v[:, s:s + chunk], gamma)
            for s in range(0, T, chunk)]


def chunk_outputs(q, k, v, chunk, prefixes, gamma=None):
    """Outputs of every chunk: the recurrence continued inside the chunk from
    that chunk's exclusive prefix state."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, _ = q.shape
    num = np.empty((U, T, v.shape[2]), _F)
    den = np.empty((U, T), _F)
    for c, s in enumerate(range(0, T, chunk)):
        P = {key: prefixes[c][key] for key in ("S", "C", "m", "G", "h")}
        n_, d_, _ = serial(q[:, s:s + chunk], k[:, s:s + chunk], v[:, s:s + chunk], gamma, P)
        num[:, s:s + chunk] = n_
        den[:, s:s + chunk] = d_
    return num, den


def chunk_scan_forward(q, k, v, chunk, gamma=None):
    """Chunk-parallel forward of [S4]: summaries -> exclusive Blelloch scan
    -> per-chunk outputs.  Also returns the prefixes and the inclusive total
    (the state after the whole sequence)."""
    sums = chunk_summaries(q, k, v, chunk, gamma)
    pre = blelloch_exclusive_scan(sums, gamma)
    num, den = chunk_outputs(q, k, v, chunk, pre, gamma)
    total = combine(pre[-1], sums[-1], gamma) if sums else None
    return num, den, pre, total


def decode_step(state, q, k, v, gamma=None):
    """One streaming step ([S1] online update, [R] constant cost per token):
    the serial recurrence applied to a single token per unit.
    state: dict of [U, ...]; q, k: [U, d]; v: [U, dv].
    Returns (num [U, dv], den [U], new state)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    num, den, st = serial(q[:, None, :], k[:, None, :], v[:, None, :], gamma, state)
    return num[:, 0, :], den[:, 0], st


def normalise(num, den, eps):
    """Ratio-normalised output of [S1]: numerator / (masked denominator + eps).
    No absolute value or clamp (the reading of the unstated placement)."""
    return _f64(num) / (_f64(den)[..., None] + float(eps))


# ----------------------------------------------------------------------------
# The unmasked second-order variant.  [S1] notes that the plain product
# S^K_t C^QV_t includes future terms (pairs with key index i after the query
# index j) -- that is the unmasked operator, o_t = q_t^T S_t C_t, which the
# cross summaries G, h are there to remove; [C2] states that the associative
# operators exist for the unmasked setting too, with and without decay.
# Readings: the same decay placement as above (S, C, m decay once per token),
# so the closed-form weight is again gamma^((t-i)+(t-j)); the ratio-normalised
# form divides by q_t^T S_t m_t (v = 1) plus eps.
# ----------------------------------------------------------------------------

def serial_unmasked(q, k, v, gamma=None, state=None):
    """Serial recurrence of the unmasked variant: for t = 1..T, in order,
      S <- g S + k_t k_t^T,  C <- g C + q_t v_t^T,  m <- g m + q_t,
      num_t = (q_t^T S) C,  den_t = (q_t^T S) m.
    Returns (num [U,T,dv], den [U,T], final state {S, C, m}).  `state`
    (optional, with S, C, m) is the state before the first token."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    g1 = g[:, None]
    if state is None:
        S, C, m = np.zeros((U, d, d), _F), np.zeros((U, d, dv), _F), np.zeros((U, d), _F)
    else:
        S, C, m = (_f64(state[key]).copy() for key in ("S", "C", "m"))
    num = np.empty((U, T, dv), _F)
    den = np.empty((U, T), _F)
    for t in range(T):
        qt, kt, vt = q[:, t, :], k[:, t, :], v[:, t, :]
        S = g1[:, :, None] * S + kt[:, :, None] * kt[:, None, :]
        C = g1[:, :, None] * C + qt[:, :, None] * vt[:, None, :]
        m = g1 * m + qt
        qS = np.matmul(qt[:, None, :], S)[:, 0, :]
        num[:, t, :] = np.matmul(qS[:, None, :], C)[:, 0, :]
        den[:, t] = np.sum(qS * m, axis=1)
    return num, den, {"S": S, "C": C, "m": m}


def brute_unmasked(q, k, v, gamma=None):
    """Closed form of the unmasked variant as a triple sum (tiny inputs only):
    num_t = sum_{i<=t} sum_{j<=t} w (q_t.k_i)(k_i.q_j) v_j, den_t without v_j,
    w = gamma^((t-i)+(t-j)): the key index i and the value index j are both
    bounded by t only, not ordered against each other."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    num = np.zeros((U, T, dv), _F)
    den = np.zeros((U, T), _F)
    for u in range(U):
        for t in range(T):
            for i in range(t + 1):
                for j in range(t + 1):
                    w = float(g[u]) ** ((t - i) + (t - j))
                    s = w * float(q[u, t] @ k[u, i]) * float(k[u, i] @ q[u, j])
                    num[u, t] += s * v[u, j]
                    den[u, t] += s
    return num, den


def combine_unmasked(A, B, gamma=None):
    """Segment A followed by segment B for the unmasked variant ([C2]): the
    moments only, no cross term.  a = gamma^(L_B):
      S = a S_A + S_B,  C = a C_A + C_B,  m = a m_A + m_B,  L = L_A + L_B."""
    U = A["S"].shape[0]
    a = powers(_gamma(gamma, U), B["L"])
    return {
        "S": a[:, None, None] * A["S"] + B["S"],
        "C": a[:, None, None] * A["C"] + B["C"],
        "m": a[:, None] * A["m"] + B["m"],
        "G": np.zeros_like(A["G"]), "h": np.zeros_like(A["h"]),
        "L": A["L"] + B["L"],
    }


def unmasked_chunk_forward(q, k, v, chunk, gamma=None):
    """Chunk-parallel form of the unmasked variant ([S4], [C2]): per segment
    the state the unmasked recurrence reaches from zero, an exclusive
    Blelloch scan under combine_unmasked, then the recurrence continued
    inside each segment from its prefix.  Returns (num, den, prefixes)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    assert chunk > 0 and T % chunk == 0
    sums = []
    for s in range(0, T, chunk):
        _, _, st = serial_unmasked(q[:, s:s + chunk], k[:, s:s + chunk], v[:, s:s + chunk], gamma)
        st["G"] = np.zeros((U, d, dv), _F)
        st["h"] = np.zeros((U, d), _F)
        st["L"] = np.full(U, chunk, dtype=np.int64)
        sums.append(st)
    pre = blelloch_exclusive_scan(sums, gamma, op=combine_unmasked)
    num = np.empty((U, T, dv), _F)
    den = np.empty((U, T), _F)
    for c, s in enumerate(range(0, T, chunk)):
        n_, d_, _ = serial_unmasked(q[:, s:s + chunk], k[:, s:s + chunk], v[:, s:s + chunk],
                                    gamma, pre[c])
        num[:, s:s + chunk] = n_
        den[:, s:s + chunk] = d_
    return num, den, pre


# ----------------------------------------------------------------------------
# The asymmetric variant AHLA (method section 2 of the pages): the operator
# Q (K^T Q)(K^T V), which weights the values along a single path through an
# intermediate key index, with the streaming summaries P^KV, m^K, E, n and
# the same linear cost per token.  Readings (not spelled out on the pages):
#   * causal masking follows the path t -> i -> j back in time:
#     o_t = sum_{i<=t} sum_{j<=i} (q_t.k_i)(q_i.k_j) v_j, the masked A A V
#     with A = Q K^T (the symmetric HLA is the masked A A^T V);
#   * P^KV_t = sum_{j<=t} k_j v_j^T and m^K_t = sum_{j<=t} k_j (inclusive),
#     E_t = sum_{i<=t} k_i (q_i^T P^KV_i), n_t = sum_{i<=t} k_i (q_i.m^K_i),
#     o_t = q_t^T E_t, den_t = q_t^T n_t (the same sums with v = 1);
#   * decay: every prefix moment (P, m, E, n) decays once per token, so the
#     closed-form weight is gamma^(t-j).
# Segment combine (A then B, a = gamma^(length of B)), derived from these
# definitions: P = a P_A + P_B, m = a m_A + m_B, E = a E_A + E_B + a X_B P_A,
# n = a n_A + n_B + a X_B m_A with X_B = sum_{i in B} k_i q_i^T (no decay
# weights: the decay of the path through i cancels), X = X_A + X_B.
# ----------------------------------------------------------------------------

def serial_ahla(q, k, v, gamma=None, state=None):
    """Serial recurrence of AHLA: for t = 1..T, in order,
      P <- g P + k_t v_t^T,  m <- g m + k_t,
      r = P^T q_t,  rm = q_t.m,
      E <- g E + k_t r^T,  n <- g n + k_t rm,
      num_t = E^T q_t,  den_t = q_t.n.
    Returns (num [U,T,dv], den [U,T], final state {P, m, E, n}); `state`
    (optional, same keys) is the state before the first token."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g1 = _gamma(gamma, U)[:, None]
    if state is None:
        P, m = np.zeros((U, d, dv), _F), np.zeros((U, d), _F)
        E, n = np.zeros((U, d, dv), _F), np.zeros((U, d), _F)
    else:
        P, m, E, n = (_f64(state[key]).copy() for key in ("P", "m", "E", "n"))
    num = np.empty((U, T, dv), _F)
    den = np.empty((U, T), _F)
    for t in range(T):
        qt, kt, vt = q[:, t, :], k[:, t, :], v[:, t, :]
        P = g1[:, :, None] * P + kt[:, :, None] * vt[:, None, :]
        m = g1 * m + kt
        r = np.matmul(qt[:, None, :], P)[:, 0, :]              # P^T q_t
        rm = np.sum(qt * m, axis=1)
        E = g1[:, :, None] * E + kt[:, :, None] * r[:, None, :]
        n = g1 * n + kt * rm[:, None]
        num[:, t, :] = np.matmul(qt[:, None, :], E)[:, 0, :]
        den[:, t] = np.sum(qt * n, axis=1)
    return num, den, {"P": P, "m": m, "E": E, "n": n}


def brute_ahla(q, k, v, gamma=None):
    """Closed form of AHLA as a triple sum (tiny inputs only):
    num_t = sum_{i<=t} sum_{j<=i} gamma^(t-j) (q_t.k_i)(q_i.k_j) v_j, den_t
    without v_j."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    num = np.zeros((U, T, dv), _F)
    den = np.zeros((U, T), _F)
    for u in range(U):
        for t in range(T):
            for i in range(t + 1):
                for j in range(i + 1):
                    w = float(g[u]) ** (t - j)
                    s = w * float(q[u, t] @ k[u, i]) * float(q[u, i] @ k[u, j])
                    num[u, t] += s * v[u, j]
                    den[u, t] += s
    return num, den


def ahla_identity(U, d, dv):
    """Neutral element of combine_ahla: zero summaries, length 0."""
    z = lambda *s: np.zeros((U,) + s, _F)
    return {"P": z(d, dv), "m": z(d), "E": z(d, dv), "n": z(d), "X": z(d, d),
            "L": np.zeros(U, dtype=np.int64)}


def ahla_segment_summary(q, k, v, gamma=None):
    """Summary of one segment: the state the AHLA recurrence reaches from
    zero, X = sum_i k_i q_i^T (undecayed) and the length L."""
    _, _, st = serial_ahla(q, k, v, gamma)
    st["X"] = np.matmul(np.swapaxes(_f64(k), 1, 2), _f64(q))
    st["L"] = np.full(np.shape(q)[0], np.shape(q)[1], dtype=np.int64)
    return st


def combine_ahla(A, B, gamma=None):
    """Segment A followed by segment B (see the section comment):
      P = a P_A + P_B, m = a m_A + m_B, E = a E_A + E_B + a X_B P_A,
      n = a n_A + n_B + a X_B m_A, X = X_A + X_B, L = L_A + L_B."""
    U = A["P"].shape[0]
    a = powers(_gamma(gamma, U), B["L"])
    a1, a3 = a[:, None], a[:, None, None]
    return {
        "P": a3 * A["P"] + B["P"],
        "m": a1 * A["m"] + B["m"],
        "E": a3 * A["E"] + B["E"] + a3 * np.matmul(B["X"], A["P"]),
        "n": a1 * A["n"] + B["n"] + a1 * np.matmul(B["X"], A["m"][:, :, None])[:, :, 0],
        "X": A["X"] + B["X"],
        "L": A["L"] + B["L"],
    }


def ahla_chunk_forward(q, k, v, chunk, gamma=None):
    """Chunk-parallel AHLA: segment summaries, exclusive prefixes under
    combine_ahla (left to right), then the recurrence continued inside each
    segment from its prefix.  Returns (num, den, prefixes)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    assert chunk > 0 and T % chunk == 0
    sums = [ahla_segment_summary(q[:, s:s + chunk], k[:, s:s + chunk], v[:, s:s + chunk], gamma)
            for s in range(0, T, chunk)]
    pre, run = [], ahla_identity(U, d, dv)
    for sm in sums:
        pre.append(run)
        run = combine_ahla(run, sm, gamma)
    num = np.empty((U, T, dv), _F)
    den = np.empty((U, T), _F)
    for c, s in enumerate(range(0, T, chunk)):
        n_, d_, _ = serial_ahla(q[:, s:s + chunk], k[:, s:s + chunk], v[:, s:s + chunk], gamma, pre[c])
        num[:, s:s + chunk] = n_
        den[:, s:s + chunk] = d_
    return num, den, pre
