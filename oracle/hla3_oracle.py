"""CPU oracle for the masked third-order HLA forward and its decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP path.

Plain NumPy in float64, batched over independent units u = (batch, head):
q, k are [U, T, d], v is [U, T, dv], gamma is [U] (None means 1).

Sources: the summaries of "Higher-order Linear Attention" (arXiv 2510.27258)
on gist.science, Japanese and French pages:

  [M3]  method section 3, third-order HLA: the interaction A A^T A with
        A = Q K^T; the masked output needs three prefix moments S^K_t, S^Q_t,
        P^KV_t and six cross summaries G^(1..3)_t, h^(1..3)_t to enforce
        strict causality; the online update stays linear in the feature
        dimension while the state grows.
  [M4]  method section 4, parallel training by associative scans: segment
        summaries joined by an associative operator, an exclusive Blelloch
        scan; for the third order the operator carries segment-level linear
        maps M^KQP and M^KQm.
  [K3]  key contribution 3: the masked third-order state, its online update,
        a strictly causal streaming kernel and an exact chunk-parallel
        algorithm.
  [C2]  key contribution 2: decayed variants of the associative operators.

The pages give no formula for any of these.  Readings (each listed with its
reason in the design notes):

  * Masked output.  A_L = L o A (L lower-triangular with the diagonal) and
    the causal mask on the A A^T factor as in the second order:
        O = (L o (A_L A_L^T)) A_L V,
    i.e. o_t = sum_{j<=t} sum_{i<=j} sum_{l<=j} (q_t.k_i)(q_j.k_i)(q_j.k_l) v_l:
    query j may use keys i and values l no later than itself.
  * Decay: every prefix moment decays by gamma once per token, so the term
    (i, j, l) at time t carries gamma^((t-i)+(t-j)+(t-l)).
  * The moments S^K = sum k k^T, S^Q = sum q q^T, P^KV = sum k v^T (and
    m^K = sum k for the denominator).  The unmasked product q_t^T S^K S^Q
    P^KV sums over every (i, j, l) <= t; the three cross summaries are the
    three classes of terms the mask forbids:
        G^(1): key after the query (i > j), value not (l <= j),
        G^(2): value after the query (l > j), key not (i <= j),
        G^(3): both after the query (i > j and l > j),
    so num_t = q_t^T (S^K S^Q P^KV - G^(1) - G^(2) - G^(3)); h^(1..3) are the
    same with v = 1 (P^KV -> m^K) and den_t = q_t^T (S^K S^Q m^K - h^(1) -
    h^(2) - h^(3)).  Their updates need the running sums
    V = sum g^(2(t-j)) S^K_j q_j q_j^T, Z = sum g^(2(t-j)) q_j q_j^T P^KV_j,
    z (Z with m^K) and the products S^K S^Q, S^Q P^KV, S^Q m^K (all kept
    with O(d^2 + d dv) work per token).
  * Equivalently o_t = q_t^T R_t with R_t = sum_{j<=t} g^(3(t-j)) p_j u_j^T,
    p_j = S^K_j q_j, u_j = P^KV_j^T q_j (and den with u_j -> m^K_j . q_j).
  * Segment combine (A then B, a = g^(length of B)), derived from the
    definitions, on the summary (S, Q, P, m, V, Z, z, R, r):
        S = a S_A + S_B, Q = a Q_A + Q_B, P = a P_A + P_B, m = a m_A + m_B,
        V = a^2 V_A + V_B + a S_A Q_B,
        Z = a^2 Z_A + Z_B + a Q_B P_A,      z likewise with m_A,
        R = a^3 R_A + R_B + a S_A Z_B + M^KQ P_A,
        r = a^3 r_A + r_B + a S_A z_B + M^KQ m_A,
    with the segment map M^KQ = a^2 S_A Q_B + a V_B (a d x d matrix built
    from the key and query moments) applied to P^KV_A and to m^K_A: the
    pages' M^KQP and M^KQm.
  * Ratio normalisation o = num / (den + eps) as in the second order.
"""

import numpy as np

__all__ = ["serial3", "serial3_r", "brute3", "brute3_classes", "matrix_form3",
           "segment_summary3", "identity3", "combine3", "blelloch_exclusive_scan3",
           "chunk_forward3", "decode_step3", "zero_state3"]

_F = np.float64


def _f64(x):
    return np.asarray(x, dtype=_F)


def _gamma(gamma, U):
    if gamma is None:
        return np.ones(U, dtype=_F)
    g = _f64(gamma).reshape(-1)
    if g.size == 1:
        g = np.full(U, g[0], dtype=_F)
    assert g.shape == (U,)
    return g


def _mv(M, x):
    """[U, a, b] @ [U, b] -> [U, a]."""
    return np.einsum("uab,ub->ua", M, x)


def _vm(x, M):
    """[U, a] @ [U, a, b] -> [U, b]."""
    return np.einsum("ua,uab->ub", x, M)


def _outer(x, y):
    return x[:, :, None] * y[:, None, :]


def serial3(q, k, v, gamma=None):
    """The pages' form ([M3]): the moments, the six cross summaries and the
    running sums their updates need, token by token; for t = 1..T, in order
    (every right-hand side uses the state before token t; g = gamma):
      G1 <- g^3 G1 + g^2 k (k^T Z)
      G2 <- g^3 G2 + g^2 (V k) v^T
      G3 <- g^3 G3 + g^2 (SQ - V) k v^T + g^2 k k^T (QP - Z) + g (k^T Q k) k v^T
      h1, h2, h3: the same with v = 1 (P -> m, Z -> z, QP -> Qm)
      SQ <- g^2 SQ + g (S q) q^T + g k (k^T Q) + (k.q) k q^T       (= S Q)
      QP <- g^2 QP + g (Q k) v^T + g q (q^T P) + (q.k) q v^T       (= Q P)
      Qm <- g^2 Qm + g Q k + g (q.m) q + (q.k) q                   (= Q m)
      S <- g S + k k^T,  Q <- g Q + q q^T,  P <- g P + k v^T,  m <- g m + k
      V <- g^2 V + (S q) q^T,  Z <- g^2 Z + q (q^T P),  z <- g^2 z + (q.m) q
                                                  (S, P, m already updated)
      num_t = ((S q)^T Q) P - q^T (G1 + G2 + G3)
      den_t = ((S q)^T Q) m - q^T (h1 + h2 + h3)
    Returns (num [U, T, dv], den [U, T])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    g1, g2, g3 = g[:, None], (g * g)[:, None], (g ** 3)[:, None]
    G1, G2, G3 = (np.zeros((U, d, dv)) for _ in range(3))
    h1, h2, h3 = (np.zeros((U, d)) for _ in range(3))
    S, Q, V, SQ = (np.zeros((U, d, d)) for _ in range(4))
    P, Z, QP = (np.zeros((U, d, dv)) for _ in range(3))
    m, z, Qm = (np.zeros((U, d)) for _ in range(3))
    num = np.empty((U, T, dv))
    den = np.empty((U, T))
    for t in range(T):
        qt, kt, vt = q[:, t], k[:, t], v[:, t]
        kZ, kz = _vm(kt, Z), np.sum(kt * z, axis=1)
        Vk = _mv(V, kt)
        SQk_Vk = _mv(SQ, kt) - Vk
        kQP_Z, kQm_z = _vm(kt, QP - Z), np.sum(kt * (Qm - z), axis=1)
        kQk = np.sum(kt * _mv(Q, kt), axis=1)
        G1 = g3[:, :, None] * G1 + g2[:, :, None] * _outer(kt, kZ)
        h1 = g3 * h1 + g2 * kt * kz[:, None]
        G2 = g3[:, :, None] * G2 + g2[:, :, None] * _outer(Vk, vt)
        h2 = g3 * h2 + g2 * Vk
        G3 = (g3[:, :, None] * G3 + g2[:, :, None] * _outer(SQk_Vk, vt)
              + g2[:, :, None] * _outer(kt, kQP_Z) + (g1 * kQk[:, None])[:, :, None] * _outer(kt, vt))
        h3 = g3 * h3 + g2 * SQk_Vk + g2 * kt * kQm_z[:, None] + g1 * kQk[:, None] * kt
        qk = np.sum(qt * kt, axis=1)[:, None]
        Sq_old, kQ_old, Qk_old = _mv(S, qt), _vm(kt, Q), _mv(Q, kt)
        qP_old, qm_old = _vm(qt, P), np.sum(qt * m, axis=1)[:, None]
        SQ = (g2[:, :, None] * SQ + g1[:, :, None] * _outer(Sq_old, qt)
              + g1[:, :, None] * _outer(kt, kQ_old) + qk[:, :, None] * _outer(kt, qt))
        QP = (g2[:, :, None] * QP + g1[:, :, None] * _outer(Qk_old, vt)
              + g1[:, :, None] * _outer(qt, qP_old) + qk[:, :, None] * _outer(qt, vt))
        Qm = g2 * Qm + g1 * Qk_old + g1 * qm_old * qt + qk * qt
        S = g1[:, :, None] * S + _outer(kt, kt)
        Q = g1[:, :, None] * Q + _outer(qt, qt)
        P = g1[:, :, None] * P + _outer(kt, vt)
        m = g1 * m + kt
        Sq = _mv(S, qt)
        V = g2[:, :, None] * V + _outer(Sq, qt)
        Z = g2[:, :, None] * Z + _outer(qt, _vm(qt, P))
        z = g2 * z + np.sum(qt * m, axis=1)[:, None] * qt
        SqQ = _vm(Sq, Q)
        num[:, t] = _vm(SqQ, P) - _vm(qt, G1 + G2 + G3)
        den[:, t] = np.sum(SqQ * m, axis=1) - np.sum(qt * (h1 + h2 + h3), axis=1)
    return num, den


def zero_state3(U, d, dv):
    """Decode state (S, P, m, R, r) after no tokens."""
    return {"S": np.zeros((U, d, d)), "P": np.zeros((U, d, dv)), "m": np.zeros((U, d)),
            "R": np.zeros((U, d, dv)), "r": np.zeros((U, d))}


def serial3_r(q, k, v, gamma=None, state=None):
    """The single-sum form of the same output: for t = 1..T, in order,
      S <- g S + k k^T,  P <- g P + k v^T,  m <- g m + k,
      p = S q,  u = P^T q,  R <- g^3 R + p u^T,  r <- g^3 r + (q.m) p,
      num_t = R^T q,  den_t = r.q.
    Returns (num, den, state) with state = {S, P, m, R, r} after the last
    token (the decode state)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    g1, g3 = g[:, None], (g ** 3)[:, None]
    st = zero_state3(U, d, dv) if state is None else {x: _f64(y).copy() for x, y in state.items()}
    S, P, m, R, r = st["S"], st["P"], st["m"], st["R"], st["r"]
    num = np.empty((U, T, dv))
    den = np.empty((U, T))
    for t in range(T):
        qt, kt, vt = q[:, t], k[:, t], v[:, t]
        S = g1[:, :, None] * S + _outer(kt, kt)
        P = g1[:, :, None] * P + _outer(kt, vt)
        m = g1 * m + kt
        p, u = _mv(S, qt), _vm(qt, P)
        R = g3[:, :, None] * R + _outer(p, u)
        r = g3 * r + np.sum(qt * m, axis=1)[:, None] * p
        num[:, t] = _vm(qt, R)
        den[:, t] = np.sum(qt * r, axis=1)
    return num, den, {"S": S, "P": P, "m": m, "R": R, "r": r}


def decode_step3(state, q, k, v, gamma=None):
    """One streaming step ([K3] online update): q, k [U, d], v [U, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    num, den, st = serial3_r(q[:, None], k[:, None], v[:, None], gamma, state)
    return num[:, 0], den[:, 0], st


def brute3(q, k, v, gamma=None):
    """The closed form as a quadruple loop (tiny inputs only):
    num_t = sum_{j<=t} sum_{i<=j} sum_{l<=j} g^((t-i)+(t-j)+(t-l))
            (q_t.k_i)(q_j.k_i)(q_j.k_l) v_l,  den_t the same without v_l."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    g = _gamma(gamma, U)
    num = np.zeros((U, T, v.shape[2]))
    den = np.zeros((U, T))
    for u in range(U):
        for t in range(T):
            for j in range(t + 1):
                for i in range(j + 1):
                    for l in range(j + 1):
                        w = g[u] ** ((t - i) + (t - j) + (t - l))
                        c = w * (q[u, t] @ k[u, i]) * (q[u, j] @ k[u, i]) * (q[u, j] @ k[u, l])
                        num[u, t] += c * v[u, l]
                        den[u, t] += c
    return num, den


def brute3_classes(q, k, v, gamma=None):
    """The unmasked product and the three forbidden classes as matrices,
    summed term by term (tiny inputs only): for each t,
      F_t  = sum over all i, j, l <= t of w k_i k_i^T q_j q_j^T k_l v_l^T,
      G1_t = the terms with i > j, l <= j;  G2_t: i <= j, l > j;
      G3_t: i > j, l > j;  w = g^((t-i)+(t-j)+(t-l)).
    Returns F, G1, G2, G3 as [U, T, d, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    out = [np.zeros((U, T, d, dv)) for _ in range(4)]
    for u in range(U):
        for t in range(T):
            for j in range(t + 1):
                for i in range(t + 1):
                    for l in range(t + 1):
                        w = g[u] ** ((t - i) + (t - j) + (t - l))
                        term = w * np.outer(k[u, i], k[u, i]) @ np.outer(q[u, j], q[u, j]) @ \
                            np.outer(k[u, l], v[u, l])
                        out[0][u, t] += term
                        if i > j and l <= j:
                            out[1][u, t] += term
                        elif i <= j and l > j:
                            out[2][u, t] += term
                        elif i > j and l > j:
                            out[3][u, t] += term
    return tuple(out)


def matrix_form3(q, k, v, gamma=None):
    """Library matmuls of the masked matrices: with L_g[t, s] = g^(t-s) [s <= t],
    P = (L_g o Q K^T) K (rows p_t = S_t q_t), U = (L_g o Q K^T) V,
    num = (L_{g^3} o Q P^T) U, den the same with U -> (L_g o Q K^T) 1."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U_, T, d = q.shape
    g = _gamma(gamma, U_)
    idx = np.arange(T)
    diff = idx[:, None] - idx[None, :]
    low = diff >= 0
    num = np.empty((U_, T, v.shape[2]))
    den = np.empty((U_, T))
    for u in range(U_):
        if g[u] == 0.0:
            L1 = np.eye(T)
            L3 = np.eye(T)
        else:
            L1 = np.where(low, g[u] ** np.where(low, diff, 0), 0.0)
            L3 = np.where(low, (g[u] ** 3) ** np.where(low, diff, 0), 0.0)
        A = L1 * (q[u] @ k[u].T)
        P = A @ k[u]
        Uv = A @ v[u]
        um = A @ np.ones(T)
        W = L3 * (q[u] @ P.T)
        num[u] = W @ Uv
        den[u] = W @ um
    return num, den


# ---- segment summaries and the third-order scan ([M4], [K3]) -------------------

def segment_summary3(q, k, v, gamma=None):
    """Summary of one segment from the zero state, by walking its tokens:
    S, Q, P, m (decayed moments), V = sum g^(2(L-j)) S_j q_j q_j^T,
    Z = sum g^(2(L-j)) q_j q_j^T P_j, z likewise with m, R, r as in
    serial3_r, and the decay a = g^L.  Positions j are local to the segment."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, L, d = q.shape
    dv = v.shape[2]
    g = _gamma(gamma, U)
    g1, g2, g3 = g[:, None], (g * g)[:, None], (g ** 3)[:, None]
    S, Q, V = (np.zeros((U, d, d)) for _ in range(3))
    P, Z, R = (np.zeros((U, d, dv)) for _ in range(3))
    m, z, r = (np.zeros((U, d)) for _ in range(3))
    for t in range(L):
        qt, kt, vt = q[:, t], k[:, t], v[:, t]
        S = g1[:, :, None] * S + _outer(kt, kt)
        Q = g1[:, :, None] * Q + _outer(qt, qt)
        P = g1[:, :, None] * P + _outer(kt, vt)
        m = g1 * m + kt
        p, u, qm = _mv(S, qt), _vm(qt, P), np.sum(qt * m, axis=1)[:, None]
        V = g2[:, :, None] * V + _outer(p, qt)
        Z = g2[:, :, None] * Z + _outer(qt, u)
        z = g2 * z + qm * qt
        R = g3[:, :, None] * R + _outer(p, u)
        r = g3 * r + qm * p
    return {"S": S, "Q": Q, "P": P, "m": m, "V": V, "Z": Z, "z": z, "R": R, "r": r,
            "a": g ** L}


def identity3(U, d, dv):
    z = lambda *s: np.zeros((U,) + s)
    return {"S": z(d, d), "Q": z(d, d), "P": z(d, dv), "m": z(d), "V": z(d, d),
            "Z": z(d, dv), "z": z(d), "R": z(d, dv), "r": z(d), "a": np.ones(U)}


def combine3(A, B):
    """A then B under the third-order operator (see the module notes):
    a = B's decay; the segment map M^KQ = a^2 S_A Q_B + a V_B acts on A's
    P^KV (M^KQP) and m^K (M^KQm)."""
    a = B["a"]
    a1, a2, a3 = a[:, None], (a * a)[:, None], (a ** 3)[:, None]
    A1, A2, A3 = a1[:, :, None], a2[:, :, None], a3[:, :, None]
    SAQB = np.matmul(A["S"], B["Q"])
    MKQ = A2 * SAQB + A1 * B["V"]
    return {
        "S": A1 * A["S"] + B["S"], "Q": A1 * A["Q"] + B["Q"],
        "P": A1 * A["P"] + B["P"], "m": a1 * A["m"] + B["m"],
        "V": A2 * A["V"] + B["V"] + A1 * SAQB,
        "Z": A2 * A["Z"] + B["Z"] + A1 * np.matmul(B["Q"], A["P"]),
        "z": a2 * A["z"] + B["z"] + a1 * _mv(B["Q"], A["m"]),
        "R": A3 * A["R"] + B["R"] + A1 * np.matmul(A["S"], B["Z"]) + np.matmul(MKQ, A["P"]),
        "r": a3 * A["r"] + B["r"] + a1 * _mv(A["S"], B["z"]) + _mv(MKQ, A["m"]),
        "a": A["a"] * B["a"],
    }


def blelloch_exclusive_scan3(summaries):
    """Exclusive Blelloch scan ([M4]) of a list of summaries under combine3,
    padded to a power of two with identities; the down-sweep puts the parent
    prefix first (the operator is not commutative)."""
    n = len(summaries)
    U = summaries[0]["a"].shape[0]
    d, dv = summaries[0]["P"].shape[1:]
    N = 1
    while N < n:
        N *= 2
    x = list(summaries) + [identity3(U, d, dv) for _ in range(N - n)]
    step = 1
    while step < N:
        for i in range(2 * step - 1, N, 2 * step):
            x[i] = combine3(x[i - step], x[i])
        step *= 2
    x[N - 1] = identity3(U, d, dv)
    step = N // 2
    while step >= 1:
        for i in range(2 * step - 1, N, 2 * step):
            left = x[i - step]
            x[i - step] = x[i]
            x[i] = combine3(x[i], left)
        step //= 2
    return x[:n]


def chunk_forward3(q, k, v, chunk, gamma=None):
    """Chunk-parallel form ([M4], [K3]): segment summaries, their exclusive
    scan, then each segment continues the single-sum recurrence from its
    exclusive prefix (S, P, m, R, r).  Returns (num, den, inclusive total)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    U, T, d = q.shape
    assert T % chunk == 0
    n = T // chunk
    seg = lambda x, s: x[:, s * chunk:(s + 1) * chunk]
    sums = [segment_summary3(seg(q, s), seg(k, s), seg(v, s), gamma) for s in range(n)]
    pre = blelloch_exclusive_scan3(sums)
    nums, dens = [], []
    for s in range(n):
        st = {x: pre[s][x] for x in ("S", "P", "m", "R", "r")}
        nm, dn, _ = serial3_r(seg(q, s), seg(k, s), seg(v, s), gamma, st)
        nums.append(nm)
        dens.append(dn)
    total = combine3(pre[-1], sums[-1])
    return np.concatenate(nums, 1), np.concatenate(dens, 1), total
