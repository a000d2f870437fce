"""The pages' chunk equations, written literally, in FP64 (a cross-check of the token
definition and the reference for the per-chunk quantities a preparation step builds).

"FlashKDA column split" post, section 1 "FlashKDA in two kernels". For a chunk of C
tokens i = 0..C-1 of one head, with D_i = Diag(exp g_i) and D_{a:b} = D_a D_{a+1} ... D_b
(the empty product is I):

    K_start  column i = D_{0:i} k_i            Q_start column i = D_{0:i} q_i
    K_end    row i    = k_i^T D_{i+1:C-1}       D_total = D_{0:C-1}
    R_ij  = beta_i <k_j| D_{j+1:i} |k_i>   for j < i   (0 otherwise)
    A_kk  = (I + R)^{-1}
    A_qk_ij = s <k_j| D_{j+1:i} |q_i>      for j <= i  (0 otherwise)

and with the chunk's values as the columns of V_c and B_c = Diag(beta):

    U_c     = (V_c - S_c K_start) B_c A_kk^T
    O_c     = s S_c Q_start + U_c A_qk^T
    S_{c+1} = S_c D_total + U_c K_end

Inverses of (I + R): ``inverse_explicit`` (numpy.linalg.inv), ``inverse_forward_substitution``
(row-by-row solve of a unit lower-triangular system) and ``inverse_neumann`` — the
repeated-squaring Neumann product (I - R)(I + R^2)(I + R^4)(I + R^8) of the K3 decay page,
section "Matrix inversion in FlashKDA", exact because a strictly lower-triangular R is
nilpotent.
"""

import numpy as np


def _decay(g, a, b):
    """Per-channel diagonal of D_{a:b} = D_a ... D_b (inclusive); identity if b < a."""
    D = g.shape[1]
    out = np.ones(D, dtype=np.float64)
    for t in range(a, b + 1):
        out = out * np.exp(g[t])
    return out


def inverse_explicit(R):
    """(I + R)^{-1} by a library dense inverse."""
    C = R.shape[0]
    return np.linalg.inv(np.eye(C) + R)


def inverse_forward_substitution(R):
    """(I + R)^{-1} for strictly lower-triangular R: row i of X solves
    X_i = e_i - sum_{j<i} R_ij X_j (unit diagonal, lower triangular)."""
    C = R.shape[0]
    X = np.zeros((C, C), dtype=np.float64)
    for i in range(C):
        row = np.zeros(C, dtype=np.float64)
        row[i] = 1.0
        for j in range(i):
            row = row - R[i, j] * X[j]
        X[i] = row
    return X


def inverse_neumann(R, return_powers=False):
    """(I + R)^{-1} = (I - R)(I + R^2)(I + R^4)... up to the largest power 2^m < C.

    With return_powers, also returns (highest power formed, max |entry| over R and every
    power formed), the two statistics the K3 decay page tabulates for its stress input.
    """
    C = R.shape[0]
    I = np.eye(C)
    result = I - R
    power = R
    exponent = 1
    max_mag = float(np.max(np.abs(R))) if R.size else 0.0
    while 2 * exponent < C:
        power = power @ power
        exponent *= 2
        max_mag = max(max_mag, float(np.max(np.abs(power))))
        result = result @ (I + power)
    if return_powers:
        return result, exponent, max_mag
    return result


_INVERSES = {
    "explicit": inverse_explicit,
    "forward": inverse_forward_substitution,
    "neumann": inverse_neumann,
}


def chunk_quantities(q, k, g, beta, scale, inverse="forward"):
    """Per-chunk workspace quantities of one head.

    q, k, g: [C, D] (token x channel); beta: [C]. Returns a dict with
    K_start [D, C], Q_start [D, C], K_end [C, D], D_total [D], R [C, C], A_kk [C, C],
    A_qk [C, C] (A_qk includes the scale s, as on the page).
    """
    q, k, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, g, beta))
    C, D = k.shape
    K_start = np.zeros((D, C))
    Q_start = np.zeros((D, C))
    K_end = np.zeros((C, D))
    for i in range(C):
        K_start[:, i] = _decay(g, 0, i) * k[i]
        Q_start[:, i] = _decay(g, 0, i) * q[i]
        K_end[i, :] = k[i] * _decay(g, i + 1, C - 1)
    D_total = _decay(g, 0, C - 1)
    R = np.zeros((C, C))
    A_qk = np.zeros((C, C))
    for i in range(C):
        for j in range(C):
            between = _decay(g, j + 1, i)
            if j < i:
                R[i, j] = beta[i] * np.sum(k[j] * between * k[i])
            if j <= i:
                A_qk[i, j] = scale * np.sum(k[j] * between * q[i])
    A_kk = _INVERSES[inverse](R)
    return dict(K_start=K_start, Q_start=Q_start, K_end=K_end, D_total=D_total,
                R=R, A_kk=A_kk, A_qk=A_qk)


def chunkwise_forward(q, k, v, g, beta, state0, scale, chunk=16, inverse="forward"):
    """One sequence of one head through the chunk equations.

    q, k, g: [T, K]; v: [T, V]; beta: [T]; state0: [V, K] or None.
    The last chunk may be shorter than ``chunk``; the equations hold for any length.
    Returns (o [T, V], final state [V, K]).
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, K = k.shape
    Vd = v.shape[1]
    S = np.zeros((Vd, K)) if state0 is None else np.array(state0, dtype=np.float64)
    o = np.zeros((T, Vd))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        w = chunk_quantities(q[sl], k[sl], g[sl], beta[sl], scale, inverse)
        Vc = v[sl].T
        Bc = np.diag(beta[sl])
        U = (Vc - S @ w["K_start"]) @ Bc @ w["A_kk"].T
        O = scale * S @ w["Q_start"] + U @ w["A_qk"].T
        S = S @ np.diag(w["D_total"]) + U @ w["K_end"]
        o[sl] = O.T
    return o, S
