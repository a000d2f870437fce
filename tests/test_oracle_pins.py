"""Pins of the FP64 oracle against what the pages and mathematics fix (CPU only).

Each test ties ``oracle`` to something other than itself: the pages' chunk equations
(a different algorithm), the K3 decay page's split-exponent form, closed forms of
special cases, a textbook reduction (causal linear attention), the delta rule's
defining property, a finite-difference gradient of the delta-rule loss, and
structural identities. ``test_planted_mistakes_are_caught`` shows that plausible
mistakes in a token recurrence fail these pins.
"""

import numpy as np
import pytest

from oracle import (
    checkpoint_starts,
    chunk_quantities,
    chunkwise_forward,
    inverse_explicit,
    inverse_forward_substitution,
    inverse_neumann,
    kda_recurrence_fp64,
    l2_normalize,
    safe_gate,
    sigmoid,
    token_step,
)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_inputs(rng, B, T, H, Dk, Dv=None, g_lo=-5.0, state=True, unit_k=True):
    Dv = Dk if Dv is None else Dv
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = g_lo * rng.uniform(0.0, 1.0, (B, T, H, Dk))
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    S0 = rng.standard_normal((B, H, Dv, Dk)) if state else None
    return q, k, v, g, beta, S0


# ---------------------------------------------------------------------------------
# 1. The pages' chunk equations reproduce the token definition (both directions).
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [1, 2, 4, 16])
@pytest.mark.parametrize("inverse", ["forward", "explicit", "neumann"])
def test_chunkwise_equations_match_token_recurrence(chunk, inverse):
    rng = np.random.default_rng(10 + chunk)
    T, Dk, Dv = 37, 16, 12  # ragged tail; V != K catches transposed operands
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, T, 1, Dk, Dv)
    s = 0.37
    o_ref, S_ref = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=s)
    o_c, S_c = chunkwise_forward(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                 beta[0, :, 0], S0[0, 0], s, chunk=chunk, inverse=inverse)
    assert rel_err(o_c, o_ref[0, :, 0]) < 1e-12
    assert rel_err(S_c, S_ref[0, 0]) < 1e-12


def test_chunkwise_full_width_config_like():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 48, 1, 128)
    s = 128 ** -0.5
    o_ref, S_ref = kda_recurrence_fp64(q, k, v, g, beta, S0)
    o_c, S_c = chunkwise_forward(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                 beta[0, :, 0], S0[0, 0], s, chunk=16)
    assert rel_err(o_c, o_ref[0, :, 0]) < 1e-12
    assert rel_err(S_c, S_ref[0, 0]) < 1e-12


# ---------------------------------------------------------------------------------
# 2. Three independent inverses of (I + R) agree and invert.
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_three_inverses_agree(seed):
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, _ = rand_inputs(rng, 1, 16, 1, 32, g_lo=-0.2)
    w = chunk_quantities(q[0, :, 0], k[0, :, 0], g[0, :, 0], beta[0, :, 0], 0.5)
    R = w["R"]
    assert np.all(np.triu(R) == 0.0)
    Xe, Xf, Xn = inverse_explicit(R), inverse_forward_substitution(R), inverse_neumann(R)
    assert rel_err(Xf, Xe) < 1e-13
    assert rel_err(Xn, Xe) < 1e-13
    assert rel_err((np.eye(16) + R) @ Xf, np.eye(16)) < 1e-13


def test_neumann_is_exact_for_any_strictly_lower_matrix():
    rng = np.random.default_rng(7)
    for C in (2, 3, 5, 8, 16, 17, 31):
        L = np.tril(rng.standard_normal((C, C)) * 0.3, -1)
        assert rel_err(inverse_neumann(L), np.linalg.inv(np.eye(C) + L)) < 1e-12


# ---------------------------------------------------------------------------------
# 3. The K3 decay page's split-exponent form of the decayed products.
# ---------------------------------------------------------------------------------
def test_split_exponent_form_per_channel_and_scalar():
    rng = np.random.default_rng(5)
    C, Dk = 16, 24
    q, k, _, g, beta, _ = rand_inputs(rng, 1, C, 1, Dk)
    q, k, g, beta = q[0, :, 0], k[0, :, 0], g[0, :, 0], beta[0, :, 0]
    s = 0.3
    w = chunk_quantities(q, k, g, beta, s)
    G = np.cumsum(g, axis=0)  # inclusive prefix: G_i = g_0 + ... + g_i
    Gam = np.exp(G)
    # Per channel: A = Tril[(Gamma . Q)(K / Gamma)^T]
    A = (Gam * q) @ (k / Gam).T
    Rk = (Gam * k) @ (k / Gam).T
    assert rel_err(w["A_qk"], s * np.tril(A)) < 1e-12
    assert rel_err(w["R"], beta[:, None] * np.tril(Rk, -1)) < 1e-12
    # Workspace vectors in the same prefix notation.
    assert rel_err(w["K_start"], (Gam * k).T) < 1e-13
    assert rel_err(w["Q_start"], (Gam * q).T) < 1e-13
    assert rel_err(w["K_end"], k * np.exp(G[-1] - G)) < 1e-13
    assert rel_err(w["D_total"], np.exp(G[-1])) < 1e-13
    # Scalar decay: beta_i (k_i . k_j) exp(G_i - G_j) for j < i.
    gs = -rng.uniform(0, 5, C)
    w2 = chunk_quantities(q, k, np.repeat(gs[:, None], Dk, 1), beta, s)
    Gs = np.cumsum(gs)
    Rs = np.tril(beta[:, None] * (k @ k.T) * np.exp(Gs[:, None] - Gs[None, :]), -1)
    assert rel_err(w2["R"], Rs) < 1e-12


# ---------------------------------------------------------------------------------
# 4. Closed forms and textbook special cases.
# ---------------------------------------------------------------------------------
def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(11)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 20, 2, 8)
    beta[:] = 0.0
    s = 0.25
    o, S = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=s)
    G = np.cumsum(g[0], axis=0)  # [T, H, K]
    for h in range(2):
        assert rel_err(S[0, h], S0[0, h] * np.exp(G[-1, h])[None, :]) < 1e-13
        o_cf = s * np.stack([(S0[0, h] * np.exp(G[t, h])[None, :]) @ q[0, t, h]
                             for t in range(20)])
        assert rel_err(o[0, :, h], o_cf) < 1e-13


def test_beta_zero_no_decay_is_linear_readout():
    rng = np.random.default_rng(12)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 9, 3, 8)
    beta[:] = 0.0
    g[:] = 0.0
    o, S = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=0.5)
    expect = 0.5 * np.einsum("hvk,thk->thv", S0[0], q[0])
    assert rel_err(o[0], expect) < 1e-14
    assert rel_err(S, S0) == 0.0


def test_orthonormal_keys_reduce_to_causal_linear_attention():
    rng = np.random.default_rng(13)
    T, Dk, Dv = 10, 16, 6
    perm = rng.permutation(Dk)[:T]
    k = np.eye(Dk)[perm][None, :, None, :]  # k_t = e_{pi(t)}, mutually orthonormal
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    g = np.zeros((1, T, 1, Dk))
    beta = np.ones((1, T, 1))
    s = 0.7
    o, _ = kda_recurrence_fp64(q, k, v, g, beta, None, scale=s)
    Q, K, V = q[0, :, 0], k[0, :, 0], v[0, :, 0]
    expect = s * (np.tril(Q @ K.T) @ V)
    assert rel_err(o[0, :, 0], expect) < 1e-14


def test_delta_rule_stores_value_exactly_for_unit_key_and_beta_one():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 7, 2, 8)
    beta[:] = 1.0
    for t in range(1, 8):
        _, S = kda_recurrence_fp64(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t],
                                   S0, scale=1.0)
        for h in range(2):
            assert rel_err(S[0, h] @ k[0, t - 1, h], v[0, t - 1, h]) < 1e-13


def test_update_is_one_gradient_step_on_the_delta_rule_loss():
    # S_t = S' - beta * grad_S 0.5 * ||S k - v||^2 at S' = S_{t-1} Diag(exp g):
    # the gradient is taken by central differences (exact for a quadratic).
    rng = np.random.default_rng(15)
    Dk, Dv = 3, 2
    S = rng.standard_normal((Dv, Dk))
    k = rng.standard_normal(Dk)
    v = rng.standard_normal(Dv)
    g = -rng.uniform(0, 2, Dk)
    beta = 0.6
    Sd = S * np.exp(g)[None, :]
    loss = lambda X: 0.5 * np.sum((X @ k - v) ** 2)
    grad = np.zeros_like(Sd)
    h = 1e-3
    for i in range(Dv):
        for j in range(Dk):
            E = np.zeros_like(Sd)
            E[i, j] = h
            grad[i, j] = (loss(Sd + E) - loss(Sd - E)) / (2 * h)
    assert rel_err(token_step(S, k, v, g, beta), Sd - beta * grad) < 1e-9


def test_linearity_in_values_and_initial_state():
    rng = np.random.default_rng(16)
    q, k, v1, g, beta, S1 = rand_inputs(rng, 1, 21, 2, 8)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    a, b = 0.7, -1.3
    o1, s1 = kda_recurrence_fp64(q, k, v1, g, beta, S1, scale=1.0)
    o2, s2 = kda_recurrence_fp64(q, k, v2, g, beta, S2, scale=1.0)
    o3, s3 = kda_recurrence_fp64(q, k, a * v1 + b * v2, g, beta, a * S1 + b * S2, scale=1.0)
    assert rel_err(o3, a * o1 + b * o2) < 1e-12
    assert rel_err(s3, a * s1 + b * s2) < 1e-12


def test_outputs_are_affine_in_the_start_state():
    # With V = 0 and the identity as start state (Dk x Dk), the recurrence carries the
    # product Phi_t of the token transitions, and its output at token t is s Phi_t q_t.
    # For any start state S0: o_t(S0) = o_t(0) + S0 (s Phi_t q_t) and
    # S_T(S0) = S0 Phi_T + S_T(0). This is the decomposition the GPU's segmented form
    # evaluates (zero-start run, transition run, then the start state applied to both).
    rng = np.random.default_rng(18)
    Dk, Dv, T = 8, 6, 23
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, T, 2, Dk, Dv=Dv, g_lo=-0.3)
    o, S = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=0.7)
    oz, Sz = kda_recurrence_fp64(q, k, v, g, beta, None, scale=0.7)
    eye = np.broadcast_to(np.eye(Dk), (1, 2, Dk, Dk)).copy()
    ophi, Phi = kda_recurrence_fp64(q, k, np.zeros((1, T, 2, Dk)), g, beta, eye, scale=0.7)
    assert rel_err(o, oz + np.einsum("bhvr,bthr->bthv", S0, ophi)) < 1e-12
    assert rel_err(S, Sz + np.einsum("bhvr,bhrk->bhvk", S0, Phi)) < 1e-12
    # The carry matters here: the start state changes the outputs at the last token.
    assert rel_err(o[:, -1], oz[:, -1]) > 1e-2


def test_channel_permutation_equivariance():
    rng = np.random.default_rng(17)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 19, 2, 8)
    o, S = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=1.0)
    pv = rng.permutation(8)
    pk = rng.permutation(8)
    o2, S2 = kda_recurrence_fp64(q[..., pk], k[..., pk], v[..., pv], g[..., pk], beta,
                                 S0[:, :, pv][:, :, :, pk], scale=1.0)
    assert rel_err(o2, o[..., pv]) < 1e-13
    assert rel_err(S2, S[:, :, pv][:, :, :, pk]) < 1e-13


def test_varlen_equals_separate_sequences_and_fixed_batch():
    rng = np.random.default_rng(18)
    lens = [5, 0, 17, 1, 33]
    T = sum(lens)
    q, k, v, g, beta, _ = rand_inputs(rng, 1, T, 2, 8, state=False)
    S0 = rng.standard_normal((len(lens), 2, 8, 8))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = kda_recurrence_fp64(q, k, v, g, beta, S0, cu_seqlens=cu, scale=1.0)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        on, Sn = kda_recurrence_fp64(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b],
                                     beta[:, a:b], S0[n:n + 1], scale=1.0)
        assert np.array_equal(o[:, a:b], on)
        assert np.array_equal(S[n], Sn[0])
    assert np.array_equal(S[1], S0[1])  # zero-length sequence passes its state through
    # Fixed layout B = 3 equals packed varlen with equal lengths.
    qb, kb, vb, gb, bb, Sb = rand_inputs(rng, 3, 12, 2, 8)
    ob, Sfb = kda_recurrence_fp64(qb, kb, vb, gb, bb, Sb, scale=1.0)
    flat = lambda x: x.reshape((1, 36) + x.shape[2:])
    ov, Sv = kda_recurrence_fp64(flat(qb), flat(kb), flat(vb), flat(gb), flat(bb), Sb,
                                 cu_seqlens=[0, 12, 24, 36], scale=1.0)
    assert np.array_equal(ov.reshape(ob.shape), ob)
    assert np.array_equal(Sv, Sfb)


def test_split_prefill_equals_one_call():
    rng = np.random.default_rng(19)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 40, 2, 8)
    o, S = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=1.0)
    oa, Sa = kda_recurrence_fp64(q[:, :13], k[:, :13], v[:, :13], g[:, :13],
                                 beta[:, :13], S0, scale=1.0)
    ob, Sb = kda_recurrence_fp64(q[:, 13:], k[:, 13:], v[:, 13:], g[:, 13:],
                                 beta[:, 13:], Sa, scale=1.0)
    assert rel_err(np.concatenate([oa, ob], 1), o) < 1e-13
    assert rel_err(Sb, S) < 1e-13


@pytest.mark.parametrize("interval", [16, 32, 7])
def test_checkpoints_are_states_before_each_interval(interval):
    # The flashinfer page's checkpoint contract ("State and graph semantics"): each
    # non-empty sequence contributes its initial state, then the states after 1, 2, ...
    # intervals that come strictly before its end: ceil(len / I) rows.
    rng = np.random.default_rng(20)
    lens = [0, 5, 16, 17, 40]
    T = sum(lens)
    q, k, v, g, beta, _ = rand_inputs(rng, 1, T, 2, 8, state=False)
    S0 = rng.standard_normal((len(lens), 2, 8, 8))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S, C = kda_recurrence_fp64(q, k, v, g, beta, S0, cu_seqlens=cu, scale=1.0,
                                  checkpoint_every=interval)
    o2, S2 = kda_recurrence_fp64(q, k, v, g, beta, S0, cu_seqlens=cu, scale=1.0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    starts = checkpoint_starts(lens, interval)
    assert C.shape[0] == starts[-1] == sum(-(-n // interval) for n in lens)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        rows = C[starts[n]:starts[n + 1]]
        assert len(rows) == -(-(b - a) // interval)
        for r, row in enumerate(rows):
            if r == 0:
                assert np.array_equal(row, S0[n])
                continue
            e = a + r * interval  # state after the first r intervals of the sequence
            _, Sr = kda_recurrence_fp64(q[:, a:e], k[:, a:e], v[:, a:e], g[:, a:e],
                                        beta[:, a:e], S0[n:n + 1], scale=1.0)
            assert np.array_equal(row, Sr[0])


def test_checkpoints_closed_form_without_writes():
    # beta = 0: checkpoint r is S0 decayed by the first r intervals' total decay.
    rng = np.random.default_rng(21)
    q, k, v, g, _, S0 = rand_inputs(rng, 1, 50, 2, 8)
    beta = np.zeros((1, 50, 2))
    _, _, C = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=1.0, checkpoint_every=16)
    assert C.shape[0] == 4
    for r in range(4):
        decay = np.exp(g[0, :16 * r].sum(axis=0))  # [H, K]
        assert rel_err(C[r], S0[0] * decay[:, None, :]) < 1e-13


# ---------------------------------------------------------------------------------
# 5. Transforms.
# ---------------------------------------------------------------------------------
def test_sigmoid_equals_tanh_form():
    x = np.linspace(-30, 30, 1001)
    assert rel_err(sigmoid(x), 0.5 + 0.5 * np.tanh(0.5 * x)) < 1e-15


def test_l2_normalize_gives_unit_rows():
    rng = np.random.default_rng(20)
    x = rng.standard_normal((5, 3, 128))
    n = np.linalg.norm(l2_normalize(x), axis=-1)
    assert np.max(np.abs(n - 1.0)) < 1e-7


def test_safe_gate_range_and_special_case():
    rng = np.random.default_rng(21)
    H = 4
    x = rng.standard_normal((2, 9, H, 128)) * 4
    A_log = rng.uniform(-1, 1, H)
    dt = 0.1 * rng.standard_normal((H, 128))
    for lb in (-5.0, -0.1):
        gg = safe_gate(x, A_log, dt, lb)
        assert np.all(gg < 0) and np.all(gg > lb)
    gg0 = safe_gate(x, np.zeros(H), np.zeros((H, 128)), -5.0)
    assert rel_err(gg0, -5.0 * sigmoid(x)) < 1e-15
    flat = safe_gate(x, A_log, dt.reshape(-1), -5.0)
    assert np.array_equal(flat, safe_gate(x, A_log, dt, -5.0))


def test_flags_compose_as_preprocessing():
    rng = np.random.default_rng(22)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 11, 2, 128, unit_k=False)
    A_log = rng.uniform(-1, 1, 2)
    dt = 0.1 * rng.standard_normal((2, 128))
    o, S = kda_recurrence_fp64(q, k, v, g, beta, S0, l2norm_qk=True, beta_is_logit=True,
                               A_log=A_log, dt_bias=dt, lower_bound=-5.0)
    o2, S2 = kda_recurrence_fp64(l2_normalize(q), l2_normalize(k), v,
                                 safe_gate(g, A_log, dt, -5.0), sigmoid(beta), S0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


def test_head_sampling_matches_full_run():
    rng = np.random.default_rng(23)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 9, 5, 8)
    o, S = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=1.0)
    o2, S2 = kda_recurrence_fp64(q, k, v, g, beta, S0, scale=1.0, heads=[3, 1])
    assert np.array_equal(o2, o[:, :, [3, 1]]) and np.array_equal(S2, S[:, [3, 1]])


# ---------------------------------------------------------------------------------
# 6. Plausible mistakes in a token recurrence fail the chunk-equation pin.
# ---------------------------------------------------------------------------------
def _mutant_run(step, q, k, v, g, beta, S0, s):
    S = S0.copy()
    o = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        S, o[t] = step(S, q[t], k[t], v[t], g[t], beta[t], s)
    return o, S


def _m_pred_before_decay(S, q, k, v, g, b, s):
    u = b * (v - S @ k)
    S = S * np.exp(g)[None, :] + np.outer(u, k)
    return S, s * S @ q


def _m_read_before_write(S, q, k, v, g, b, s):
    Sd = S * np.exp(g)[None, :]
    o = s * Sd @ q
    return Sd + np.outer(b * (v - Sd @ k), k), o


def _m_wrong_sign(S, q, k, v, g, b, s):
    Sd = S * np.exp(g)[None, :]
    S = Sd + np.outer(b * (v + Sd @ k), k)
    return S, s * S @ q


def _m_decay_after_write(S, q, k, v, g, b, s):
    S = (S + np.outer(b * (v - S @ k), k)) * np.exp(g)[None, :]
    return S, s * S @ q


def _m_transposed_state(S, q, k, v, g, b, s):
    Sd = S * np.exp(g)[:, None]
    S = Sd + np.outer(b * (v - Sd.T @ k), k).T
    return S, s * S.T @ q


@pytest.mark.parametrize("mutant", [_m_pred_before_decay, _m_read_before_write,
                                    _m_wrong_sign, _m_decay_after_write,
                                    _m_transposed_state])
def test_planted_mistakes_are_caught(mutant):
    rng = np.random.default_rng(24)
    q, k, v, g, beta, S0 = rand_inputs(rng, 1, 20, 1, 8, g_lo=-1.0)
    args = (q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0])
    o_c, S_c = chunkwise_forward(*args, S0[0, 0], 0.5, chunk=16)
    o_m, S_m = _mutant_run(mutant, *args, S0[0, 0], 0.5)
    assert max(rel_err(o_m, o_c), rel_err(S_m, S_c)) > 1e-3
