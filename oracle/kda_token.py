"""The definition: KDA token-by-token recurrence in FP64.

For one head, with state S (values x keys, V x K), per-channel log-decay g_t, write
strength beta_t, key k_t, value v_t and query q_t:

    S'   = S_{t-1} Diag(exp g_t)                 decay every key channel
    u_t  = beta_t (v_t - S' k_t)                 delta-rule error of the prediction
    S_t  = S' + u_t k_t^T                        write
    o_t  = s S_t q_t                             read with the updated state

The pages print this only in chunk form: the "FlashKDA column split" post, section 1
"FlashKDA in two kernels", defines the chunk quantities and the three chunk equations
(U, O, S_{c+1}) and defers the token form to another post that is not among the pages.
The token form above is the one those chunk equations reduce to at chunk length 1, and
the chunk equations at length 16 are exactly its unrolling; ``tests/test_oracle_pins.py``
checks both directions against ``oracle.kda_chunk`` (which follows the page's
definitions literally). State layout [N, H, V, K] and the in-place / varlen contract
follow the "flashinfer.kda_prefill" page, sections "State and graph semantics" and
"Optimized Blackwell prefill subset".
"""

import numpy as np

from .transforms import l2_normalize, safe_gate, sigmoid


def token_step(S, k, v, g, beta):
    """One token for one head. S: [V, K]; k, g: [K]; v: [V]; beta scalar. Returns S_t."""
    S_dec = S * np.exp(g)[None, :]
    u = beta * (v - S_dec @ k)
    return S_dec + np.outer(u, k)


def _as64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def kda_recurrence_fp64(
    q,
    k,
    v,
    g,
    beta,
    state0=None,
    cu_seqlens=None,
    scale=None,
    *,
    l2norm_qk=False,
    beta_is_logit=False,
    A_log=None,
    dt_bias=None,
    lower_bound=None,
    heads=None,
    checkpoint_every=None,
):
    """Run the recurrence over every sequence and head, in float64.

    q, k, g: [B, T, H, K]; v: [B, T, H, V]; beta: [B, T, H]  (any float dtype; the values
    are taken exactly as given, so BF16 inputs are not counted as error).
    state0: [N, H, V, K] or None (zeros).
    cu_seqlens: None (fixed layout, N = B) or int [N+1] with B = 1 (packed varlen).
    scale: output scale s (default 1/sqrt(K)).
    Flags as on the flashinfer.kda_prefill page: l2norm_qk normalises q and k per
    (token, head); beta_is_logit applies the logistic to beta; A_log / dt_bias /
    lower_bound (all given) turn g into the lower-bounded gate of ``safe_gate``.
    heads: optional list of head indices; only those heads are computed and returned.
    checkpoint_every: optional interval I (tokens). Following the checkpoint contract of
    the "flashinfer.kda_prefill" page (section "State and graph semantics"), every
    non-empty sequence then contributes the states before each interval: its initial
    state, then the states after I, 2I, ... tokens that come strictly before its end,
    i.e. ceil(len / I) rows, stacked in sequence order (``checkpoint_starts`` gives the
    row offsets).

    Returns (o [B, T, H', V] float64, state [N, H', V, K] float64), and with
    checkpoint_every also checkpoints [C, H', V, K] float64.
    """
    q, k, v, g, beta = (_as64(x) for x in (q, k, v, g, beta))
    B, T, H, K = k.shape
    V = v.shape[-1]
    heads = list(range(H)) if heads is None else list(heads)
    hs = np.asarray(heads)
    q, k, v, g, beta = q[:, :, hs], k[:, :, hs], v[:, :, hs], g[:, :, hs], beta[:, :, hs]
    Hs = len(heads)
    if scale is None:
        scale = 1.0 / np.sqrt(K)

    if l2norm_qk:
        q = l2_normalize(q)
        k = l2_normalize(k)
    if beta_is_logit:
        beta = sigmoid(beta)
    if A_log is not None:
        A_log = _as64(A_log)
        dt = _as64(dt_bias).reshape(H, -1)
        g = safe_gate(g, A_log[hs], dt[hs], lower_bound)

    # Flatten batch into one token axis; sequences are [start, end) ranges of it.
    q, k, v, g, beta = (x.reshape((B * T,) + x.shape[2:]) for x in (q, k, v, g, beta))
    if cu_seqlens is None:
        bounds = [(b * T, (b + 1) * T) for b in range(B)]
    else:
        cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
        bounds = list(zip(cu[:-1], cu[1:]))
    N = len(bounds)

    o = np.zeros((B * T, Hs, V), dtype=np.float64)
    states = np.zeros((N, Hs, V, K), dtype=np.float64)
    ckpts = []
    for n, (start, end) in enumerate(bounds):
        if state0 is None:
            S = np.zeros((Hs, V, K), dtype=np.float64)
        else:
            S = np.array(_as64(state0)[n][hs], dtype=np.float64)
        for t in range(start, end):
            if checkpoint_every is not None and (t - start) % checkpoint_every == 0:
                ckpts.append(S.copy())  # the state before this interval
            # token_step for all heads at once: S Diag(alpha), delta-rule write, read.
            S = S * np.exp(g[t])[:, None, :]
            pred = np.matmul(S, k[t][:, :, None])[:, :, 0]
            u = beta[t][:, None] * (v[t] - pred)
            S = S + u[:, :, None] * k[t][:, None, :]
            o[t] = scale * np.matmul(S, q[t][:, :, None])[:, :, 0]
        states[n] = S
    if checkpoint_every is not None:
        C = np.stack(ckpts) if ckpts else np.zeros((0, Hs, V, K), dtype=np.float64)
        return o.reshape(B, T, Hs, V), states, C
    return o.reshape(B, T, Hs, V), states


def checkpoint_starts(lengths, interval):
    """Row offsets [N + 1] of each sequence's checkpoints: ceil(len / interval) rows per
    sequence (none for an empty one), as on the "flashinfer.kda_prefill" page."""
    counts = [(int(n) + interval - 1) // interval for n in lengths]
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
