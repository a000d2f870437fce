"""In-kernel input transforms of KDA prefill, in FP64 (oracle side).

The "flashinfer.kda_prefill" API page, section "Optimized Blackwell prefill subset"
and "SM120a prefill subset", names three optional in-kernel transforms:
``use_qk_l2norm_in_kernel``, ``beta_is_logit`` and the in-kernel lower-bound gate
(``use_gate_in_kernel`` with ``A_log[H]``, ``dt_bias[H,128]`` and ``lower_bound`` in
[-5, 0)). The page gives their inputs but not their formulas; the readings below are
the plainest ones consistent with the pages, each stated with its function below.
"""

import numpy as np

# Reading: the L2 norm adds a small epsilon inside the square root. The pages do not
# state it; for 128-channel inputs its effect is far below every tolerance used here.
L2_EPS = 1e-6


def l2_normalize(x, eps=L2_EPS):
    """Normalise the last axis: x / sqrt(sum(x^2) + eps), in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    """Logistic function 1 / (1 + exp(-x)), in float64.

    The FlashKDA column-split post (section 3.4) notes FlashKDA evaluates it as
    1/2 + 1/2 tanh(x/2); the two are the same function (a test pins that).
    """
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def safe_gate(g_raw, A_log, dt_bias, lower_bound):
    """Lower-bounded per-channel log-decay computed from raw gate inputs.

    g = lower_bound * sigmoid(exp(A_log[h]) * (g_raw + dt_bias[h, c]))

    g_raw: [..., H, D]; A_log: [H]; dt_bias: [H, D] (or [H*D]); lower_bound < 0.

    The result lies in (lower_bound, 0), the range the K3 decay page motivates
    (section "Why a diagonal tile needs lower-bounded decay"). The formula itself is not
    printed on any page: parity unpinned against the pages. Tests pin only its range and
    that A_log = 0, dt_bias = 0 reduces it to lower_bound * sigmoid(g_raw), the
    "model_like" log-decay of the K3 decay page's experiment.
    """
    g_raw = np.asarray(g_raw, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    H = A_log.shape[0]
    dt_bias = np.asarray(dt_bias, dtype=np.float64).reshape(H, -1)
    a = np.exp(A_log)[:, None]  # [H, 1]
    return float(lower_bound) * sigmoid(a * (g_raw + dt_bias))
