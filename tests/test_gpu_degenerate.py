"""Degenerate inputs through the GPU path, checked against closed forms written here
(independent of the oracle) and against the FP64 oracle.

- beta = 0: nothing is written, the state only decays: S_T = S_0 Diag(exp(sum_t g_t)) and
  o_t = s S_0 Diag(exp(G_t)) q_t with G_t the prefix sum of g through token t.
- beta = 1, g = 0, S_0 = 0 and mutually orthonormal keys (one-hot, distinct): the delta
  rule is causal linear attention, o_t = s sum_{tau <= t} (k_tau . q_t) v_tau and
  S_T = sum_tau v_tau k_tau^T (every correction term S k_t vanishes).
- q = 0: every output is exactly zero (Qt and A_qk vanish), the state is unchanged.
- g = 0 with random beta: no decay at all, against the oracle.

Each runs in the serial form and in the segmented form (short segments, so that the
transition, the combine and the scan output all take part), at sizes with a ragged last
chunk. Bound: max|err| / max|ref| <= 2e-2 for o and the final state.
"""

import dataclasses

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2
FORMS = [dict(segment_chunks=-1), dict(segment_chunks=2)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def _bf16(a):
    """Round to BF16 values (round to nearest even), kept as float64."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _inputs(T, H, seed, **fields):
    x = kda_synth.config(1, T=T, H=H)
    rng = np.random.default_rng(seed)
    if "state0" not in fields:
        fields["state0"] = _bf16(0.1 * rng.standard_normal((1, H, 128, 128)))
    return dataclasses.replace(x, **{k: np.asarray(v, np.float32) if isinstance(v, np.ndarray)
                                     else v for k, v in fields.items()})


@pytest.mark.parametrize("form", FORMS, ids=["serial", "segmented"])
def test_zero_beta_is_pure_decay(form):
    T, H = 150, 2
    rng = np.random.default_rng(11)
    g = _bf16(-0.02 * rng.random((1, T, H, 128)))
    x = _inputs(T, H, 11, beta=np.zeros((1, T, H)), g=g)
    s = x.scale
    S0 = x.state0.astype(np.float64)[0]                      # [H, V, K]
    G = np.cumsum(x.g.astype(np.float64)[0], axis=0)         # [T, H, K]
    q = x.q.astype(np.float64)[0]                            # [T, H, K]
    o_ref = s * np.einsum("hvk,thk->thv", S0, np.exp(G) * q)[None]
    s_ref = (S0 * np.exp(G[-1])[:, None, :])[None]
    o, st, _ = run_gpu(x, **form)
    assert rel_err(o, o_ref) <= TOL and rel_err(st, s_ref) <= TOL
    o2, s2 = run_oracle(x)
    assert rel_err(o, o2) <= TOL and rel_err(st, s2) <= TOL


@pytest.mark.parametrize("form", FORMS, ids=["serial", "segmented"])
def test_orthonormal_keys_give_causal_linear_attention(form):
    T, H = 100, 2
    rng = np.random.default_rng(12)
    k = np.zeros((1, T, H, 128))
    for h in range(H):
        k[0, np.arange(T), h, rng.permutation(128)[:T]] = 1.0
    x = _inputs(T, H, 12, k=k, g=np.zeros((1, T, H, 128)), beta=np.ones((1, T, H)),
                state0=None)
    q = x.q.astype(np.float64)[0]
    v = x.v.astype(np.float64)[0]
    kk = k[0]
    scores = np.einsum("shk,thk->hts", kk, q)                # k_s . q_t
    scores = scores * np.tril(np.ones((T, T)))[None]
    o_ref = x.scale * np.einsum("hts,shv->thv", scores, v)[None]
    s_ref = np.einsum("thv,thk->hvk", v, kk)[None]
    o, st, _ = run_gpu(x, **form)
    assert rel_err(o, o_ref) <= TOL and rel_err(st, s_ref) <= TOL


@pytest.mark.parametrize("form", FORMS, ids=["serial", "segmented"])
def test_zero_queries_give_zero_outputs(form):
    T, H = 70, 3
    x = _inputs(T, H, 13, q=np.zeros((1, T, H, 128)))
    o, st, _ = run_gpu(x, **form)
    assert np.all(o == 0.0)
    _, s2 = run_oracle(x)
    assert rel_err(st, s2) <= TOL


@pytest.mark.parametrize("form", FORMS, ids=["serial", "segmented"])
def test_zero_decay_with_random_beta(form):
    T, H = 90, 2
    x = _inputs(T, H, 14, g=np.zeros((1, 90, 2, 128)))
    o, st, _ = run_gpu(x, **form)
    o2, s2 = run_oracle(x)
    assert rel_err(o, o2) <= TOL and rel_err(st, s2) <= TOL
