"""Seeded synthetic inputs for KDA prefill: the only module both the oracle side and the
HIP side are fed from. It draws random numbers and rounds them to the storage dtype; it
holds none of the method's arithmetic.

Workload recipes (the five benchmark configurations; d_k = d_v = 128, chunk 16):

* ``config(0)``: B=1, H=1, T=256, FP32. q, k ~ N(0,1) then scaled to unit L2 norm per
  (token, head); v ~ N(0,1); beta = logistic(N(0,1)); per-channel log-decay
  g = -5 * logistic(N(0,1)), in (-5, 0); zero initial state; s = 1/sqrt(128).
* ``config(1)``: B=1, H=6, T=8192, BF16, drawn as config 0; zero BF16 initial state.
* ``config(2)``: H=12, as config 1 with initial state 0.02 * N(0,1) (BF16).
* ``config(3)``: H=96, as config 1.
* ``config(4)``: packed varlen, B=1, N=8 sequences with lengths integers(512, 4096)
  inclusive, H=24, BF16. q, k, v ~ N(0,1) raw (normalised in-kernel); raw gate
  g_raw ~ N(0,1); A_log ~ U(-1, 1) FP32 [H]; dt_bias ~ 0.1 N(0,1) FP32 [H,128];
  lower_bound -5; beta logits ~ N(0,1); per-sequence initial state 0.02 * N(0,1).

Every draw uses ``numpy.random.default_rng(seed)`` in float64 in the fixed order
(lengths,) q, k, v, g, beta, state (, A_log, dt_bias); values are then rounded to the
storage dtype (round-to-nearest-even for BF16) and returned as float32 arrays whose
values are exactly representable in that dtype, so both sides receive identical numbers.

Stress families (the K3 decay page, section "Numerical experiments on H200", generalised
to per-channel decay): ``weak_decay`` (g = -0.05 * logistic(N(0,1)), initial state
N(0,1)), ``correlated`` (one shared unit key, g = -0.01, beta = 0.5), ``floor``
(g = -5 everywhere), ``gate_weak`` (config 4's raw-gate recipe with lower_bound -0.1) and
``weak_carry`` (g = -gscale * logistic(N(0,1)), beta = bscale * logistic(N(0,1)),
initial state 0.1 * N(0,1); small enough decay and write strength that the transition
over hundreds of tokens stays of order 0.1-0.5, so that a time segment's start state
visibly shapes every later output of the segment).
"""

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

D = 128


def round_bf16(x):
    """Round to the nearest BF16 value (ties to even); returns float32 values."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def _store(x, dtype):
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _logistic(x):
    return 1.0 / (1.0 + np.exp(-x))


@dataclass
class KdaInputs:
    """One synthetic call. Arrays are float32 holding values exact in ``dtype``."""

    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state0: Optional[np.ndarray] = None
    cu_seqlens: Optional[np.ndarray] = None
    A_log: Optional[np.ndarray] = None
    dt_bias: Optional[np.ndarray] = None
    lower_bound: Optional[float] = None
    l2norm_qk: bool = False
    beta_is_logit: bool = False
    dtype: str = "bf16"
    state_dtype: str = "bf16"
    scale: float = 1.0 / np.sqrt(D)
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.q.shape[2]

    @property
    def N(self):
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def oracle_kwargs(self):
        """Keyword arguments for the oracle's recurrence (the same values the GPU gets)."""
        return dict(
            state0=self.state0, cu_seqlens=self.cu_seqlens, scale=self.scale,
            l2norm_qk=self.l2norm_qk, beta_is_logit=self.beta_is_logit,
            A_log=self.A_log, dt_bias=self.dt_bias, lower_bound=self.lower_bound,
        )

    def tokens(self):
        return self.B * self.T if self.cu_seqlens is None else int(self.cu_seqlens[-1])


CONFIG_SHAPES = {
    0: dict(B=1, H=1, T=256, dtype="fp32"),
    1: dict(B=1, H=6, T=8192, dtype="bf16"),
    2: dict(B=1, H=12, T=8192, dtype="bf16"),
    3: dict(B=1, H=96, T=8192, dtype="bf16"),
    4: dict(B=1, H=24, N=8, lmin=512, lmax=4096, dtype="bf16"),
}


def _normal_family(name, rng, B, T, H, dtype, state_sd, N=None, decay=-5.0):
    shp = (B, T, H, D)
    q = _unit_rows(rng.standard_normal(shp))
    k = _unit_rows(rng.standard_normal(shp))
    v = rng.standard_normal(shp)
    g = decay * _logistic(rng.standard_normal(shp))
    beta = _logistic(rng.standard_normal((B, T, H)))
    n = B if N is None else N
    state0 = None if state_sd is None else state_sd * rng.standard_normal((n, H, D, D))
    return KdaInputs(
        name=name, q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
        g=_store(g, dtype), beta=_store(beta, dtype),
        state0=None if state0 is None else _store(state0, dtype),
        dtype=dtype, state_dtype=dtype,
    )


def varlen_lengths(rng, n, lmin, lmax):
    return rng.integers(lmin, lmax + 1, size=n).astype(np.int64)


def _raw_gate_family(name, rng, lengths, H, dtype, lower_bound, state_sd=0.02):
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    N = len(lengths)
    shp = (1, T, H, D)
    q = rng.standard_normal(shp)
    k = rng.standard_normal(shp)
    v = rng.standard_normal(shp)
    g_raw = rng.standard_normal(shp)
    beta_logit = rng.standard_normal((1, T, H))
    state0 = state_sd * rng.standard_normal((N, H, D, D))
    A_log = rng.uniform(-1.0, 1.0, size=H)
    dt_bias = 0.1 * rng.standard_normal((H, D))
    return KdaInputs(
        name=name, q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
        g=_store(g_raw, dtype), beta=_store(beta_logit, dtype),
        state0=_store(state0, dtype), cu_seqlens=cu,
        A_log=A_log.astype(np.float32), dt_bias=dt_bias.astype(np.float32),
        lower_bound=float(lower_bound), l2norm_qk=True, beta_is_logit=True,
        dtype=dtype, state_dtype=dtype,
    )


def config(i, *, T=None, H=None, B=None, lengths=None, seed=None, dtype=None):
    """Benchmark configuration ``i`` (0..4), optionally at a reduced shape.

    Overrides keep the recipe and change only the shape (or, for config 4, the sequence
    lengths). The seed defaults to the configuration index.
    """
    s = CONFIG_SHAPES[i]
    seed = i if seed is None else seed
    rng = np.random.default_rng(seed)
    dt = dtype or s["dtype"]
    if i == 4:
        if lengths is None:
            lengths = varlen_lengths(rng, s["N"], s["lmin"], s["lmax"])
        return _raw_gate_family("config4", rng, lengths, s["H"] if H is None else H, dt,
                                -5.0)
    state_sd = 0.02 if i == 2 else None
    pick = lambda v, key: s[key] if v is None else v
    return _normal_family(f"config{i}", rng, pick(B, "B"), pick(T, "T"), pick(H, "H"), dt,
                          state_sd)


def stress(family, *, T, H, B=1, seed=100, dtype="bf16", lengths=None, gscale=2e-3,
           bscale=0.2):
    """Stress inputs that make the inter-chunk carry and the inverse matter. gscale and
    bscale are the decay and write-strength scales of ``weak_carry``."""
    rng = np.random.default_rng(seed)
    if family == "weak_carry":
        shp = (B, T, H, D)
        q = _unit_rows(rng.standard_normal(shp))
        k = _unit_rows(rng.standard_normal(shp))
        v = rng.standard_normal(shp)
        g = -gscale * _logistic(rng.standard_normal(shp))
        beta = bscale * _logistic(rng.standard_normal((B, T, H)))
        state0 = 0.1 * rng.standard_normal((B, H, D, D))
        return KdaInputs(
            name="weak_carry", q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
            g=_store(g, dtype), beta=_store(beta, dtype), state0=_store(state0, dtype),
            dtype=dtype, state_dtype=dtype, meta=dict(gscale=gscale, bscale=bscale),
        )
    if family == "weak_decay":
        return _normal_family("weak_decay", rng, B, T, H, dtype, 1.0, decay=-0.05)
    if family == "floor":
        x = _normal_family("floor", rng, B, T, H, dtype, 0.02)
        x.g = _store(np.full(x.g.shape, -5.0), dtype)
        return x
    if family == "correlated":
        shp = (B, T, H, D)
        key = _unit_rows(rng.standard_normal((1, 1, H, D)))
        k = np.broadcast_to(key, shp).copy()
        q = _unit_rows(rng.standard_normal(shp))
        v = rng.standard_normal(shp)
        state0 = 0.02 * rng.standard_normal((B, H, D, D))
        return KdaInputs(
            name="correlated", q=_store(q, dtype), k=_store(k, dtype),
            v=_store(v, dtype), g=_store(np.full(shp, -0.01), dtype),
            beta=_store(np.full((B, T, H), 0.5), dtype), state0=_store(state0, dtype),
            dtype=dtype, state_dtype=dtype,
        )
    if family == "gate_weak":
        if lengths is None:
            lengths = varlen_lengths(rng, 4, 16, 300)
        return _raw_gate_family("gate_weak", rng, lengths, H, dtype, -0.1)
    raise ValueError(family)


def with_dtype(x: KdaInputs, dtype):
    """The same draw re-rounded to another storage dtype (values already exact in BF16
    stay exact in FP32)."""
    f = lambda a: None if a is None else _store(a, dtype)
    return replace(x, q=f(x.q), k=f(x.k), v=f(x.v), g=f(x.g), beta=f(x.beta),
                   state0=f(x.state0), dtype=dtype, state_dtype=dtype)


def large_device(*, B, T, H, seed, device="cuda"):
    """Config 1's recipe (q, k ~ N(0,1) at unit L2 norm per row, v ~ N(0,1),
    g = -5 logistic(N(0,1)), beta = logistic(N(0,1)), zero initial state), drawn on the
    GPU with a seeded torch generator in FP32 and stored as BF16: for shapes too large
    to draw on the host. Returns a dict of device tensors q, k, v, g, beta
    ([B, T, H, 128] / [B, T, H]); the oracle is fed host copies of the heads it checks.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shp = (B, T, H, D)
    out = {}
    for name in ("q", "k", "v", "g"):
        x = torch.randn(shp, generator=gen, device=device, dtype=torch.float32)
        if name in ("q", "k"):
            x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        elif name == "g":
            x = -5.0 * torch.sigmoid(x)
        out[name] = x.to(torch.bfloat16)
        del x
    b = torch.randn((B, T, H), generator=gen, device=device, dtype=torch.float32)
    out["beta"] = torch.sigmoid(b).to(torch.bfloat16)
    return out
