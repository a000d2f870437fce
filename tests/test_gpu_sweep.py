"""A seeded sweep of valid random shapes vs the FP64 oracle: every path the library picks
(token loop, serial, both segmented forms, the fused form, varlen with transforms) at
sizes the oracle finishes in well under a second, with forced and automatic geometry.
Each case draws, from its own seed: the layout (fixed batch or packed varlen with empty
and ragged sequences), T or the lengths, H, the I/O precision, an initial state or none,
the recurrence geometry (automatic, or explicit rows and segment length), for some the
fused form (chunk preparation inside the recurrence workgroups) and, for some,
checkpoints. Bound: max|err| / max|ref| <= 2e-2 for o, the final state and the
checkpoints."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2
CASES = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    H = int(rng.integers(1, 4))
    dtype = "fp32" if rng.random() < 0.25 else "bf16"
    if rng.random() < 0.4:
        n = int(rng.integers(1, 6))
        lengths = [int(v) for v in rng.integers(0, 260, n)]
        if rng.random() < 0.3:
            lengths[int(rng.integers(0, n))] = 0
        x = kda_synth.config(4, H=H, lengths=lengths, seed=2000 + seed, dtype=dtype)
    else:
        T = int(rng.choice([1, 3, 8, 16, 17, 40, 100, 255, 300]))
        B = int(rng.integers(1, 4))
        fam = rng.random()
        if fam < 0.5:
            x = kda_synth.config(2, T=T, H=H, B=B, seed=2000 + seed, dtype=dtype)
        else:
            x = kda_synth.stress("weak_decay", T=T, H=H, B=B, seed=2000 + seed, dtype=dtype)
    kw = {}
    geo = rng.random()
    if geo < 0.35:
        kw["segment_chunks"] = int(rng.choice([1, 2, 3, 5, 8]))
        rows = int(rng.choice([0, 64, 128]))
        if rows:
            kw["rows_per_workgroup"] = rows
    elif geo < 0.55:
        kw["segment_chunks"] = -1
        kw["rows_per_workgroup"] = int(rng.choice([16, 32, 64, 128]))
    if rng.random() < 0.3:
        kw["fuse_prepare"] = 1
    if rng.random() < 0.2:
        kw["checkpoint_every"] = int(rng.choice([16, 32, 64]))
    return x, kw


@pytest.mark.parametrize("seed", range(CASES))
def test_random_shape(seed):
    from oracle import checkpoint_starts, kda_recurrence_fp64

    x, kw = draw(seed)
    print(f"[case] sweep {seed}: B={x.B} T={x.T} H={x.H} N={x.N} dtype={x.dtype} "
          f"varlen={x.cu_seqlens is not None} {kw}", flush=True)
    out = run_gpu(x, **kw)
    o, s = out[0], out[1]
    every = kw.get("checkpoint_every")
    if every:
        o_ref, s_ref, c_ref = kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta,
                                                  checkpoint_every=every, **x.oracle_kwargs())
        ck = out[2][2].float().cpu().numpy().astype(np.float64)
        assert ck.shape == c_ref.shape
        if ck.size:
            assert rel_err(ck, c_ref) <= TOL
    else:
        o_ref, s_ref = run_oracle(x)
    if o.size:
        eo = rel_err(o, o_ref)
        print(f"[case] sweep {seed}: o err {eo:.3e}", flush=True)
        assert np.all(np.isfinite(o)) and eo <= TOL
    assert rel_err(s, s_ref) <= TOL
