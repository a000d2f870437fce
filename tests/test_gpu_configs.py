"""The five benchmark configurations at full size, in the launch configuration bench.py
times (automatic geometry). The oracle computes a sample of heads in full (heads are
independent, so a sampled head is an exact, complete check of that head's outputs and
final state over all tokens); config 0 and 1 are checked on every head."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("cfg,heads", [(0, None), (1, None), (2, [0, 7, 11]),
                                       (3, [0, 45, 95]), (4, [0, 13, 23])])
def test_config_full_size(cfg, heads):
    x = kda_synth.config(cfg)
    print(f"[config{cfg}] T={x.T} H={x.H} N={x.N} tokens={x.tokens()} heads={heads}",
          flush=True)
    o, s, _ = run_gpu(x)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    o_ref, s_ref = run_oracle(x, heads=heads)
    hs = slice(None) if heads is None else heads
    eo = rel_err(o[:, :, hs], o_ref)
    es = rel_err(s[:, hs], s_ref)
    print(f"[config{cfg}] o err {eo:.3e} state err {es:.3e}", flush=True)
    assert eo <= TOL and es <= TOL
