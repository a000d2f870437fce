"""Maximum sizes: a prefill whose element offsets exceed 2^31 (B=1, T=20480, H=1024,
d=128: 2.7e9 elements per input tensor, 1,280 chunks per head), against the FP64 oracle
on two heads (the first and the last, whose offsets are the largest) over the whole
sequence. Inputs follow config 1's recipe, drawn on the GPU by
``kda_synth.large_device`` (too large to draw on the host); the oracle gets host copies
of the heads it checks. Bound: max|err| / max|ref| <= 2e-2 for o and the final state."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err

pytestmark = pytest.mark.gpu

T, H = 20480, 1024


def test_offsets_beyond_2_pow_31():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda
    from oracle import kda_recurrence_fp64

    free, _ = torch.cuda.mem_get_info()
    if free < 64 << 30:
        pytest.skip("needs about 50 GB of device memory")
    assert T * H * 128 > 2 ** 31
    print(f"[case] large: T={T} H={H}", flush=True)
    d = kda_synth.large_device(B=1, T=T, H=H, seed=7)
    o, st = kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    heads = [0, H - 1]
    host = {n: d[n][:, :, heads].float().cpu().numpy() for n in ("q", "k", "v", "g", "beta")}
    o_h = o[:, :, heads].float().cpu().numpy()
    s_h = st[:, heads].float().cpu().numpy()
    del d, o, st
    torch.cuda.empty_cache()
    o_ref, s_ref = kda_recurrence_fp64(host["q"], host["k"], host["v"], host["g"],
                                       host["beta"])
    eo, es = rel_err(o_h, o_ref), rel_err(s_h, s_ref)
    print(f"[case] large: o err {eo:.3e} state err {es:.3e}", flush=True)
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(s_h))
    assert eo <= 2e-2 and es <= 2e-2
