"""Every pairing of the I/O dtype (BF16, FP32) with the state dtype (BF16, FP32) through
each form of the recurrence, against the FP64 oracle: the serial form, the segmented
form with the combine and scan-output launches (four segments) and the segmented form
with the carry-and-output launch (thirteen segments of one chunk). The inputs are the
weak-decay family with a unit-scale initial state, T = 200 (13 chunks, the last one of
8 tokens), B = 2, H = 2, so that each segment's start state and the carry between
segments decide the result (the "FlashKDA column split" post, section 1: a run of
chunks acts on the entering state as S Phi + Z). Bound: max|err| / max|ref| <= 2e-2 for
o and the final state. The same pairings also go through the token-loop kernel that a
call of one to eight tokens per sequence takes (T = 1, a decode step, and T = 4, the
verification of draft tokens).
"""

import dataclasses

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2
FORMS = {"serial": -1, "combine": 4, "carry": 1}
PAIRS = [("bf16", "bf16"), ("bf16", "fp32"), ("fp32", "bf16"), ("fp32", "fp32")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def inputs(io, st, T=200, H=2, B=2):
    x = kda_synth.stress("weak_decay", T=T, H=H, B=B, dtype=io)
    # the state the GPU receives, exactly: BF16 values when the state is BF16
    s0 = kda_synth.round_bf16(x.state0) if st == "bf16" else x.state0
    return dataclasses.replace(x, state0=s0, state_dtype=st)


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("io,st", PAIRS)
def test_dtype_pairing_through_each_form(io, st, form):
    import chunkwise_delta_rule_kda_amd as kda

    x = inputs(io, st)
    L = FORMS[form]
    code = {"bf16": kda.KDA_BF16, "fp32": kda.KDA_FP32}
    p = kda.kda_prefill_plan(kda.make_args(B=x.B, T=x.T, H=x.H, N=x.N, io_dtype=code[io],
                                           state_dtype=code[st], segment_chunks=L))
    print(f"[case] io={io} state={st} form={form}: segment_chunks={p['segment_chunks']} "
          f"combine_wgs={p['combine_workgroups']} last_wgs={p['scan_c_workgroups']}",
          flush=True)
    if form == "serial":
        assert p["segment_chunks"] == 0
    else:
        assert p["segment_chunks"] == L and p["scan_affine_output"] == 1
        assert (p["combine_workgroups"] == 0) == (form == "carry")
    o, s, _ = run_gpu(x, segment_chunks=L)
    o_ref, s_ref = run_oracle(x)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print(f"[case] io={io} state={st} form={form}: o err {eo:.3e} state err {es:.3e}",
          flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= TOL and es <= TOL


@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("io,st", PAIRS)
def test_dtype_pairing_through_the_token_loop(io, st, T):
    import chunkwise_delta_rule_kda_amd as kda

    x = inputs(io, st, T=T, H=3, B=5)
    code = {"bf16": kda.KDA_BF16, "fp32": kda.KDA_FP32}
    p = kda.kda_prefill_plan(kda.make_args(B=x.B, T=x.T, H=x.H, N=x.N, io_dtype=code[io],
                                           state_dtype=code[st]))
    assert p["decode"] == 1
    o, s, _ = run_gpu(x)
    o_ref, s_ref = run_oracle(x)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print(f"[case] token loop io={io} state={st} T={T}: o err {eo:.3e} state err {es:.3e}",
          flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= TOL and es <= TOL
