"""The segmented recurrence at the geometries the automatic plan picks for T = 8192,
on inputs whose segment carry is significant (GPU vs the FP64 oracle).

At T = 8192 the automatic plan cuts each (sequence, head) into P time segments: P = 11
segments of 47 chunks with 64-row workgroups at H = 6 and with 128-row workgroups at
H = 12 (both with the carry-and-output launch, two of its workgroups per CU at H = 12),
P = 5 of 103 chunks at H = 24 and P = 3 of 171 chunks at H = 48 (128-row, combine and
scan output). Under the benchmark recipe's strong decay only the
first chunk of a segment feels its start state, so these runs use the weak_carry family,
whose transition over one segment keeps every singular value above 0.1
(tests/test_carry_family.py): the S_p Phi_p + Z_p products that form each start state
(at H = 6 and 12 inside the carry-and-output launch, at H = 24 and 48 in the combine), the
(Qt Phi^T) S_p^T term at every chunk of a segment and the BF16 start states over ten
steps all decide the result. Bound: max|err| / max|ref| <= 2e-2 for o and the
final state, on every head at H = 6 and on sampled heads (each one complete over all
tokens) at H = 12, 24 and 48. The serial form (segment_chunks = -1) is checked on the same
inputs.
"""

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
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


CASES = [
    # H, decay and write scales, expected segments, chunks per segment, rows, heads
    (6, 2e-3, 0.2, 11, 47, 64, None),
    (12, 2e-3, 0.2, 11, 47, 128, [0, 5, 11]),
    (24, 5e-4, 0.05, 5, 103, 128, [0, 11, 23]),
    (48, 5e-4, 0.05, 3, 171, 128, [0, 47]),
]


@pytest.mark.parametrize("H,gscale,bscale,P,L,rows,heads", CASES)
def test_automatic_segments_carry(H, gscale, bscale, P, L, rows, heads):
    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.stress("weak_carry", T=8192, H=H, gscale=gscale, bscale=bscale)
    plan = kda.kda_prefill_plan(kda.make_args(B=1, T=x.T, H=H, N=1))
    print(f"[carry] H={H} plan segment_chunks={plan['segment_chunks']} "
          f"segments={plan['segments_per_head_bound']} rows={plan['rows_per_workgroup']}",
          flush=True)
    assert plan["segment_chunks"] == L
    assert plan["segments_per_head_bound"] == P
    assert plan["rows_per_workgroup"] == rows
    assert plan["scan_affine_output"] == 1
    # ten later segments: the carry-and-output launch; four or two: the combine and scan
    # output
    later = P - 1
    carry = later >= 6 and (H * later * 4 <= 256 or later >= 9)
    assert (plan["combine_workgroups"] == 0) == carry
    o_ref, s_ref = run_oracle(x, heads=heads)
    hs = slice(None) if heads is None else heads
    for seg in (0, -1):  # automatic (segmented), then serial
        o, s, _ = run_gpu(x, segment_chunks=seg)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
        eo = rel_err(o[:, :, hs], o_ref)
        es = rel_err(s[:, hs], s_ref)
        print(f"[carry] H={H} segment_chunks={seg}: o err {eo:.3e} state err {es:.3e}",
              flush=True)
        assert eo <= TOL and es <= TOL, (seg, eo, es)
