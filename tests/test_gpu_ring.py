"""Run lengths around the recurrence's loader pipeline vs the FP64 oracle.

The loader waves stage chunks through a 4-slot LDS ring and keep their global loads in
register sets used in rotation, unrolled in whole groups of sets, with a remainder loop
for the last chunks of a run. One varlen call whose sequences span every chunk count
from 1 to 13 (ragged tails and whole chunks) exercises every remainder and every slot
wrap-around, for each workgroup shape (16, 32, 64 and 128 rows: different loader counts and
set counts) in the serial form, with and without state checkpoints, and, with short
segments, in the segmented form. The weak gate keeps the carry across chunks large,
so a chunk staged in the wrong slot or read too early changes the result.
Bound: max|err| / max|ref| <= 2e-2.
"""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2

# chunk counts 1 .. 13, alternating a ragged tail and whole chunks
LENGTHS = [11, 32, 45, 64, 75, 96, 109, 128, 140, 160, 171, 192, 205]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


@pytest.fixture(scope="module")
def inputs():
    x = kda_synth.stress("gate_weak", T=None, H=2, lengths=LENGTHS)
    return x, run_oracle(x)


def check(inputs, name, **kw):
    x, (o_ref, s_ref) = inputs
    print(f"[case] ring {name}: lengths={LENGTHS} H={x.H} {kw}", flush=True)
    o, s, _ = run_gpu(x, **kw)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print(f"[case] ring {name}: o err {eo:.3e} state err {es:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= TOL and es <= TOL, (name, eo, es)


def test_lengths_cover_every_chunk_count():
    assert sorted((n + 15) // 16 for n in LENGTHS) == list(range(1, 14))


@pytest.mark.parametrize("rows", [16, 32, 64, 128])
def test_serial_run_lengths(inputs, rows):
    check(inputs, f"serial rows={rows}", rows_per_workgroup=rows, segment_chunks=-1)


@pytest.mark.parametrize("rows", [16, 64, 128])
def test_serial_run_lengths_with_checkpoints(inputs, rows):
    check(inputs, f"serial rows={rows} checkpoints", rows_per_workgroup=rows,
          segment_chunks=-1, checkpoint_every=32)


@pytest.mark.parametrize("L", [1, 2, 3, 6])
def test_segmented_run_lengths(inputs, L):
    check(inputs, f"segmented L={L}", segment_chunks=L)
