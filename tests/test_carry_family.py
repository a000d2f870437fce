"""The weak_carry input family keeps the segment carry significant (CPU, oracle only).

The GPU's time-segmented form is exact only if its transition Phi (the product of the
token transitions over a segment, the "FlashKDA column split" post's S_{c+1} update
applied with V = 0 from the identity) and its combine are right. Under the benchmark
recipe (g = -5 logistic(N(0,1))) Phi over a segment is below 1e-300, so a wrong Phi
cannot show in any output. These pins show, with the oracle's identity-start, V = 0
run, that ``kda_synth.stress("weak_carry", ...)`` at the scales the GPU carry tests use
keeps every singular value of Phi above 0.1 over one automatic segment: 47 chunks (the
automatic segment at H = 6 and H = 12, T = 8192), 103 chunks (H = 24) and 171 chunks
(H = 48), and that the
start state then moves the last outputs of the segment by a visible fraction.
"""

import numpy as np
import pytest

import kda_synth
from oracle import kda_recurrence_fp64

D = 128


@pytest.mark.parametrize("chunks,gscale,bscale",
                         [(47, 2e-3, 0.2), (103, 5e-4, 0.05), (171, 5e-4, 0.05)])
def test_transition_over_one_segment_is_significant(chunks, gscale, bscale):
    x = kda_synth.stress("weak_carry", T=16 * chunks, H=1, gscale=gscale, bscale=bscale)
    eye = np.eye(D)[None, None]
    zeros = np.zeros_like(x.v)
    _, phi = kda_recurrence_fp64(x.q, x.k, zeros, x.g, x.beta, state0=eye, scale=x.scale)
    sv = np.linalg.svd(phi[0, 0], compute_uv=False)
    assert sv.min() >= 0.1, sv.min()
    assert sv.max() <= 1.0 + 1e-12  # a product of contractions
    # The start state shapes the segment's last outputs: with and without it they
    # differ by more than 10 % of their size.
    o, _ = kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta, state0=x.state0, scale=x.scale)
    oz, _ = kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta, state0=None, scale=x.scale)
    last = slice(-16, None)
    diff = np.abs(o[:, last] - oz[:, last]).max() / np.abs(o[:, last]).max()
    assert diff > 0.1, diff


def test_family_values_are_in_range():
    x = kda_synth.stress("weak_carry", T=64, H=2)
    assert np.all(x.g <= 0) and np.all(x.g >= -2e-3)
    assert np.all(x.beta >= 0) and np.all(x.beta <= 0.2)
    np.testing.assert_allclose(np.linalg.norm(x.k, axis=-1), 1.0, atol=1e-2)
