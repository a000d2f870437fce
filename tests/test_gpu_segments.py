"""The segmented (time-parallel) form of the recurrence vs the FP64 oracle.

The chunk carry is affine in the state, so a sequence cut into segments is evaluated as:
the first segment from the true initial state; each later segment's zero-start run
(its end state Z_p and its output O^Z) and transition run (Phi_p, and Qt Phi^T per
chunk); the serial combine S_{p+1} = S_p Phi_p + Z_p, whose last step gives the final
state; and a parallel pass adding (Qt Phi^T) S_p^T to each later chunk's output (the
affine-output form, taken when no checkpoints are asked for; the re-run form that
checkpoints need is covered by the checkpoint tests). These tests force segment lengths
from one chunk upward so that every part runs (a single combine step with two segments,
many with one-chunk segments), on inputs whose decay is weak enough that the carry
across segments decides the result. Bound: max|err| / max|ref| <= 2e-2.
"""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2


def check(x, name, tol=TOL, **kw):
    print(f"[case] {name}: B={x.B} T={x.T} H={x.H} N={x.N} dtype={x.dtype} {kw}", flush=True)
    o, s, _ = run_gpu(x, **kw)
    o_ref, s_ref = run_oracle(x)
    eo = rel_err(o, o_ref)
    es = None if s is None else rel_err(s, s_ref)
    print(f"[case] {name}: o err {eo:.3e} state err {es}", flush=True)
    assert np.all(np.isfinite(o))
    assert eo <= tol, (name, eo)
    if s is not None:
        assert np.all(np.isfinite(s))
        assert es <= tol, (name, es)
    return o, s


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


# T = 200: 13 chunks, the last one 8 tokens.
@pytest.mark.parametrize("L", [1, 2, 3, 5, 7, 13, 40])
def test_weak_decay_segment_lengths(L):
    x = kda_synth.stress("weak_decay", T=200, H=2)
    check(x, f"weak_decay L={L}", segment_chunks=L)


@pytest.mark.parametrize("L", [1, 4])
def test_config2_recipe_with_initial_state(L):
    check(kda_synth.config(2, T=300, H=3), f"config2 L={L}", segment_chunks=L)


def test_fp32_config0_segments():
    check(kda_synth.config(0), "config0 L=3", segment_chunks=3)


@pytest.mark.parametrize("family", ["correlated", "floor", "weak_decay"])
def test_stress_families_segments(family):
    check(kda_synth.stress(family, T=256, H=2), f"{family} L=2", segment_chunks=2)


def test_varlen_segments_with_transforms():
    # Segments per sequence with L = 2: 2, 1 (empty), 3, 1, 7, 1.
    x = kda_synth.config(4, H=2, lengths=[20, 0, 33, 5, 200, 16])
    check(x, "config4 varlen L=2", segment_chunks=2)


def test_varlen_weak_gate_segments():
    check(kda_synth.stress("gate_weak", T=0, H=2, lengths=[130, 3, 77]), "gate_weak L=1",
          segment_chunks=1)


def test_batch_fixed_layout_segments():
    check(kda_synth.config(2, T=100, H=2, B=3), "batch3 L=2", segment_chunks=2)


def test_bitwise_identical_across_row_blocks():
    x = kda_synth.stress("weak_decay", T=200, H=2)
    ref_o, ref_s, _ = run_gpu(x, segment_chunks=3, rows_per_workgroup=64)
    for rows in (16, 32, 64, 0):
        o, s, _ = run_gpu(x, segment_chunks=3, rows_per_workgroup=rows)
        assert np.array_equal(o, ref_o) and np.array_equal(s, ref_s), rows


def test_segments_agree_with_serial():
    x = kda_synth.stress("weak_decay", T=512, H=1)
    o1, s1, _ = run_gpu(x, segment_chunks=-1)
    o2, s2, _ = run_gpu(x, segment_chunks=4)
    scale_o = np.max(np.abs(o1))
    scale_s = np.max(np.abs(s1))
    assert np.max(np.abs(o1 - o2)) <= 2e-2 * scale_o
    assert np.max(np.abs(s1 - s2)) <= 2e-2 * scale_s


def test_in_place_state_and_no_final_state():
    import torch

    import chunkwise_delta_rule_kda_amd as kda
    from kda_testlib import to_device

    x = kda_synth.stress("weak_decay", T=160, H=2)
    o_ref, s_ref = run_oracle(x)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    st = d.pop("state_in").clone()
    o, s = kda.kda_prefill(q, k, v, g, beta, st, state_out=st, segment_chunks=2, **d)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    assert rel_err(o.float().cpu().numpy(), o_ref) <= TOL
    assert rel_err(st.float().cpu().numpy(), s_ref) <= TOL
    d2 = to_device(x)
    q, k, v, g, beta = (d2.pop(n) for n in ("q", "k", "v", "g", "beta"))
    o2, s2 = kda.kda_prefill(q, k, v, g, beta, output_final_state=False, segment_chunks=2,
                             **d2)
    torch.cuda.synchronize()
    assert s2 is None
    assert rel_err(o2.float().cpu().numpy(), o_ref) <= TOL


def test_automatic_segments_on_a_long_sequence():
    # H = 2, T = 4096 (256 chunks): the automatic rule cuts it into segments.
    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.stress("weak_decay", T=4096, H=2)
    args = kda.make_args(B=1, T=x.T, H=x.H, N=1)
    plan = kda.kda_prefill_plan(args)
    assert plan["segment_chunks"] > 0 and plan["segments_per_head_bound"] >= 3
    check(x, "weak_decay auto segments")
