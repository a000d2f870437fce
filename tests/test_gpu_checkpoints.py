"""State checkpoints vs the FP64 oracle (the flashinfer page's checkpoint contract,
section "State and graph semantics"): every non-empty sequence writes its initial state
and the states after each whole interval that ends before the sequence does, at rows
checkpoint_cu_starts[n] + r. Covers the serial and the segmented form (checkpoints come
from the first segment's run and from the re-run of the others, the form a segmented
call takes when checkpoints are asked for), varlen with empty sequences, FP32 state,
intervals past the sequence length and the row cap.
Bound: max|err| / max|ref| <= 2e-2 over all rows; row 0 of a sequence is its initial
state exactly."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, to_device

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def lengths(x):
    if x.cu_seqlens is None:
        return [x.T] * x.B
    cu = list(np.asarray(x.cu_seqlens))
    return [b - a for a, b in zip(cu[:-1], cu[1:])]


def check(x, name, every, **kw):
    from oracle import checkpoint_starts, kda_recurrence_fp64

    print(f"[case] {name}: T={x.T} H={x.H} N={x.N} dtype={x.dtype} every={every} {kw}", flush=True)
    o, s, raw = run_gpu(x, checkpoint_every=every, **kw)
    ck = raw[2].float().cpu().numpy().astype(np.float64)
    o_ref, s_ref, c_ref = kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta,
                                              checkpoint_every=every, **x.oracle_kwargs())
    starts = checkpoint_starts(lengths(x), every)
    assert ck.shape == c_ref.shape and ck.shape[0] == starts[-1], (ck.shape, c_ref.shape)
    e = rel_err(ck, c_ref) if ck.size else 0.0
    print(f"[case] {name}: {ck.shape[0]} rows, checkpoint err {e:.3e}, o err "
          f"{rel_err(o, o_ref):.3e}", flush=True)
    assert np.all(np.isfinite(ck)) and e <= TOL, (name, e)
    assert rel_err(o, o_ref) <= TOL and rel_err(s, s_ref) <= TOL
    s0 = (np.zeros((x.N, x.H, 128, 128)) if x.state0 is None
          else np.asarray(x.state0, np.float64))
    for n, L in enumerate(lengths(x)):
        if L > 0:
            assert np.array_equal(ck[starts[n]], s0[n]), n  # row 0: the initial state
    o2, s2, _ = run_gpu(x, **kw)
    if kw.get("segment_chunks", 0) > 0:
        # Segmented: without checkpoints the call takes the affine-output form, which
        # rounds differently from the re-run form that checkpoints need.
        assert rel_err(o2, o_ref) <= TOL and rel_err(s2, s_ref) <= TOL
    else:
        # Serial form: checkpoints change nothing else.
        assert np.array_equal(o, o2) and np.array_equal(s, s2)
    return ck


@pytest.mark.parametrize("every", [16, 48, 160])
def test_serial_fixed_layout(every):
    check(kda_synth.config(2, T=200, H=3), f"config2 serial", every, segment_chunks=-1)


@pytest.mark.parametrize("L,every", [(3, 32), (1, 16), (4, 80)])
def test_segmented_form(L, every):
    check(kda_synth.stress("weak_decay", T=300, H=2), f"weak_decay L={L}", every,
          segment_chunks=L)


def test_batch_fixed_layout():
    check(kda_synth.config(2, T=100, H=2, B=3), "batch3", 32, segment_chunks=2)


@pytest.mark.parametrize("L", [-1, 2])
def test_varlen_with_empty_sequences(L):
    x = kda_synth.config(4, H=2, lengths=[20, 0, 33, 5, 200, 16])
    check(x, f"config4 varlen L={L}", 32, segment_chunks=L)


def test_fp32_state():
    check(kda_synth.config(0), "config0 fp32", 64)


def test_interval_past_every_length():
    # One row per non-empty sequence: its initial state.
    x = kda_synth.config(4, H=2, lengths=[20, 0, 33])
    ck = check(x, "long interval", 1024)
    assert ck.shape[0] == 2


def test_rows_beyond_the_buffer_are_not_written():
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.config(2, T=200, H=2)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    starts = torch.tensor([0, 13], dtype=torch.int64, device="cuda")  # 200 / 16 -> 13 rows
    big = torch.full((13, 2, 128, 128), 7.0, dtype=d["state_dtype"], device="cuda")
    view = big[:5]  # the library may write rows 0..4 only
    _, _, ck = kda.kda_prefill(q, k, v, g, beta, checkpoint_every=16, state_checkpoints=view,
                               checkpoint_cu_starts=starts, **d)
    torch.cuda.synchronize()
    assert ck.data_ptr() == big.data_ptr()
    assert torch.all(big[5:] == 7.0)
    assert not torch.all(big[:5] == 7.0)


@pytest.mark.parametrize("lens", [[0], [0, 0, 0]])
@pytest.mark.parametrize("L", [-1, 2])
def test_every_sequence_empty(lens, L):
    # No token at all: zero checkpoint rows (a zero-size buffer, whose pointer may be
    # NULL), no output, and each final state is its initial state.
    x = kda_synth.config(4, H=2, lengths=lens)
    print(f"[case] all empty {lens} L={L}", flush=True)
    o, s, raw = run_gpu(x, checkpoint_every=16, segment_chunks=L)
    assert o.size == 0 and raw[2].shape[0] == 0
    s0 = (np.zeros((x.N, x.H, 128, 128)) if x.state0 is None
          else np.asarray(x.state0, np.float64))
    assert np.array_equal(s, s0)
