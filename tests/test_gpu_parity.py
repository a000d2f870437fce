"""HIP path vs the FP64 oracle, element by element, at sizes the oracle finishes in
seconds (several chunks and a ragged tail), plus the structural identities of the
method and the launch geometry. Bound: max|err| / max|ref| <= 2e-2 for o and the final
state (the target's tolerance)."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

TOL = 2e-2


def check(x, name, tol=TOL, **kw):
    print(f"[case] {name}: B={x.B} T={x.T} H={x.H} N={x.N} dtype={x.dtype} {kw}", flush=True)
    o, s, _ = run_gpu(x, **kw)
    o_ref, s_ref = run_oracle(x)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print(f"[case] {name}: o err {eo:.3e} state err {es:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= tol, (name, eo)
    assert es <= tol, (name, es)
    return eo, es


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


# ---- config-shaped small cases -------------------------------------------------------
def test_config0_full_fp32():
    check(kda_synth.config(0), "config0")


@pytest.mark.parametrize("T,H", [(16, 1), (1, 2), (80, 2), (257, 3)])
def test_config1_recipe_small(T, H):
    check(kda_synth.config(1, T=T, H=H), f"config1 T={T} H={H}")


def test_config2_recipe_with_initial_state():
    check(kda_synth.config(2, T=200, H=3), "config2-small")


def test_config4_recipe_small_varlen_with_transforms():
    x = kda_synth.config(4, H=3, lengths=[17, 0, 45, 1, 64, 33])
    check(x, "config4-small")


def test_fp32_io_bf16_state_mix():
    x = kda_synth.config(1, T=96, H=2, dtype="fp32")
    check(x, "fp32-io-bf16-state", state_dtype=__import__("torch").bfloat16)


def test_batch_fixed_layout():
    check(kda_synth.config(2, T=48, H=2, B=3), "batch3")


def test_heads_fast_preparation_grid_end_to_end():
    # H = 32 (the preparation grid's heads-fastest order) with packed sequences, an empty
    # one and a ragged last grid row; the oracle runs three heads in full.
    x = kda_synth.config(4, H=32, lengths=[700, 0, 33, 513, 250])
    heads = [0, 17, 31]
    print(f"[case] heads-fast grid: N={x.N} T={x.T} H={x.H} heads={heads}", flush=True)
    o, s, _ = run_gpu(x)
    o_ref, s_ref = run_oracle(x, heads=heads)
    eo, es = rel_err(o[:, :, heads], o_ref), rel_err(s[:, heads], s_ref)
    print(f"[case] heads-fast grid: o err {eo:.3e} state err {es:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= TOL and es <= TOL


# ---- stress inputs (carry and inverse matter) ----------------------------------------
@pytest.mark.parametrize("family,T", [("weak_decay", 256), ("correlated", 128),
                                      ("floor", 128)])
def test_stress_families(family, T):
    check(kda_synth.stress(family, T=T, H=2), family)


def test_stress_weak_decay_fp32():
    x = kda_synth.with_dtype(kda_synth.stress("weak_decay", T=512, H=1), "fp32")
    check(x, "weak_decay fp32")


def test_stress_gate_weak_varlen():
    check(kda_synth.stress("gate_weak", T=0, H=2, lengths=[40, 3, 77]), "gate_weak")


# ---- structural identities -----------------------------------------------------------
def test_bitwise_identical_across_slices_and_runs():
    x = kda_synth.config(2, T=160, H=2)
    ref_o, ref_s, _ = run_gpu(x, rows_per_workgroup=16)
    for rows in (16, 32, 64, 128, 0):
        o, s, _ = run_gpu(x, rows_per_workgroup=rows)
        assert np.array_equal(o, ref_o) and np.array_equal(s, ref_s), rows


def test_varlen_equals_separate_calls_bitwise():
    x = kda_synth.config(4, H=2, lengths=[33, 16, 0, 70])
    o, s, _ = run_gpu(x)
    cu = x.cu_seqlens
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            assert np.array_equal(s[n], x.state0[n].astype(np.float64))
            continue
        xn = kda_synth.KdaInputs(
            name="seq", q=x.q[:, a:b], k=x.k[:, a:b], v=x.v[:, a:b], g=x.g[:, a:b],
            beta=x.beta[:, a:b], state0=x.state0[n:n + 1], A_log=x.A_log, dt_bias=x.dt_bias,
            lower_bound=x.lower_bound, l2norm_qk=True, beta_is_logit=True)
        # Explicit geometry keeps a short sequence on the chunked path (a call of 8 or
        # fewer tokens would otherwise take the token-loop kernel, which rounds
        # differently); the row choice never changes results.
        on, sn, _ = run_gpu(xn, rows_per_workgroup=64)
        assert np.array_equal(o[:, a:b], on), n
        assert np.array_equal(s[n], sn[0]), n


def test_fixed_batch_equals_varlen_equal_lengths_bitwise():
    x = kda_synth.config(2, T=40, H=2, B=3)
    o, s, _ = run_gpu(x)
    flat = lambda a: a.reshape((1, 120) + a.shape[2:])
    xv = kda_synth.KdaInputs(name="v", q=flat(x.q), k=flat(x.k), v=flat(x.v), g=flat(x.g),
                             beta=flat(x.beta), state0=x.state0,
                             cu_seqlens=np.array([0, 40, 80, 120]))
    ov, sv, _ = run_gpu(xv)
    assert np.array_equal(ov.reshape(o.shape), o) and np.array_equal(sv, s)


def test_split_prefill_equals_one_call():
    import torch

    x = kda_synth.with_dtype(kda_synth.config(2, T=96, H=2), "fp32")
    o, s, _ = run_gpu(x)
    cut = 48  # chunk boundary: with an FP32 state the two calls are exact
    part = lambda a, sl: a[:, sl]
    xa = kda_synth.KdaInputs(name="a", q=x.q[:, :cut], k=x.k[:, :cut], v=x.v[:, :cut],
                             g=x.g[:, :cut], beta=x.beta[:, :cut], state0=x.state0,
                             dtype="fp32", state_dtype="fp32")
    oa, sa, _ = run_gpu(xa)
    xb = kda_synth.KdaInputs(name="b", q=x.q[:, cut:], k=x.k[:, cut:], v=x.v[:, cut:],
                             g=x.g[:, cut:], beta=x.beta[:, cut:],
                             state0=sa.astype(np.float32), dtype="fp32", state_dtype="fp32")
    ob, sb, _ = run_gpu(xb)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(sb, s)
    # A cut inside a chunk is a different chunking: equal within tolerance.
    xc = kda_synth.KdaInputs(name="c", q=x.q[:, :37], k=x.k[:, :37], v=x.v[:, :37],
                             g=x.g[:, :37], beta=x.beta[:, :37], state0=x.state0,
                             dtype="fp32", state_dtype="fp32")
    oc, sc, _ = run_gpu(xc)
    xd = kda_synth.KdaInputs(name="d", q=x.q[:, 37:], k=x.k[:, 37:], v=x.v[:, 37:],
                             g=x.g[:, 37:], beta=x.beta[:, 37:],
                             state0=sc.astype(np.float32), dtype="fp32", state_dtype="fp32")
    od, sd, _ = run_gpu(xd)
    assert rel_err(np.concatenate([oc, od], axis=1), o) < 1e-2
    assert rel_err(sd, s) < 1e-2


def test_in_place_state_update():
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.config(2, T=64, H=2)
    o_ref, s_ref, _ = run_gpu(x)
    d = to_device(x)
    st = d["state_in"]
    o, s2 = kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert s2.data_ptr() == st.data_ptr()
    assert np.array_equal(st.float().cpu().numpy(), s_ref)
    assert np.array_equal(o.float().cpu().numpy(), o_ref)


def test_no_final_state_and_zero_initial_state():
    x = kda_synth.config(1, T=50, H=2)
    o, s, _ = run_gpu(x, output_final_state=False)
    assert s is None
    o_ref, _ = run_oracle(x)
    assert rel_err(o, o_ref) <= TOL


def test_zero_tokens_passes_state_through():
    x = kda_synth.config(2, T=0, H=2)
    o, s, _ = run_gpu(x)
    assert o.size == 0
    assert np.array_equal(s, x.state0.astype(np.float64))


def test_workspace_too_small_is_rejected_before_launch():
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.config(1, T=32, H=1)
    d = to_device(x)
    for kw in (dict(), dict(fuse_prepare=1)):
        need = kda.kda_prefill_workspace_bytes(kda.make_args(B=1, T=32, H=1, N=1, **kw))
        ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
        with pytest.raises(kda.KdaError) as e:
            kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], workspace=ws, **kw)
        assert e.value.status == 7


def test_debug_check_cu_seqlens():
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    good = torch.tensor([0, 5, 5, 9], dtype=torch.int64, device="cuda")
    assert kda.kda_debug_check_cu_seqlens(good, 9) == 0
    bad = torch.tensor([0, 5, 4, 9], dtype=torch.int64, device="cuda")
    assert kda.kda_debug_check_cu_seqlens(bad, 9) == 9
    assert kda.kda_debug_check_cu_seqlens(good, 10) == 9
