"""A few tokens per sequence (fixed layout, 1 <= T <= 8): the token-loop kernel vs the
FP64 oracle (the token recurrence itself), including the in-kernel transforms, FP32 I/O,
the state pool, the chunked path on the same inputs, and step-by-step decoding (one and
three tokens per call) that must agree with a prefill over the same tokens.
Bound: max|err| / max|ref| <= 2e-2."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def check(x, name, **kw):
    print(f"[case] decode {name}: B={x.B} T={x.T} H={x.H} dtype={x.dtype} {kw}", flush=True)
    o, s, _ = run_gpu(x, **kw)
    o_ref, s_ref = run_oracle(x)
    eo, es = rel_err(o, o_ref), rel_err(s, s_ref)
    print(f"[case] decode {name}: o err {eo:.3e} state err {es:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= TOL and es <= TOL


def test_plan_uses_the_token_loop_kernel():
    import chunkwise_delta_rule_kda_amd as kda

    plan = lambda **kw: kda.kda_prefill_plan(kda.make_args(B=64, H=8, N=64, **kw))
    for T in (1, 2, 8):
        a = kda.make_args(B=64, T=T, H=8, N=64)
        assert kda.kda_prefill_plan(a)["decode"] == 1, T
        assert kda.kda_prefill_workspace_bytes(a) == 0
    assert plan(T=9)["decode"] == 0
    # explicit geometry, or checkpoints, select the chunked path
    assert plan(T=4, rows_per_workgroup=64)["decode"] == 0
    assert plan(T=4, segment_chunks=-1)["decode"] == 0
    assert plan(T=4, checkpoint_every=16)["decode"] == 0


@pytest.mark.parametrize("B,H", [(1, 1), (5, 3), (64, 8)])
def test_bf16_with_initial_state(B, H):
    check(kda_synth.config(2, T=1, H=H, B=B), f"config2 B={B} H={H}")


def test_fp32():
    check(kda_synth.config(0, T=1, B=4), "config0 fp32")


@pytest.mark.parametrize("T,B,H", [(2, 5, 3), (5, 8, 4), (8, 3, 2)])
def test_draft_tokens_with_initial_state(T, B, H):
    check(kda_synth.config(2, T=T, H=H, B=B), f"config2 T={T} B={B} H={H}")


def test_draft_tokens_fp32_weak_decay():
    check(kda_synth.stress("weak_decay", T=7, H=2, B=2, dtype="fp32"), "weak decay fp32 T=7")


def test_token_loop_agrees_with_chunked_path():
    x = kda_synth.config(2, T=8, H=3, B=4)
    o1, s1, _ = run_gpu(x)                          # token loop
    o2, s2, _ = run_gpu(x, rows_per_workgroup=64)   # prepare + recurrence
    o_ref, s_ref = run_oracle(x)
    for o, s in ((o1, s1), (o2, s2)):
        assert rel_err(o, o_ref) <= TOL and rel_err(s, s_ref) <= TOL
    assert rel_err(o1, o2) <= TOL and rel_err(s1, s2) <= TOL


@pytest.mark.parametrize("T", [1, 7])
def test_transforms_gate_l2_beta_logit(T):
    # config 4's raw-gate recipe with every sequence T tokens long, as a fixed layout
    x = kda_synth.config(4, H=3, lengths=[T] * 6)
    f = lambda a: a.reshape((6, T) + a.shape[2:])
    y = kda_synth.KdaInputs(
        name="decode-transforms", q=f(x.q), k=f(x.k), v=f(x.v), g=f(x.g), beta=f(x.beta),
        state0=x.state0, dtype=x.dtype, state_dtype=x.state_dtype, A_log=x.A_log,
        dt_bias=x.dt_bias, lower_bound=x.lower_bound, l2norm_qk=x.l2norm_qk,
        beta_is_logit=x.beta_is_logit)
    check(y, f"transforms T={T}")


@pytest.mark.parametrize("step", [1, 3])
def test_steps_equal_prefill(step):
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.config(2, T=40, H=2, B=3)
    o_ref, s_ref = run_oracle(x)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    st = d.pop("state_in").clone()
    outs = []
    for t in range(0, x.T, step):
        sl = lambda a: a[:, t:t + step].contiguous()
        o, _ = kda.kda_prefill(sl(q), sl(k), sl(v), sl(g), sl(beta), st, state_out=st, **d)
        outs.append(o)
    torch.cuda.synchronize()
    o_dec = torch.cat(outs, 1).float().cpu().numpy()
    assert rel_err(o_dec, o_ref) <= TOL
    assert rel_err(st.float().cpu().numpy(), s_ref) <= TOL


def test_state_pool():
    import torch

    import chunkwise_delta_rule_kda_amd as kda
    from oracle import kda_recurrence_fp64

    x = kda_synth.config(2, T=3, H=2, B=3)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    d.pop("state_in")
    rng = np.random.default_rng(9)
    init = kda_synth.round_bf16(0.02 * rng.standard_normal((4, 2, 128, 128)))
    pool = torch.from_numpy(init).to("cuda", torch.bfloat16)
    before = pool.clone()
    idx = [3, 0, 9]  # the last one is out of range: zero start, nothing written
    ids = torch.tensor(idx, dtype=torch.int32, device="cuda")
    o, _ = kda.kda_prefill(q, k, v, g, beta, pool, ssm_state_indices=ids, **d)
    torch.cuda.synchronize()
    s0 = np.stack([init[3], init[0], np.zeros((2, 128, 128), np.float32)])
    o_ref, s_ref = kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta, s0, scale=x.scale)
    assert rel_err(o.float().cpu().numpy(), o_ref) <= TOL
    got = pool.float().cpu().numpy()
    assert rel_err(got[3], s_ref[0]) <= TOL and rel_err(got[0], s_ref[1]) <= TOL
    assert torch.equal(pool[1], before[1]) and torch.equal(pool[2], before[2])
