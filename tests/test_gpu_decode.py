"""One token per sequence (T = 1, fixed layout): the single-token kernel vs the FP64
oracle (the token recurrence itself), including the in-kernel transforms, FP32 I/O, the
state pool, and a multi-step decode that must agree with a prefill over the same tokens.
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


def test_plan_uses_the_single_token_kernel():
    import chunkwise_delta_rule_kda_amd as kda

    a = kda.make_args(B=64, T=1, H=8, N=64)
    assert kda.kda_prefill_plan(a)["decode"] == 1
    assert kda.kda_prefill_workspace_bytes(a) == 0
    assert kda.kda_prefill_plan(kda.make_args(B=64, T=2, H=8, N=64))["decode"] == 0


@pytest.mark.parametrize("B,H", [(1, 1), (5, 3), (64, 8)])
def test_bf16_with_initial_state(B, H):
    check(kda_synth.config(2, T=1, H=H, B=B), f"config2 B={B} H={H}")


def test_fp32():
    check(kda_synth.config(0, T=1, B=4), "config0 fp32")


def test_transforms_gate_l2_beta_logit():
    # config 4's raw-gate recipe with every sequence one token long, as a fixed layout
    x = kda_synth.config(4, H=3, lengths=[1] * 6)
    f = lambda a: a.reshape((6, 1) + a.shape[2:])
    y = kda_synth.KdaInputs(
        name="decode-transforms", q=f(x.q), k=f(x.k), v=f(x.v), g=f(x.g), beta=f(x.beta),
        state0=x.state0, dtype=x.dtype, state_dtype=x.state_dtype, A_log=x.A_log,
        dt_bias=x.dt_bias, lower_bound=x.lower_bound, l2norm_qk=x.l2norm_qk,
        beta_is_logit=x.beta_is_logit)
    check(y, "transforms")


def test_steps_equal_prefill():
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.config(2, T=40, H=2, B=3)
    o_ref, s_ref = run_oracle(x)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    st = d.pop("state_in").clone()
    outs = []
    for t in range(x.T):
        sl = lambda a: a[:, t:t + 1].contiguous()
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

    x = kda_synth.config(2, T=1, H=2, B=3)
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
