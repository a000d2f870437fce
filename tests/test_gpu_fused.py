"""The fused form (fuse_prepare > 0): the chunk preparation runs in producer waves of the
recurrence workgroups and reaches the compute waves through the LDS ring, never through
HBM. Checked against the FP64 oracle at the same bound as the separate-kernel form
(max|err| / max|ref| <= 2e-2 for o and the final state), against that form, for bitwise
determinism across row-block counts and runs, and for a clear status word (no bounded
wait of the hand-over timed out)."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

TOL = 2e-2
FUSED = dict(fuse_prepare=1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def run_fused(x, **kw):
    """(o, state) as float64 arrays and the status word of the call's workspace."""
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    flags = (kda.KDA_FLAG_L2NORM_QK if x.l2norm_qk else 0) | \
            (kda.KDA_FLAG_BETA_IS_LOGIT if x.beta_is_logit else 0) | \
            (kda.KDA_FLAG_GATE_IN_KERNEL if x.A_log is not None else 0)
    dtype = {"bf16": kda.KDA_BF16, "fp32": kda.KDA_FP32}
    args = kda.make_args(B=x.B, T=x.T, H=x.H, N=x.N, cu_seqlens=d.get("cu_seqlens"),
                         A_log=d.get("A_log"), dt_bias=d.get("dt_bias"),
                         io_dtype=dtype[x.dtype], state_dtype=dtype[x.state_dtype],
                         lower_bound=x.lower_bound if x.A_log is not None else 0.0,
                         flags=flags, **FUSED, **kw)
    plan = kda.kda_prefill_plan(args)
    assert plan["fused"] == 1
    ws = torch.zeros(kda.kda_prefill_workspace_bytes(args), dtype=torch.uint8, device="cuda")
    o, s = kda.kda_prefill(q, k, v, g, beta, workspace=ws, **FUSED, **kw, **d)
    torch.cuda.synchronize()
    off = plan["status_offset"]
    status = int(ws[off:off + 4].cpu().numpy().view(np.int32)[0])
    return (o.float().cpu().numpy().astype(np.float64),
            s.float().cpu().numpy().astype(np.float64), status)


def check(x, name, heads=None, **kw):
    print(f"[fused] {name}: B={x.B} T={x.T} H={x.H} N={x.N} {kw}", flush=True)
    o, s, status = run_fused(x, **kw)
    assert status == 0, status
    o_ref, s_ref = run_oracle(x, heads=heads)
    hs = slice(None) if heads is None else heads
    eo, es = rel_err(o[:, :, hs], o_ref), rel_err(s[:, hs], s_ref)
    print(f"[fused] {name}: o err {eo:.3e} state err {es:.3e}", flush=True)
    assert eo <= TOL and es <= TOL, (name, eo, es)
    return o, s


@pytest.mark.parametrize("cfg,heads", [(0, None), (1, None), (2, [0, 11]), (3, [0, 95]),
                                       (4, [0, 23])])
def test_fused_configs_full_size(cfg, heads):
    check(kda_synth.config(cfg), f"config{cfg}", heads=heads)


@pytest.mark.parametrize("family", ["weak_decay", "correlated", "floor"])
@pytest.mark.parametrize("seg", [-1, 3])
def test_fused_stress_families(family, seg):
    check(kda_synth.stress(family, T=300, H=2), f"{family} L={seg}", segment_chunks=seg)


def test_fused_carry_at_the_automatic_segments():
    check(kda_synth.stress("weak_carry", T=8192, H=6), "weak_carry H=6 automatic")


def test_fused_varlen_transforms_and_empty_sequences():
    check(kda_synth.config(4, H=3, lengths=[20, 0, 33, 5, 200, 16, 1]), "config4 varlen",
          segment_chunks=-1)
    check(kda_synth.config(4, H=3, lengths=[20, 0, 33, 5, 200, 16, 1]), "config4 varlen L=2",
          segment_chunks=2)


@pytest.mark.parametrize("rows", [16, 32, 64, 128])
def test_fused_row_blocks_bitwise_identical(rows):
    x = kda_synth.stress("weak_decay", T=200, H=2)
    ref_o, ref_s, _ = run_fused(x, segment_chunks=-1, rows_per_workgroup=64)
    o, s, st = run_fused(x, segment_chunks=-1, rows_per_workgroup=rows)
    assert st == 0
    assert np.array_equal(o, ref_o) and np.array_equal(s, ref_s), rows
    o2, s2, _ = run_fused(x, segment_chunks=-1, rows_per_workgroup=rows)
    assert np.array_equal(o, o2) and np.array_equal(s, s2)


def test_fused_agrees_with_the_separate_kernel():
    x = kda_synth.config(2, T=1000, H=4)
    o_f, s_f, _ = run_fused(x)
    o_s, s_s, _ = run_gpu(x, fuse_prepare=-1)
    assert rel_err(o_f, o_s) <= 1e-2 and rel_err(s_f, s_s) <= 1e-2


def test_fused_checkpoints_and_pool():
    import torch

    import chunkwise_delta_rule_kda_amd as kda
    from oracle import kda_recurrence_fp64

    x = kda_synth.stress("weak_decay", T=160, H=2)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    o, s, ck = kda.kda_prefill(q, k, v, g, beta, checkpoint_every=32, **FUSED, **d)
    torch.cuda.synchronize()
    o_ref, s_ref, ck_ref = kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta,
                                               checkpoint_every=32, **x.oracle_kwargs())
    assert rel_err(ck.float().cpu().numpy(), ck_ref) <= TOL
    assert rel_err(o.float().cpu().numpy(), o_ref) <= TOL
    # state pool: sequence 0 from slot 2, written back there
    pool = torch.zeros((3, 2, 128, 128), dtype=torch.bfloat16, device="cuda")
    pool[2] = d["state_in"][0]
    ids = torch.tensor([2], dtype=torch.int32, device="cuda")
    d.pop("state_in")
    o2, _ = kda.kda_prefill(q, k, v, g, beta, pool, ssm_state_indices=ids, **FUSED, **d)
    torch.cuda.synchronize()
    assert rel_err(pool[2].float().cpu().numpy(), s_ref[0]) <= TOL
    assert rel_err(o2.float().cpu().numpy(), o_ref) <= TOL
