"""The carry-and-output launch of the affine-output segmented form vs the FP64 oracle.

With seven or more segments per sequence (fixed layout) the combine launch and the
scan-output launch are replaced by one launch in which every later segment's workgroups
form their start state S_p from segment 0's end state by the chain S_{s+1} =
S_s Phi_s + Z_s, add (Qt Phi^T) S_p^T to each of the segment's chunks, and the last
segment's take one more step to the final state (the "FlashKDA column split" post,
section 1: the state update is affine in the entering state, so a run of chunks acts on
it as S Phi + Z). These cases force that form on small inputs whose decay is weak enough
for the carry to decide the result: FP32 and BF16 I/O, several sequences with a ragged
last chunk, last segments shorter than four chunks (waves without a chunk), a state
pool with an out-of-range slot, and calls without a final state. Bound:
max|err| / max|ref| <= 2e-2 for o and the final state.
"""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

TOL = 2e-2
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def plan_of(x, L):
    import chunkwise_delta_rule_kda_amd as kda

    io = kda.KDA_FP32 if x.dtype == "fp32" else kda.KDA_BF16
    return kda.kda_prefill_plan(kda.make_args(B=x.B, T=x.T, H=x.H, N=x.N, io_dtype=io,
                                              segment_chunks=L))


def check(x, name, L, **kw):
    p = plan_of(x, L)
    later = -(-((x.T + 15) // 16) // L) - 1
    print(f"[case] {name}: B={x.B} T={x.T} H={x.H} dtype={x.dtype} L={L} later={later} "
          f"combine_wgs={p['combine_workgroups']} last_wgs={p['scan_c_workgroups']}",
          flush=True)
    assert p["scan_affine_output"] == 1 and p["combine_workgroups"] == 0
    assert p["scan_c_workgroups"] == x.H * x.N * later * 4
    o, s, _ = run_gpu(x, segment_chunks=L, **kw)
    o_ref, s_ref = run_oracle(x)
    eo = rel_err(o, o_ref)
    es = None if s is None else rel_err(s, s_ref)
    print(f"[case] {name}: o err {eo:.3e} state err {es}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= TOL
    if s is not None:
        assert np.all(np.isfinite(s)) and es <= TOL
    return s


def test_carry_out_fp32():
    # T = 256: 16 chunks, L = 2 -> 8 segments; FP32 inputs, outputs and state.
    check(kda_synth.config(0), "config0 fp32", 2)


@pytest.mark.parametrize("L", [1, 2])
def test_carry_out_batch_ragged(L):
    # T = 200: 13 chunks (the last one 8 tokens). L = 1: 13 segments of one chunk (three
    # of a workgroup's four waves have no chunk); L = 2: 7 segments, the last of one chunk.
    x = kda_synth.stress("weak_decay", T=200, H=2, B=3)
    check(x, f"weak_decay B=3 L={L}", L)


def test_carry_out_initial_state_and_strong_decay():
    # The benchmark recipe with an initial state (config 2's draw), 19 chunks.
    check(kda_synth.config(2, T=300, H=3), "config2 T=300", 2)


def test_carry_out_without_final_state():
    x = kda_synth.stress("weak_decay", T=200, H=2, B=2)
    s = check(x, "no final state", 1, output_final_state=False)
    assert s is None


def test_carry_out_state_pool():
    import torch

    import chunkwise_delta_rule_kda_amd as kda
    from oracle import kda_recurrence_fp64

    x = kda_synth.stress("weak_decay", T=200, H=2, B=3)
    idx, slots = [4, 9, 2], 5  # slot 9 is out of range: start from zero, write nothing
    print(f"[case] carry-out pool idx={idx}", flush=True)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    d.pop("state_in")
    rng = np.random.default_rng(7)
    init = kda_synth.round_bf16(0.05 * rng.standard_normal((slots, 2, D, D)))
    pool = torch.from_numpy(init).to("cuda", torch.bfloat16)
    before = pool.clone()
    ids = torch.tensor(idx, dtype=torch.int32, device="cuda")
    out = kda.kda_prefill(q, k, v, g, beta, pool, ssm_state_indices=ids, segment_chunks=1, **d)
    torch.cuda.synchronize()
    s0 = np.stack([init[i] if 0 <= i < slots else np.zeros((2, D, D), np.float32) for i in idx])
    o_ref, s_ref = kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta, s0, **{
        k2: v2 for k2, v2 in x.oracle_kwargs().items() if k2 != "state0"})[:2]
    assert rel_err(out[0].float().cpu().numpy(), o_ref) <= TOL
    after = pool.float().cpu().numpy()
    for j in range(slots):
        if j in idx:
            assert rel_err(after[j], s_ref[idx.index(j)]) <= TOL, j
        else:
            assert np.array_equal(after[j], before[j].float().cpu().numpy()), j
