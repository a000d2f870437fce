"""State pool (ssm_state_indices) and scheduling order (seq_order), the flashinfer
page's sections "State and graph semantics" and "Packed scheduling": sequence n starts
from pool slot idx[n] and writes its final state back there, in place; other slots are
untouched; an out-of-range slot id makes the sequence start from zero and write nothing.
seq_order changes only the order in which work starts: results are bitwise identical.
Bound: max|err| / max|ref| <= 2e-2."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, to_device

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


def pool_case(idx, slots=5, pad=64, **kw):
    import torch

    import chunkwise_delta_rule_kda_amd as kda
    from oracle import kda_recurrence_fp64

    x = kda_synth.config(4, H=2, lengths=[40, 17, 70])
    print(f"[case] pool idx={idx} slots={slots} pad={pad} {kw}", flush=True)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    d.pop("state_in")
    rng = np.random.default_rng(5)
    init = kda_synth.round_bf16(0.02 * rng.standard_normal((slots, 2, D, D)))
    dense = 2 * D * D
    store = torch.zeros((slots, dense + pad), dtype=torch.bfloat16, device="cuda")
    store[:, :dense] = torch.from_numpy(init.reshape(slots, dense)).to("cuda", torch.bfloat16)
    pool = store[:, :dense].view(slots, 2, D, D)  # slot pitch dense + pad elements
    before = store.clone()
    ids = torch.tensor(idx, dtype=torch.int32, device="cuda")
    out = kda.kda_prefill(q, k, v, g, beta, pool, ssm_state_indices=ids, **d, **kw)
    torch.cuda.synchronize()
    o = out[0].float().cpu().numpy()
    assert out[1].data_ptr() == pool.data_ptr()
    s0 = np.stack([init[i] if 0 <= i < slots else np.zeros((2, D, D), np.float32)
                   for i in idx])
    ref = kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta, s0, **{
        k2: v2 for k2, v2 in x.oracle_kwargs().items() if k2 != "state0"},
        checkpoint_every=kw.get("checkpoint_every"))
    o_ref, s_ref = ref[0], ref[1]
    assert rel_err(o, o_ref) <= TOL
    after = store.float().cpu().numpy()
    for j in range(slots):
        if j in idx:
            n = idx.index(j)
            got = after[j, :dense].reshape(2, D, D)
            assert rel_err(got, s_ref[n]) <= TOL, j
        else:
            assert np.array_equal(after[j], before[j].float().cpu().numpy()), j
        assert np.array_equal(after[j, dense:], before[j, dense:].float().cpu().numpy())
    if kw.get("checkpoint_every"):
        ck = out[2].float().cpu().numpy()
        assert rel_err(ck, ref[2]) <= TOL
    return o


def test_pool_in_place_serial():
    pool_case([4, 0, 2], segment_chunks=-1)


def test_pool_in_place_segmented():
    pool_case([4, 0, 2], segment_chunks=2)


def test_pool_with_checkpoints():
    pool_case([1, 3, 0], segment_chunks=-1, checkpoint_every=32)


def test_out_of_range_slot_starts_from_zero_and_writes_nothing():
    pool_case([4, 9, 2], segment_chunks=-1)
    pool_case([-1, 0, 2], segment_chunks=2)


@pytest.mark.parametrize("L", [-1, 2])
def test_pool_whole_head_workgroups(L):
    # 128 value rows per workgroup (eight compute waves), serial and segmented, with an
    # out-of-range slot and checkpoints in the serial case.
    pool_case([4, 0, 9], segment_chunks=L, rows_per_workgroup=128,
              **({"checkpoint_every": 32} if L < 0 else {}))


@pytest.mark.parametrize("L", [-1, 2])
def test_seq_order_changes_nothing(L):
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.config(4, H=3, lengths=[50, 0, 130, 7, 90])
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    base = kda.kda_prefill(q, k, v, g, beta, segment_chunks=L, **d)
    torch.cuda.synchronize()
    for order in ([4, 3, 2, 1, 0], [2, 4, 0, 3, 1]):
        so = torch.tensor(order, dtype=torch.int32, device="cuda")
        got = kda.kda_prefill(q, k, v, g, beta, segment_chunks=L, seq_order=so, **d)
        torch.cuda.synchronize()
        assert torch.equal(got[0], base[0]) and torch.equal(got[1], base[1]), order


def test_seq_order_fixed_layout():
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    x = kda_synth.config(2, T=100, H=2, B=3)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    base = kda.kda_prefill(q, k, v, g, beta, segment_chunks=-1, **d)
    so = torch.tensor([2, 0, 1], dtype=torch.int32, device="cuda")
    got = kda.kda_prefill(q, k, v, g, beta, segment_chunks=-1, seq_order=so, **d)
    torch.cuda.synchronize()
    assert torch.equal(got[0], base[0]) and torch.equal(got[1], base[1])


def test_automatic_order_changes_nothing():
    # Varlen serial calls without a seq_order start the sequences longest first (ordered
    # on the device); the results equal those of the natural order bitwise.
    import torch

    import chunkwise_delta_rule_kda_amd as kda
    from kda_testlib import run_oracle

    x = kda_synth.config(4, H=2, lengths=[5, 300, 40, 0, 170, 33])
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    auto = kda.kda_prefill(q, k, v, g, beta, segment_chunks=-1, **d)
    ident = torch.arange(x.N, dtype=torch.int32, device="cuda")
    nat = kda.kda_prefill(q, k, v, g, beta, segment_chunks=-1, seq_order=ident, **d)
    torch.cuda.synchronize()
    assert torch.equal(auto[0], nat[0]) and torch.equal(auto[1], nat[1])
    o_ref, s_ref = run_oracle(x)
    assert rel_err(auto[0].float().cpu().numpy(), o_ref) <= 2e-2
    assert rel_err(auto[1].float().cpu().numpy(), s_ref) <= 2e-2

