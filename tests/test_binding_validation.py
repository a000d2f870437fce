"""The Python binding rejects, before any pointer reaches the C ABI, every argument the
C layer cannot check: it sees pointers, not sizes, dtypes or devices (CPU only: the
tensors here are host tensors, so a call that passed every check would still stop at the
device check, before any launch)."""

import pytest

torch = pytest.importorskip("torch")

import chunkwise_delta_rule_kda_amd as kda  # noqa: E402

B, T, H, D = 1, 32, 2, 128


def base(**over):
    a = dict(
        q=torch.zeros(B, T, H, D, dtype=torch.bfloat16),
        k=torch.zeros(B, T, H, D, dtype=torch.bfloat16),
        v=torch.zeros(B, T, H, D, dtype=torch.bfloat16),
        g=torch.zeros(B, T, H, D, dtype=torch.bfloat16),
        beta=torch.zeros(B, T, H, dtype=torch.bfloat16),
    )
    a.update(over)
    return a


def call(**over):
    a = base(**over)
    q, k, v, g, beta = (a.pop(n) for n in ("q", "k", "v", "g", "beta"))
    return kda.kda_prefill(q, k, v, g, beta, **a)


def expect(status, text, **over):
    with pytest.raises(kda.KdaError) as e:
        call(**over)
    assert e.value.status == status, str(e.value)
    assert text in str(e.value), str(e.value)


def test_valid_host_tensors_stop_at_the_device_check():
    expect(2, "must be a CUDA tensor")


def test_head_dim_and_shapes():
    expect(2, "head dimension", q=torch.zeros(B, T, H, 64, dtype=torch.bfloat16))
    expect(2, "k has shape", k=torch.zeros(B, T, H + 1, D, dtype=torch.bfloat16))
    expect(2, "v has shape", v=torch.zeros(B, T - 1, H, D, dtype=torch.bfloat16))
    expect(2, "beta has shape", beta=torch.zeros(B, T, H, 1, dtype=torch.bfloat16))


def test_dtypes():
    expect(3, "unsupported dtype", q=torch.zeros(B, T, H, D, dtype=torch.float16),
           k=torch.zeros(B, T, H, D, dtype=torch.float16),
           v=torch.zeros(B, T, H, D, dtype=torch.float16),
           g=torch.zeros(B, T, H, D, dtype=torch.float16),
           beta=torch.zeros(B, T, H, dtype=torch.float16))
    expect(3, "g is", g=torch.zeros(B, T, H, D, dtype=torch.float32))


def test_cu_seqlens():
    expect(3, "int64", cu_seqlens=torch.tensor([0, 32], dtype=torch.int32))
    expect(2, "1-D", cu_seqlens=torch.tensor([[0, 32]], dtype=torch.int64))
    two = torch.zeros(2, T, H, D, dtype=torch.bfloat16)
    expect(2, "B = 1", q=two, k=two.clone(), v=two.clone(), g=two.clone(),
           beta=torch.zeros(2, T, H, dtype=torch.bfloat16),
           cu_seqlens=torch.tensor([0, 32], dtype=torch.int64))


def test_gate_parameters():
    a_log = torch.zeros(H, dtype=torch.float32)
    dtb = torch.zeros(H, D, dtype=torch.float32)
    expect(4, "both", A_log=a_log)
    expect(4, "lower_bound", A_log=a_log, dt_bias=dtb)
    expect(3, "float32", A_log=a_log.double(), dt_bias=dtb, lower_bound=-5.0)
    expect(2, "A_log has shape", A_log=torch.zeros(H + 1), dt_bias=dtb, lower_bound=-5.0)
    expect(2, "dt_bias has shape", A_log=a_log, dt_bias=torch.zeros(H, D - 1),
           lower_bound=-5.0)


def test_states():
    st = torch.zeros(B, H, D, D, dtype=torch.bfloat16)
    expect(3, "state dtype", state_in=st, state_dtype=torch.float32)
    expect(2, "state_in has shape", state_in=torch.zeros(B, H + 1, D, D, dtype=torch.bfloat16))
    expect(2, "state_out must be", state_out=torch.zeros(B + 1, H, D, D, dtype=torch.bfloat16))
    expect(3, "state_out is", state_out=torch.zeros(B, H, D, D, dtype=torch.float32))
    expect(2, "o must be", o=torch.zeros(B, T, H, D, dtype=torch.float32))
    expect(2, "state_in must be contiguous",
           state_in=torch.zeros(B, H, D, D, dtype=torch.bfloat16).transpose(2, 3))


def test_pool_and_order():
    ids = torch.zeros(B, dtype=torch.int32)
    expect(10, "needs state_in", ssm_state_indices=ids)
    pool = torch.zeros(3, H, D, D, dtype=torch.bfloat16)
    expect(3, "ssm_state_indices", state_in=pool,
           ssm_state_indices=torch.zeros(B, dtype=torch.int64))
    expect(3, "seq_order", seq_order=torch.zeros(B + 1, dtype=torch.int32))
    expect(2, "state pool", state_in=torch.zeros(3, H, D, D - 8, dtype=torch.bfloat16),
           ssm_state_indices=ids)


def test_checkpoint_buffers():
    expect(2, "state_checkpoints", checkpoint_every=16,
           state_checkpoints=torch.zeros(2, H, D, D - 1, dtype=torch.bfloat16))
    expect(3, "state dtype", checkpoint_every=16,
           state_checkpoints=torch.zeros(2, H, D, D, dtype=torch.float32))
    expect(2, "checkpoint_cu_starts", checkpoint_every=16,
           checkpoint_cu_starts=torch.zeros(B + 2, dtype=torch.int64))
    expect(10, "multiple of 16", checkpoint_every=24)
