"""Helpers shared by the GPU tests: move a synthetic draw to the device, run the HIP path
through the C ABI, run the oracle on the same values, and measure the error."""

import numpy as np

import kda_synth


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def torch_dtype(name):
    import torch

    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def to_device(x: kda_synth.KdaInputs, device="cuda"):
    import torch

    dt = torch_dtype(x.dtype)
    sdt = torch_dtype(x.state_dtype)
    t = lambda a, d: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device, d)
    out = dict(q=t(x.q, dt), k=t(x.k, dt), v=t(x.v, dt), g=t(x.g, dt), beta=t(x.beta, dt),
               state_in=t(x.state0, sdt))
    if x.cu_seqlens is not None:
        out["cu_seqlens"] = torch.from_numpy(np.asarray(x.cu_seqlens, np.int64)).to(device)
    if x.A_log is not None:
        out["A_log"] = t(x.A_log, torch.float32)
        out["dt_bias"] = t(x.dt_bias, torch.float32)
        out["lower_bound"] = x.lower_bound
    out["l2norm_qk"] = x.l2norm_qk
    out["beta_is_logit"] = x.beta_is_logit
    out["state_dtype"] = sdt
    out["scale"] = x.scale
    return out


def run_gpu(x, **kw):
    """Returns (o, state_out) as float64 numpy arrays plus the raw torch outputs (o, state_out
    and, with checkpoint_every, the checkpoints)."""
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    d = to_device(x)
    d.update(kw)
    q, k, v, g, beta = d.pop("q"), d.pop("k"), d.pop("v"), d.pop("g"), d.pop("beta")
    raw = kda.kda_prefill(q, k, v, g, beta, **d)  # (o, state[, checkpoints])
    o, st = raw[0], raw[1]
    torch.cuda.synchronize()
    on = o.float().cpu().numpy().astype(np.float64)
    sn = None if st is None else st.float().cpu().numpy().astype(np.float64)
    return on, sn, raw


def run_oracle(x, heads=None):
    from oracle import kda_recurrence_fp64

    return kda_recurrence_fp64(x.q, x.k, x.v, x.g, x.beta, heads=heads, **x.oracle_kwargs())


def bf16_bits_to_f32(u16):
    return (np.asarray(u16, np.uint32) << 16).view(np.float32)
