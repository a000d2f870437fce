"""kda_prefill_no_alloc: the entry point for callers that cannot allocate device memory
takes its workspace from the library's static device scratch (KDA_NO_ALLOC_SCRATCH_BYTES
per device). It must give bitwise the results of kda_prefill with a caller-allocated
workspace (same kernels, same workspace layout), also on a second call that reuses the
scratch with a smaller input, and must reject calls whose workspace would not fit before
anything is launched."""

import os

import numpy as np
import pytest

import chunkwise_delta_rule_kda_amd as kda
import kda_synth
from kda_testlib import rel_err, run_oracle, to_device

TOL = 2e-2


def _call(fn, x, **kw):
    import torch

    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    d.update(kw)
    o, s = fn(q, k, v, g, beta, **d)
    torch.cuda.synchronize()
    return o.cpu(), s.cpu()


@pytest.mark.gpu
def test_no_alloc_matches_kda_prefill_on_two_calls():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kda.load_library()
    cases = [
        # the bench workload (segmented form, records and scan slots in the scratch)
        ("config1 full", kda_synth.config(1), {}),
        # then a smaller varlen call with in-kernel transforms (serial form)
        ("varlen small", kda_synth.config(4, H=2, lengths=[100, 37, 0, 60]),
         dict(segment_chunks=-1)),
    ]
    for name, x, kw in cases:
        args = kda.make_args(B=x.B, T=x.T, H=x.H, N=x.N,
                             cu_seqlens=None if x.cu_seqlens is None else 1, **kw)
        need = kda.kda_prefill_workspace_bytes(args)
        print(f"[no_alloc] {name}: T={x.T} H={x.H} N={x.N} workspace {need} bytes", flush=True)
        assert 0 < need <= kda.KDA_NO_ALLOC_SCRATCH_BYTES
        o1, s1 = _call(kda.kda_prefill_no_alloc, x, **kw)
        o2, s2 = _call(kda.kda_prefill, x, **kw)
        assert torch.equal(o1, o2) and torch.equal(s1, s2), name
        o_ref, s_ref = run_oracle(x)
        eo = rel_err(o1.float().numpy(), o_ref)
        es = rel_err(s1.float().numpy(), s_ref)
        print(f"[no_alloc] {name}: o err {eo:.3e} state err {es:.3e}", flush=True)
        assert eo <= TOL and es <= TOL


def test_no_alloc_rejects_calls_beyond_the_scratch():
    if not os.path.exists(kda.lib_path()):
        pytest.skip("libkda.so not built")
    lib = kda.load_library()
    import ctypes

    # H = 12, T = 8192 with the separate preparation kernel needs ~85 MB of records:
    # rejected before any pointer is used or any kernel launched (the pointers here are
    # never dereferenced).
    a = kda.make_args(B=1, T=8192, H=12, N=1, q=1 << 20, k=2 << 20, v=3 << 20, g=4 << 20,
                      beta=5 << 20, o=6 << 20)
    assert kda.kda_prefill_workspace_bytes(a) > kda.KDA_NO_ALLOC_SCRATCH_BYTES
    assert lib.kda_prefill_no_alloc(ctypes.byref(a), None) == 7
    assert "static scratch" in kda.kda_last_error()
    # a caller-supplied workspace is refused too
    b = kda.make_args(B=1, T=64, H=1, N=1, workspace=7 << 20, workspace_bytes=1 << 20)
    assert lib.kda_prefill_no_alloc(ctypes.byref(b), None) == 7
