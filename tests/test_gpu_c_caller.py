"""The C ABI from C: tests/c_caller/kda_c_caller.c (plain C against include/kda.h and the
HIP runtime, no Python or PyTorch in the process) runs one prefill from raw BF16 input
files. Its outputs must be bitwise those of the Python binding on the same inputs (the
same library, called through the same ABI), and within the parity bound of the FP64
oracle (max|err| / max|ref| <= 2e-2)."""

import os
import subprocess

import numpy as np
import pytest

import kda_synth
from kda_testlib import bf16_bits_to_f32, rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_caller", "kda_c_caller")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()
    if not os.path.exists(EXE):  # normally built by __graft_entry__.build()
        from chunkwise_delta_rule_kda_amd.csrc import build

        build.build_c_caller()


def _bf16_bits(a):
    """Values exact in BF16 (float32 arrays) as their 16-bit patterns."""
    return (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("T,H", [(300, 3), (8192, 6)])
def test_c_client_matches_python_binding_and_oracle(tmp_path, T, H):
    x = kda_synth.config(2, T=T, H=H)  # BF16, nonzero initial state
    assert x.dtype == "bf16" and x.state_dtype == "bf16"
    for name, arr in (("q", x.q), ("k", x.k), ("v", x.v), ("g", x.g), ("beta", x.beta),
                      ("state_in", x.state0)):
        _bf16_bits(arr).tofile(str(tmp_path / f"{name}.bin"))
    print(f"[c_caller] T={T} H={H}", flush=True)
    run = subprocess.run([EXE, str(tmp_path), str(T), str(H)], capture_output=True, text=True,
                         timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    o_c = bf16_bits_to_f32(np.fromfile(str(tmp_path / "o.bin"), np.uint16)).reshape(x.q.shape)
    s_c = bf16_bits_to_f32(np.fromfile(str(tmp_path / "state_out.bin"), np.uint16)).reshape(
        x.state0.shape)
    o_py, s_py, _ = run_gpu(x)
    assert np.array_equal(o_c.astype(np.float64), o_py)
    assert np.array_equal(s_c.astype(np.float64), s_py)
    heads = None if H <= 3 else [0, H - 1]
    o_ref, s_ref = run_oracle(x, heads=heads)
    hs = slice(None) if heads is None else heads
    assert rel_err(o_c[:, :, hs], o_ref) <= 2e-2
    assert rel_err(s_c[:, hs], s_ref) <= 2e-2
