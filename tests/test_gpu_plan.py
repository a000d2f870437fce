"""Bit-exact check of the varlen plan kernel's integer outputs (GPU).

The plan kernel writes, at the start of the workspace (layout in include/kda.h): the
compact chunk prefix cu_chunks[N + 1] of ceil(len_n / 16) (the "flashinfer.kda_prefill"
page, section "Packed scheduling"), in the segmented form the prefix cu_segs[N + 1] of
max(1, ceil(chunks_n / segment_chunks)), and in the serial form without a caller's
seq_order and with N <= 256 the sequences by decreasing chunk count, ties by index. The
test reads them back and compares them with prefixes computed here, integer for integer,
on lengths with empty sequences and ties, and with N past one 256-thread block of the
kernel's scan (N = 300, where no automatic order is written, and N = 1000).
"""

import numpy as np
import pytest

import kda_synth
from kda_testlib import rel_err, run_oracle, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 0xAB


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def expected(lengths, seg_len):
    chunks = [(n + 15) // 16 for n in lengths]
    cu_chunks = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    segs = [max(1, (c + seg_len - 1) // seg_len) if seg_len > 0 else 0 for c in chunks]
    cu_segs = np.concatenate([[0], np.cumsum(segs)]).astype(np.int64)
    order = sorted(range(len(lengths)), key=lambda i: (-chunks[i], i))
    return cu_chunks, cu_segs, np.asarray(order, np.int32)


def run_with_workspace(x, segment_chunks):
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    args = kda.make_args(B=1, T=x.T, H=x.H, N=x.N, cu_seqlens=d["cu_seqlens"],
                         segment_chunks=segment_chunks)
    plan = kda.kda_prefill_plan(args)
    need = kda.kda_prefill_workspace_bytes(args)
    ws = torch.full((need,), SENTINEL, dtype=torch.uint8, device="cuda")
    o, s = kda.kda_prefill(q, k, v, g, beta, workspace=ws, segment_chunks=segment_chunks,
                           **d)
    torch.cuda.synchronize()
    head = ws[:plan["workspace_header_bytes"]].cpu().numpy()
    return plan, head, o, s


def decode(head, N):
    cu_chunks = head[:8 * (N + 1)].view(np.int64)
    cu_segs = head[8 * (N + 1):16 * (N + 1)].view(np.int64)
    order_bytes = head[16 * (N + 1):16 * (N + 1) + 4 * N]
    return cu_chunks, cu_segs, order_bytes


LENGTHS = {
    "ties_and_empty": [0, 33, 16, 0, 33, 1, 200, 17, 16, 0, 48, 47],
    "n300": list(np.random.default_rng(31).integers(0, 41, size=300)),
    "n1000": list(np.random.default_rng(32).integers(0, 20, size=1000)),
}


@pytest.mark.parametrize("name", sorted(LENGTHS))
@pytest.mark.parametrize("seg", [-1, 2])
def test_plan_outputs_bit_exact(name, seg):
    lengths = [int(n) for n in LENGTHS[name]]
    N = len(lengths)
    print(f"[plan] {name} N={N} segment_chunks={seg}", flush=True)
    x = kda_synth.config(4, H=1, lengths=lengths)
    plan, head, o, s = run_with_workspace(x, seg)
    ref_chunks, ref_segs, ref_order = expected(lengths, seg if seg > 0 else 0)
    cu_chunks, cu_segs, order_bytes = decode(head, N)
    np.testing.assert_array_equal(cu_chunks, ref_chunks)
    if seg > 0:
        assert plan["segment_chunks"] == seg
        np.testing.assert_array_equal(cu_segs, ref_segs)
    else:
        assert plan["segment_chunks"] == 0
        # cu_segs is not written in the serial form
        assert np.all(head[8 * (N + 1):16 * (N + 1)] == SENTINEL)
    if seg <= 0 and N <= 256:
        np.testing.assert_array_equal(order_bytes.view(np.int32), ref_order)
    else:
        # no automatic order: its bytes are left as they were
        assert np.all(order_bytes == SENTINEL)
    if N <= 300:  # the outputs themselves, against the oracle
        o_ref, s_ref = run_oracle(x)
        on = o.float().cpu().numpy()
        sn = s.float().cpu().numpy()
        assert rel_err(on, o_ref) <= 2e-2 and rel_err(sn, s_ref) <= 2e-2
