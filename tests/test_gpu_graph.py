"""kda_prefill under HIP graph capture (the flashinfer page, section "State and graph
semantics": capture needs caller-owned workspace and preallocated outputs). The library
allocates nothing and never synchronises inside a call, so a captured call replays the
same kernels: every replay, with eager work and synchronisation between replays, must
equal the eager result bitwise (the kernels are deterministic)."""

import numpy as np
import pytest

import kda_synth
from kda_testlib import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_delta_rule_kda_amd as kda

    kda.load_library()


def captured_equals_eager(x, name, **kw):
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    print(f"[case] graph {name}: T={x.T} H={x.H} N={x.N} {kw}", flush=True)
    d = to_device(x)
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    st_in = d.pop("state_in")
    o = torch.empty_like(v)
    st = torch.empty((x.N, x.H, 128, 128), dtype=d["state_dtype"], device="cuda")
    args = kda.make_args(B=x.B, T=x.T, H=x.H, N=x.N, cu_seqlens=d.get("cu_seqlens"),
                         segment_chunks=kw.get("segment_chunks", 0),
                         checkpoint_every=kw.get("checkpoint_every", 0))
    ws = torch.empty(max(1, kda.kda_prefill_workspace_bytes(args)), dtype=torch.uint8,
                     device="cuda")
    extra = dict(kw)
    if kw.get("checkpoint_every"):
        every = kw["checkpoint_every"]
        cu = np.asarray(x.cu_seqlens) if x.cu_seqlens is not None else np.arange(x.B + 1) * x.T
        counts = [(int(b - a) + every - 1) // every for a, b in zip(cu[:-1], cu[1:])]
        starts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        extra["checkpoint_cu_starts"] = torch.from_numpy(starts).cuda()
        extra["state_checkpoints"] = torch.empty((int(starts[-1]), x.H, 128, 128),
                                                 dtype=d["state_dtype"], device="cuda")
    run = lambda: kda.kda_prefill(q, k, v, g, beta, st_in, o=o, state_out=st, workspace=ws,
                                  **d, **extra)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, st) + ((extra["state_checkpoints"],)
                                         if "state_checkpoints" in extra else ())]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for i in range(3):
        o.zero_()
        st.zero_()
        scratch = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (o, st) + ((extra["state_checkpoints"],) if "state_checkpoints" in extra else ())
        for a, b in zip(got, ref):
            assert torch.equal(a, b), (name, i)
        del scratch


def test_graph_serial():
    captured_equals_eager(kda_synth.config(2, T=300, H=3), "serial", segment_chunks=-1)


def test_graph_segmented():
    captured_equals_eager(kda_synth.stress("weak_decay", T=1024, H=2), "segmented",
                          segment_chunks=8)


def test_graph_varlen_checkpoints():
    x = kda_synth.config(4, H=2, lengths=[40, 0, 70, 9])
    captured_equals_eager(x, "varlen checkpoints", segment_chunks=2, checkpoint_every=32)
