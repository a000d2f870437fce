"""The prepared per-chunk records vs the oracle's literal chunk quantities, from both
places the preparation runs: the separate kda_prepare kernel (fuse_prepare < 0) and the
producer waves of the fused recurrence (which write what they put in the LDS ring to the
workspace when KDA_FLAG_KEEP_RECORDS is set).

After such a call the caller-owned workspace holds one record per (chunk, head) in the
layout documented in include/kda.h. Each record is decoded here and compared with the folded
quantities built from ``oracle.chunk_quantities`` (the page's K_start, Q_start, K_end,
D_{0:15}, A_kk, A_qk) by the algebra the header states:
Mb = A_kk Diag(beta), Kn = -Mb K_start^T, Qt = s Q_start^T + A_qk Kn.
Pad tokens of a short last chunk are k = q = 0, g = 0, beta = 0.

Errors are max|err| / max|ref| per record, except for A_qk: its entries are s-scaled inner
products s * sum_c Q_start_i[c] k_j[c] / Gamma_j[c] with j <= i, where the decay ratio is
at most 1, so |A_qk[i, j]| <= s |q_i| |k_j|, and the BF16 operands' error scales with that
bound, not with the entry. A chunk whose few entries all nearly cancel (a one-token chunk
with q . k close to 0) is therefore judged against max(max|ref|, s max_i |q_i| max_j |k_j|).
"""

import numpy as np
import pytest

import kda_synth
from kda_testlib import bf16_bits_to_f32, rel_err, to_device
from oracle import chunk_quantities, l2_normalize, safe_gate, sigmoid

pytestmark = pytest.mark.gpu

REC = 13824


def kappa(kb, grp, e):
    return 32 * kb + 16 * (e // 4) + 4 * grp + (e % 4)


def decode(rec):
    """One record (uint8[13824]) -> dict of float arrays in natural layouts."""
    u16 = rec.view(np.uint16)
    kn = bf16_bits_to_f32(u16[0:2048]).reshape(4, 64, 8)
    qt = bf16_bits_to_f32(u16[2048:4096]).reshape(4, 64, 8)
    ke = bf16_bits_to_f32(u16[4096:6144]).reshape(4, 64, 2, 4)
    D = rec[12288:12800].view(np.float32).reshape(64, 2)
    ma = bf16_bits_to_f32(u16[6400:6912]).reshape(64, 2, 4)
    Kn = np.zeros((16, 128)); Qt = np.zeros((16, 128)); Ke = np.zeros((16, 128))
    M = np.zeros((16, 16)); A = np.zeros((16, 16)); Dn = np.zeros(128)
    for L in range(64):
        m, grp = L % 16, L // 16
        for kb in range(4):
            for e in range(8):
                Kn[m, kappa(kb, grp, e)] = kn[kb, L, e]
                Qt[m, kappa(kb, grp, e)] = qt[kb, L, e]
        for bp in range(4):
            for h in range(2):
                for j in range(4):
                    Ke[4 * grp + j, 16 * (2 * bp + h) + m] = ke[bp, L, h, j]
        for c in range(2):
            Dn[16 * (m // 2) + 4 * grp + 2 * (m % 2) + c] = D[L, c]
        for j in range(4):
            M[m, 4 * grp + j] = ma[L, 0, j]
            A[m, 4 * grp + j] = ma[L, 1, j]
    return dict(Kn=Kn, Qt=Qt, K_end=Ke, D=Dn, Mb=M, A_qk=A)


def expected(q, k, g, beta, s):
    """Folded record from the oracle's chunk quantities (chunk padded to 16 tokens)."""
    r = q.shape[0]
    pad = lambda a: np.concatenate([a, np.zeros((16 - r,) + a.shape[1:])], 0)
    q, k, g, beta = pad(q), pad(k), pad(g), pad(beta)
    w = chunk_quantities(q, k, g, beta, s)
    Mb = w["A_kk"] @ np.diag(beta)
    Kn = -Mb @ w["K_start"].T
    Qt = s * w["Q_start"].T + w["A_qk"] @ Kn
    return dict(Kn=Kn, Qt=Qt, K_end=w["K_end"], D=w["D_total"], Mb=Mb, A_qk=w["A_qk"])


TOLS = dict(Kn=1e-2, Qt=1e-2, K_end=1e-2, D=1e-5, Mb=1e-2, A_qk=1e-2)


MODES = {"separate": dict(fuse_prepare=-1), "fused": dict(fuse_prepare=1, keep_records=True)}


def run_and_check(x, mode, chunks_to_check=None, tols=TOLS):
    import torch

    import chunkwise_delta_rule_kda_amd as kda

    d = to_device(x)
    kw = MODES[mode]
    args = kda.make_args(B=x.B, T=x.T, H=x.H, N=x.N, cu_seqlens=d.get("cu_seqlens"),
                         fuse_prepare=kw.get("fuse_prepare", 0),
                         flags=kda.KDA_FLAG_KEEP_RECORDS if kw.get("keep_records") else 0)
    need = kda.kda_prefill_workspace_bytes(args)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    q, k, v, g, beta = (d.pop(n) for n in ("q", "k", "v", "g", "beta"))
    kda.kda_prefill(q, k, v, g, beta, workspace=ws, **kw, **d)
    torch.cuda.synchronize()
    wsn = ws.cpu().numpy()
    plan = kda.kda_prefill_plan(args)
    assert plan["has_records"] == 1 and plan["fused"] == (mode == "fused")
    header = plan["records_offset"]
    status = wsn[plan["status_offset"]:plan["status_offset"] + 4].view(np.int32)[0]
    assert status == 0, status
    max_chunks = (x.N * ((x.T + 15) // 16) if x.cu_seqlens is None
                  else (x.T + 15 * x.N) // 16)
    # Oracle-side inputs after the in-kernel transforms (FP64).
    q64, k64, g64, b64 = (np.asarray(a, np.float64) for a in (x.q, x.k, x.g, x.beta))
    if x.l2norm_qk:
        q64, k64 = l2_normalize(q64), l2_normalize(k64)
    if x.A_log is not None:
        g64 = safe_gate(g64, x.A_log, x.dt_bias, x.lower_bound)
    if x.beta_is_logit:
        b64 = sigmoid(b64)
    bounds = ([(b * x.T, (b + 1) * x.T) for b in range(x.B)] if x.cu_seqlens is None
              else list(zip(x.cu_seqlens[:-1], x.cu_seqlens[1:])))
    flat = lambda a: a.reshape((x.B * x.T,) + a.shape[2:])
    q64, k64, g64, b64 = flat(q64), flat(k64), flat(g64), flat(b64)
    gc = 0
    worst = {n: 0.0 for n in TOLS}
    for (a, b) in bounds:
        for c0 in range(int(a), int(b), 16):
            sl = slice(c0, min(c0 + 16, int(b)))
            if chunks_to_check is None or gc in chunks_to_check:
                for h in range(x.H):
                    off = header + (h * max_chunks + gc) * REC
                    got = decode(wsn[off:off + REC])
                    ref = expected(q64[sl, h], k64[sl, h], g64[sl, h], b64[sl, h], x.scale)
                    for n in TOLS:
                        if n == "A_qk":
                            bound = (abs(x.scale) * np.linalg.norm(q64[sl, h], axis=1).max()
                                     * np.linalg.norm(k64[sl, h], axis=1).max())
                            den = max(np.abs(ref[n]).max(), bound)
                            err = np.abs(got[n] - ref[n]).max()
                            e = err / den if den > 0 else err  # q or k all zero: exact 0
                        else:
                            e = rel_err(got[n], ref[n])
                        worst[n] = max(worst[n], e)
            gc += 1
    print(f"[prepare] {mode} worst relative errors:", {n: f"{e:.2e}" for n, e in worst.items()},
          flush=True)
    for n, e in worst.items():
        assert e <= tols[n], (n, e)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("mode", sorted(MODES))
def test_prepare_config0_fp32(mode):
    run_and_check(kda_synth.config(0), mode)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_prepare_bf16_ragged(mode):
    run_and_check(kda_synth.config(1, T=93, H=2), mode)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_prepare_varlen_transforms(mode):
    run_and_check(kda_synth.config(4, H=2, lengths=[20, 0, 33, 5]), mode)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_prepare_floor_decay(mode):
    # g = -5 everywhere: exp(+-G) spans e^{+-80}, the split-exponent's widest range.
    run_and_check(kda_synth.stress("floor", T=48, H=1), mode)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_prepare_correlated_keys(mode):
    # Identical keys, weak decay, beta 0.5: (I + R)^{-1} has entries up to ~1e1.
    run_and_check(kda_synth.stress("correlated", T=32, H=1), mode,
                  tols=dict(TOLS, Kn=2e-2, Qt=2e-2, Mb=2e-2))


def test_prepare_heads_fast_grid_fixed():
    # From H = 32 on, the preparation grid puts the heads of a chunk side by side, in
    # rows of 64 chunks. Two sequences of 66 chunks (the last of 10 tokens) are 132
    # chunks: three grid rows, the last one mostly idle. Checked: every head of the
    # chunks at the row seams, the sequence seam and the ragged chunks.
    x = kda_synth.config(1, T=1050, H=32, B=2)
    run_and_check(x, "separate", chunks_to_check={0, 1, 63, 64, 65, 66, 127, 128, 131})


def test_prepare_heads_fast_grid_varlen():
    # Packed sequences with the in-kernel transforms at H = 32: 44 + 0 + 3 + 33 + 16 = 96
    # chunks under a bound of 98, two grid rows; the workgroups past the last real
    # chunk exit.
    x = kda_synth.config(4, H=32, lengths=[700, 0, 33, 513, 250])
    run_and_check(x, "separate", chunks_to_check={0, 43, 44, 46, 47, 63, 64, 79, 80, 95})
