"""The C-ABI library loads, exports every declared symbol, and its host-side validation
rejects what the contract forbids (CPU only: no HIP call is made; pointers are fake)."""

import os
import re
import subprocess

import pytest

import chunkwise_delta_rule_kda_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kda.lib_path()),
                                reason="libkda.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["kda_prefill", "kda_prefill_workspace_bytes", "kda_prefill_check",
              "kda_status_string", "kda_last_error", "kda_debug_check_cu_seqlens",
              "kda_prefill_plan", "kda_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", kda.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    lib = kda.load_library()
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_record_size_matches_header():
    m = re.search(r"#define KDA_WS_RECORD (\d+)", open(HEADER).read())
    assert int(m.group(1)) == kda.KDA_WS_RECORD


def test_abi_version_and_status_strings():
    lib = kda.load_library()
    assert lib.kda_abi_version() == 7
    for code in range(11):
        assert kda.kda_status_string(code) and kda.kda_status_string(code) != "unknown status"
    assert kda.kda_status_string(99) == "unknown status"


MB = 1 << 20


def fake(B=1, T=64, H=2, N=None, varlen=False, io=kda.KDA_BF16, st=kda.KDA_BF16, **kw):
    """Args with fake, disjoint, aligned device addresses (never dereferenced)."""
    base = 0x7F0000000000
    slot = lambda i: base + i * 256 * MB
    N = (B if not varlen else 3) if N is None else N
    d = dict(q=slot(0), k=slot(1), v=slot(2), g=slot(3), beta=slot(4), state_in=slot(5),
             o=slot(6), state_out=slot(7), workspace=slot(8), workspace_bytes=200 * MB,
             B=B, T=T, H=H, N=N, io_dtype=io, state_dtype=st)
    if varlen:
        d["cu_seqlens"] = slot(9)
    d.update(kw)
    return kda.make_args(**d)


def status(a):
    return kda.kda_prefill_check(a)


def test_valid_args_pass():
    assert status(fake()) == 0
    assert status(fake(varlen=True)) == 0
    assert status(fake(io=kda.KDA_FP32, st=kda.KDA_FP32)) == 0
    assert status(fake(state_in=None)) == 0          # zero initial state
    assert status(fake(state_out=None)) == 0         # no final state
    assert status(fake(state_out=0x7F0000000000 + 5 * 256 * MB)) == 0  # in place


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "beta", "o"])
def test_null_required_pointer(field):
    assert status(fake(**{field: None})) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), 2), (dict(H=0), 2), (dict(T=-1), 2), (dict(B=2, N=3), 2),
    (dict(io_dtype=7), 3), (dict(state_dtype=-1), 3),
    (dict(flags=1 << 5), 4), (dict(rows_per_workgroup=24), 10),
    (dict(scale=float("nan")), 5),
    # sizes bounded before any arithmetic on them (no signed overflow)
    (dict(T=(1 << 40) + 1), 2), (dict(T=(1 << 63) - 1), 2), (dict(B=(1 << 31) + 1), 2),
    (dict(H=4096, T=1 << 30, B=1 << 8, N=1 << 8), 2),
    (dict(checkpoint_every=1 << 41), 10), (dict(checkpoint_every=16, checkpoint_rows=1 << 41), 10),
])
def test_shape_dtype_flag_rejections(kw, code):
    assert status(fake(**kw)) == code


def test_varlen_needs_batch_one():
    assert status(fake(B=2, varlen=True)) == 2


def test_gate_needs_params_and_bound():
    G = kda.KDA_FLAG_GATE_IN_KERNEL
    p = dict(A_log=0x7F0000000000 + 10 * 256 * MB, dt_bias=0x7F0000000000 + 11 * 256 * MB)
    assert status(fake(flags=G, lower_bound=-5.0)) == 4          # no A_log / dt_bias
    assert status(fake(flags=G, lower_bound=-5.0, **p)) == 0
    assert status(fake(flags=G, lower_bound=-0.1, **p)) == 0
    # The flashinfer page's accepted range is [-5, 0): the cliff near -5.4585 is outside.
    for lb in (-5.4585, -5.0001, 0.0, 0.5, float("nan")):
        assert status(fake(flags=G, lower_bound=lb, **p)) == 5, lb


def test_aliasing_rejected():
    base = 0x7F0000000000
    assert status(fake(o=base + 1 * 256 * MB)) == 6                 # o == k
    assert status(fake(o=base + 2 * 256 * MB + 4096)) == 6          # o inside v
    assert status(fake(state_out=base + 5 * 256 * MB + 64)) == 6    # partial overlap
    assert status(fake(state_out=base + 0 * 256 * MB)) == 6         # state_out == q
    assert status(fake(workspace=base + 4 * 256 * MB)) == 6         # workspace == beta
    assert status(fake(state_out=base + 6 * 256 * MB)) == 6         # state_out == o


def test_workspace_checks():
    # Separate preparation kernel (the default): ceil(100/16) = 7 chunk records for each
    # of 3 heads, then the 256-byte status block.
    two = dict(fuse_prepare=0)
    need = kda.kda_prefill_workspace_bytes(fake(T=100, H=3, **two))
    assert need == 7 * 3 * kda.KDA_WS_RECORD + 256
    assert status(fake(T=100, H=3, workspace_bytes=need, **two)) == 0
    assert status(fake(T=100, H=3, workspace_bytes=need - 1, **two)) == 7
    assert status(fake(T=100, H=3, workspace=None, **two)) == 7
    assert status(fake(T=100, H=3, workspace=0x7F0000000000 + 8 * 256 * MB + 128, **two)) == 7
    assert kda.kda_prefill_workspace_bytes(fake(T=100, H=3, fuse_prepare=-1)) == need
    # Fused form: no records, only the status block; with KDA_FLAG_KEEP_RECORDS the
    # records too.
    assert kda.kda_prefill_workspace_bytes(fake(T=100, H=3, fuse_prepare=1)) == 256
    keep = fake(T=100, H=3, fuse_prepare=1, flags=kda.KDA_FLAG_KEEP_RECORDS)
    assert kda.kda_prefill_workspace_bytes(keep) == 7 * 3 * kda.KDA_WS_RECORD + 256
    p = kda.kda_prefill_plan(keep)
    assert p["fused"] == 1 and p["has_records"] == 1 and p["records_offset"] == 0
    assert p["status_offset"] == 7 * 3 * kda.KDA_WS_RECORD
    # varlen: (T + 15 N) / 16 chunk records after the 256-byte-rounded header
    # (cu_chunks, cu_segs, order)
    v = fake(T=100, H=3, N=5, varlen=True, **two)
    assert kda.kda_prefill_workspace_bytes(v) == 256 + ((100 + 15 * 5) // 16) * 3 * kda.KDA_WS_RECORD + 256
    assert kda.kda_prefill_workspace_bytes(fake(T=100, H=3, N=5, varlen=True,
                                                fuse_prepare=1)) == 256 + 256


def test_checkpoint_validation():
    base = 0x7F0000000000
    ck = dict(checkpoint_every=32, checkpoint_rows=4, state_checkpoints=base + 10 * 256 * MB,
              checkpoint_cu_starts=base + 11 * 256 * MB)
    assert status(fake(**ck)) == 0
    assert status(fake(**dict(ck, checkpoint_every=8))) == 10      # not a multiple of 16
    assert status(fake(**dict(ck, checkpoint_every=-16))) == 10
    assert status(fake(**dict(ck, checkpoint_rows=-1))) == 10
    assert status(fake(**dict(ck, state_checkpoints=None))) == 1
    # No rows: nothing is written, so a NULL buffer (a zero-size tensor's pointer) is fine;
    # the row offsets are still required.
    assert status(fake(**dict(ck, checkpoint_rows=0, state_checkpoints=None))) == 0
    assert status(fake(**dict(ck, checkpoint_rows=0, state_checkpoints=None,
                              checkpoint_cu_starts=None))) == 1
    assert status(fake(**dict(ck, checkpoint_cu_starts=None))) == 1
    assert status(fake(**dict(ck, state_checkpoints=base + 10 * 256 * MB + 8))) == 2
    assert status(fake(**dict(ck, state_checkpoints=base + 2 * 256 * MB))) == 6   # == v
    assert status(fake(**dict(ck, state_checkpoints=base + 6 * 256 * MB))) == 6   # == o
    assert status(fake(**dict(ck, checkpoint_cu_starts=base + 10 * 256 * MB))) == 6
    # Off: the checkpoint pointers are ignored.
    assert status(fake(checkpoint_every=0, state_checkpoints=base + 2 * 256 * MB)) == 0


def test_state_pool_and_order_validation():
    base = 0x7F0000000000
    dense = 2 * 128 * 128
    pool = dict(ssm_state_indices=base + 12 * 256 * MB, state_pool_slots=5, state_out=None)
    assert status(fake(**pool)) == 0
    assert status(fake(**dict(pool, state_slot_pitch=dense + 64))) == 0
    assert status(fake(**dict(pool, state_out=base + 5 * 256 * MB))) == 0   # == state_in
    assert status(fake(**dict(pool, state_out=base + 7 * 256 * MB))) == 6   # elsewhere
    assert status(fake(**dict(pool, state_in=None))) == 10
    assert status(fake(**dict(pool, state_pool_slots=0))) == 10
    assert status(fake(**dict(pool, state_slot_pitch=dense - 8))) == 10
    assert status(fake(**dict(pool, state_slot_pitch=dense + 4))) == 10
    assert status(fake(**dict(pool, ssm_state_indices=base + 6 * 256 * MB))) == 6  # == o
    assert status(fake(seq_order=base + 13 * 256 * MB)) == 0
    assert status(fake(seq_order=base + 6 * 256 * MB)) == 6                     # == o


def test_misaligned_vector_pointer_rejected():
    assert status(fake(q=0x7F0000000000 + 8)) == 2


def test_plan_follows_the_slice_rule():
    # Smallest slice keeping N*H*(128/rows) within the compute units, 16 rows per wave.
    assert kda.kda_prefill_plan(fake(H=6), 256)["rows_per_workgroup"] == 16
    assert kda.kda_prefill_plan(fake(H=12), 256)["rows_per_workgroup"] == 16
    assert kda.kda_prefill_plan(fake(H=48), 256)["rows_per_workgroup"] == 32
    p = kda.kda_prefill_plan(fake(H=96, T=8192), 256)
    assert p["rows_per_workgroup"] == 64 and p["recurrence_workgroups"] == 192
    assert p["prepare_workgroups"] == 512 * 96 and p["fused"] == 0
    f = kda.kda_prefill_plan(fake(H=96, T=8192, fuse_prepare=1), 256)
    assert f["prepare_workgroups"] == 0 and f["fused"] == 1  # prepared in the recurrence
    assert f["waves_per_workgroup"] == 4 + 4  # compute waves and producer waves
    # Past one round of 64-row slices, whole heads (BF16 I/O): 8 x 24 pairs.
    v = kda.kda_prefill_plan(fake(H=24, T=20000, N=8, varlen=True), 256)
    assert v["rows_per_workgroup"] == 128 and v["waves_per_workgroup"] == 12
    f32 = kda.kda_prefill_plan(fake(H=24, T=20000, N=8, varlen=True, io=kda.KDA_FP32), 256)
    assert f32["rows_per_workgroup"] == 64
    # serial grid: whole rounds of 8 (sequence, head) pairs, each with its row blocks
    assert kda.kda_prefill_plan(fake(H=6, rows_per_workgroup=64), 256)["recurrence_workgroups"] == 16
    assert status(fake(rows_per_workgroup=128)) == 0
    assert status(fake(rows_per_workgroup=48)) == 10
    assert status(fake(rows_per_workgroup=256)) == 10


def test_plan_segments_small_head_counts():
    # H = 6, T = 8192: 512 chunks. Affine-output form (no checkpoints), 64-row
    # workgroups: launch A has 2 (2 P - 1) workgroups per pair, so
    # P = (256 / 12 + 1) / 2 = 11 segments of 47 chunks.
    p = kda.kda_prefill_plan(fake(H=6, T=8192), 256)
    assert p["segment_chunks"] == 47 and p["segments_per_head_bound"] == 11
    assert p["rows_per_workgroup"] == 64 and p["scan_affine_output"] == 1
    # Active row blocks of 64 rows only: segment 0's value rows, then value (Z) and
    # transition (Phi) rows of segments 1 .. 10; with ten later segments the
    # carry-and-output launch (four 32-row blocks per later segment) replaces the
    # combine and the scan output.
    assert p["recurrence_workgroups"] == 6 * (2 + 4 * 10)
    assert p["scan_c_workgroups"] == 6 * 10 * 4
    assert p["combine_workgroups"] == 0
    # From ten pairs on, 128-row segments: H = 12 gets P = (256 / 12 + 1) / 2 = 11
    # segments of 47 chunks and the carry-and-output launch; H = 24 P = 5 segments of 103
    # chunks, four later ones: the combine (8 row blocks x 24 pairs) and the scan output
    # (groups of 4 chunks).
    p12 = kda.kda_prefill_plan(fake(H=12, T=8192), 256)
    assert p12["segment_chunks"] == 47 and p12["rows_per_workgroup"] == 128
    assert p12["recurrence_workgroups"] == 12 * (1 + 2 * 10)
    assert p12["combine_workgroups"] == 0 and p12["scan_c_workgroups"] == 12 * 10 * 4
    p24 = kda.kda_prefill_plan(fake(H=24, T=8192), 256)
    assert p24["segment_chunks"] == 103 and p24["rows_per_workgroup"] == 128
    assert p24["combine_workgroups"] == 192
    assert p24["scan_c_workgroups"] == 24 * 4 * ((103 + 3) // 4)
    # The carry-and-output launch needs six later segments, and nine when its grid
    # (H x later x 4 workgroups) exceeds 256: H = 8 (64-row, 7 later, 224) and H = 13
    # (128-row, 9 later, 468) take it, H = 14 (8 later, 448) keeps the combine.
    for H, later, carry in ((8, 7, True), (13, 9, True), (14, 8, False), (18, 6, False)):
        ph = kda.kda_prefill_plan(fake(H=H, T=8192), 256)
        assert -(-512 // ph["segment_chunks"]) - 1 == later, H
        assert (ph["combine_workgroups"] == 0) == carry, H
    # The fused form keeps 64-row segments up to 32 pairs: H = 24, P = (256 / 48 + 1) / 2
    # = 3 segments of 171 chunks; H = 48 takes 128 rows like the two-kernel form.
    f24 = kda.kda_prefill_plan(fake(H=24, T=8192, fuse_prepare=1), 256)
    assert f24["rows_per_workgroup"] == 64 and f24["segment_chunks"] == 171
    f48 = kda.kda_prefill_plan(fake(H=48, T=8192, fuse_prepare=1), 256)
    assert f48["rows_per_workgroup"] == 128 and f48["segment_chunks"] == 171
    # Nine pairs keep 64-row segments: P = (256 / 18 + 1) / 2 = 7.
    p9 = kda.kda_prefill_plan(fake(H=9, T=8192), 256)
    assert p9["rows_per_workgroup"] == 64 and p9["segment_chunks"] == 74
    records = 512 * 6 * kda.KDA_WS_RECORD
    assert p["scan_state_offset"] == records            # already 256-byte aligned
    slots = 6 * 11
    assert p["scan_transition_offset"] == records + slots * 128 * 128 * 4
    assert p["scan_output_offset"] == records + slots * 128 * 128 * 6
    need = kda.kda_prefill_workspace_bytes(fake(H=6, T=8192))
    assert need == records + slots * 128 * 128 * 6 + 512 * 6 * 2048 * 2 + 256
    # the fused form keeps no records: the scan slots come first
    fp = kda.kda_prefill_plan(fake(H=6, T=8192, fuse_prepare=1), 256)
    assert fp["scan_state_offset"] == 0 and fp["has_records"] == 0
    assert kda.kda_prefill_workspace_bytes(fake(H=6, T=8192, fuse_prepare=1)) == need - records
    # With checkpoints every later segment is re-run: 2 (2 P - 3) workgroups per pair in
    # launch A, P = (256 / 12 + 3) / 2 = 12 segments of 43 chunks.
    c = kda.kda_prefill_plan(fake(H=6, T=8192, checkpoint_every=1024), 256)
    assert c["segment_chunks"] == 43 and c["segments_per_head_bound"] == 12
    assert c["scan_affine_output"] == 0 and c["scan_output_offset"] == 0
    assert c["recurrence_workgroups"] == 6 * (2 + 4 * 10)
    assert c["scan_c_workgroups"] == 6 * 11 * 2
    assert c["combine_workgroups"] == 64  # 8 row blocks x 6 pairs, padded to 8 XCDs
    # 128-row workgroups when asked for: 2 P - 1 per pair, P = (256 / 6 + 1) / 2 = 21.
    w = kda.kda_prefill_plan(fake(H=6, T=8192, rows_per_workgroup=128), 256)
    assert w["segment_chunks"] == 25 and w["segments_per_head_bound"] == 21
    assert w["rows_per_workgroup"] == 128 and w["waves_per_workgroup"] == 8 + 4
    assert w["recurrence_workgroups"] == 6 * (1 + 2 * 20)
    # Past 32 pairs (BF16 I/O, 128-row workgroups as from 10 pairs on) the automatic
    # segments need three segments: H = 48 (P = 3) is segmented, H = 64 (P = 2) and
    # H = 96 are not; with FP32 I/O (64-row) H = 48 stays serial.
    h48 = kda.kda_prefill_plan(fake(H=48, T=8192), 256)
    assert h48["segment_chunks"] == 171 and h48["rows_per_workgroup"] == 128
    assert h48["recurrence_workgroups"] == 48 * 5
    assert kda.kda_prefill_plan(fake(H=64, T=8192), 256)["segment_chunks"] == 0
    assert kda.kda_prefill_plan(fake(H=48, T=8192, io=kda.KDA_FP32), 256)["segment_chunks"] == 0
    # Forced serial, forced length, and no segments for many heads.
    s = kda.kda_prefill_plan(fake(H=6, T=8192, segment_chunks=-1), 256)
    assert s["segment_chunks"] == 0 and s["rows_per_workgroup"] == 16
    assert kda.kda_prefill_workspace_bytes(fake(H=6, T=8192, segment_chunks=-1)) == records + 256
    f = kda.kda_prefill_plan(fake(H=6, T=8192, segment_chunks=100), 256)
    assert f["segment_chunks"] == 100 and f["segments_per_head_bound"] == 6
    assert kda.kda_prefill_plan(fake(H=96, T=8192), 256)["segment_chunks"] == 0
    # Varlen: slots bound = ceil(max_chunks / L) + N.
    v = kda.kda_prefill_plan(fake(H=2, T=4000, N=3, varlen=True, segment_chunks=20), 256)
    mc = (4000 + 15 * 3) // 16
    assert v["segments_per_head_bound"] == (mc + 19) // 20 + 3
    bound = v["segments_per_head_bound"]
    assert v["recurrence_workgroups"] == 2 * bound * 4
    assert v["scan_c_workgroups"] == 2 * bound * ((20 + 3) // 4)
    assert v["workspace_header_bytes"] == 256
    # header: cu_chunks and cu_segs (int64 [N + 1]) and the automatic order (int32 [N])
    big = kda.kda_prefill_plan(fake(H=2, T=4000, N=100, varlen=True), 256)
    assert big["workspace_header_bytes"] == ((101 * 16 + 100 * 4 + 255) // 256) * 256
    assert status(fake(segment_chunks=1 << 25)) == 10


def test_last_error_explains_rejection():
    assert status(fake(D=64)) == 2
    assert "128" in kda.kda_last_error()
