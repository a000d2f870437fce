"""Benchmark of the KDA prefill hot path on one MI355X.

One step = one kda_prefill call (every kernel of the path: varlen plan when packed,
preparation, recurrence) over one batch of synthetic inputs already resident in HBM.
Default workload: T = 8192 tokens, H = 6 heads, d = 128, BF16 (one GPU's share of a
96-head model under 16-way head parallelism). Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1] [--no-cpu-baseline]
                    [--extra-configs 2,3] [--calib-copy-mib 1024]

Each timed pass follows an untimed warm-up of at least W calls and at least 100 ms
(--warmup-ms) of them, so that the GPU clocks have reached their sustained-load rate.
The step time comes from the timed calls alone. Per-kernel durations come from a second
pass in which the library records HIP events between its launches on the call's stream;
the stream time of one event record (measured in the same run) is subtracted from each.
"""

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

D = 128
C = 16
# Algorithmic work per token-head (BF16 I/O): q, k, v, g read (4 x 256 B), beta (2 B),
# o written (256 B); plus the 128x128 state read and written per (sequence, head).
BYTES_PER_TOKEN_HEAD_BF16 = 4 * 256 + 2 + 256
STATE_BYTES_BF16 = 2 * D * D * 2
# FLOP per token-head: recurrence 6 d^2 + 4 C d (S K_start, S Q_start, U K_end and the
# two 16x16 products), preparation 2 x 2 C d (R and A_qk as dense 16x16x128 tiles).
FLOP_REC_PER_TOKEN_HEAD = 6 * D * D + 4 * C * D
FLOP_PREP_PER_TOKEN_HEAD = 2 * 2 * C * D
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

KERNEL_SOURCES = ["kda_prepare.hip", "kda_recurrence.hip", "kda_fused.hip", "kda_decode.hip",
                  "kda_device.h", "kda_internal.h", "kda_recurrence_core.h", "kda_producer.h"]


def kernel_hash():
    """Hash of the kernel sources' code: comments and blank space are dropped first, so
    that a comment edit does not orphan the counter profiles taken of the same code."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "chunkwise_delta_rule_kda_amd", "csrc")
    for n in KERNEL_SOURCES:
        with open(os.path.join(d, n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from a committed counter summary, if it matches the current
    kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_source_hash:\s*(\w+)", txt)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not b or m.group(1) != kernel_hash():
        return None
    return float(b.group(1))


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (one instance)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventCreate.restype = ctypes.c_int
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.restype = ctypes.c_int
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventRecord.restype = ctypes.c_int

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            out.append(e.value)
        return out

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


FUSE_PREPARE = 0  # --fuse-prepare


def make_call(x, device, **extra):
    """Device inputs, outputs and workspace for one configuration (allocated once).
    extra: further kda_prefill keyword arguments (launch geometry)."""
    import torch

    extra.setdefault("fuse_prepare", FUSE_PREPARE)

    import chunkwise_delta_rule_kda_amd as kda
    from tests.kda_testlib import to_device

    d = to_device(x, device)
    o = torch.empty_like(d["v"])
    st = torch.empty((x.N, x.H, D, D), dtype=d["state_dtype"], device=device)
    sized = dict(extra)
    if extra.get("state_checkpoints") is not None:  # the size query sees the call's rows
        sized["checkpoint_rows"] = extra["state_checkpoints"].shape[0]
    args = kda.make_args(B=x.B, T=x.T, H=x.H, N=x.N, cu_seqlens=d.get("cu_seqlens"), **sized)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(args), dtype=torch.uint8, device=device)

    def call(trace=None):
        kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"],
                        d.get("cu_seqlens"), scale=x.scale, A_log=d.get("A_log"),
                        dt_bias=d.get("dt_bias"), lower_bound=d.get("lower_bound"),
                        l2norm_qk=x.l2norm_qk, beta_is_logit=x.beta_is_logit,
                        state_dtype=d["state_dtype"], o=o, state_out=st, workspace=ws,
                        trace_events=trace, **extra)

    return call, (o, st)


# GPU clocks ramp up under sustained load: after an idle pause, back-to-back calls take
# about 20-25 ms to reach their steady rate (H=6: 77 -> 71 us per call, H=96: 645 -> 558 us,
# events between calls). The untimed warm-up therefore runs for at least this long, and
# for at least the requested number of calls.
WARMUP_MIN_S = 0.1


def warm_up(fn, warmup, min_s=None):
    """Untimed calls of fn: at least `warmup` of them and at least `min_s` seconds of
    them (the host waits for the GPU every few calls); returns the number made."""
    import torch

    min_s = WARMUP_MIN_S if min_s is None else min_s
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_graph(x, steps, warmup, device):
    """Microseconds per call when one kda_prefill call is captured in a HIP graph and the
    graph is replayed back to back (the capture semantics are covered by the graph tests)."""
    import torch

    call, _ = make_call(x, device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    warm_up(graph.replay, warmup)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        graph.replay()
    s1.record()
    torch.cuda.synchronize()
    us = s0.elapsed_time(s1) / steps * 1e3
    del graph
    return round(us, 2)


def time_config(x, steps, warmup, device, hip, **extra):
    """Three passes over `steps` calls each:
    1. untimed-inside: the calls back to back between two events (the step time);
    2. traced: the library records five events per call between its launches, giving
       the prepare / first recurrence launch / combine / last launch (carry and output,
       or the re-run)
       durations;
    3. calibration: two events recorded back to back, `steps` times. Each traced phase
       spans exactly one event record (its start marker), whose stream time is this
       gap; it is subtracted from every phase."""
    import torch

    call, _ = make_call(x, device, **extra)
    progress(f"warm-up: {warm_up(call, warmup)} calls")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)

    # Events per call: start, after prepare, after the last recurrence launch, after the
    # first recurrence launch, after the segment combine (see kda.h).
    E = 5
    evs = hip.create(E * steps)
    for i in range(steps):
        call(trace=evs[E * i:E * i + E])
    torch.cuda.synchronize()
    ev = lambda i, j: evs[E * i + j]
    raw = lambda a, b: [hip.elapsed_ms(ev(i, a), ev(i, b)) for i in range(steps)]
    prep, rec, rec_a, comb, rec_c = raw(0, 1), raw(1, 2), raw(1, 3), raw(3, 4), raw(4, 2)
    hip.destroy(evs)

    cal = hip.create(2 * steps)
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(steps):
        hip.record(cal[2 * i], stream)
        hip.record(cal[2 * i + 1], stream)
    torch.cuda.synchronize()
    gap = statistics.median(hip.elapsed_ms(cal[2 * i], cal[2 * i + 1]) for i in range(steps))
    hip.destroy(cal)

    # Per-call distribution, each call between two events, one marker subtracted, with
    # warm caches; "flushed": after a 512 MB write between calls (evicts L2 and the 256 MB
    # MALL, and leaves them full of dirty lines that the call's own traffic writes back);
    # "cold": after a 512 MB read between calls (evicts the inputs, leaves clean lines).
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=device)
    flush_f = flush.view(torch.float32)
    sink = torch.zeros(1, dtype=torch.float32, device=device)
    per_call = {}
    for mode in ("warm", "flushed", "cold"):
        ev = hip.create(2 * steps)
        for i in range(steps):
            if mode == "flushed":
                flush.fill_(i & 0xFF)
            elif mode == "cold":
                sink += flush_f.sum()
            hip.record(ev[2 * i], stream)
            call()
            hip.record(ev[2 * i + 1], stream)
        torch.cuda.synchronize()
        us = sorted(max(0.0, hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) - gap) * 1e3
                    for i in range(steps))
        hip.destroy(ev)
        per_call[mode] = dict(median=round(statistics.median(us), 2), min=round(us[0], 2),
                              p90=round(us[min(steps - 1, int(0.9 * steps))], 2))
    del flush, flush_f, sink
    fix = lambda xs: [max(0.0, v - gap) for v in xs]
    # The serial form has no combine or third launch, and the carry-and-output form no
    # combine: such phases hold only markers.
    no_comb = statistics.median(comb) <= 1.5 * gap
    serial = no_comb and statistics.median(rec_c) <= 1.5 * gap
    return dict(ms_per_step=total_ms / steps, wall_s=t_wall, prep_ms=fix(prep),
                rec_ms=[max(0.0, v - 3 * gap) for v in rec],  # ev 1 -> 2 spans three records
                rec_a_ms=fix(rec_a), combine_ms=[0.0] * steps if no_comb else fix(comb),
                rec_c_ms=[0.0] * steps if serial else fix(rec_c), event_gap_ms=gap,
                serial=serial, per_call_us=per_call)


_ORACLE_X = None  # the workload the pool's workers read (inherited through fork)


def _oracle_block(h):
    """One (sequence, head) block of the FP64 oracle: head h of a fixed-layout workload
    with B = 1, the oracle as it stands, on one thread. Returns seconds."""
    from oracle import kda_recurrence_fp64

    x = _ORACLE_X
    sl = lambda a: None if a is None else a[:, :, h:h + 1]
    s0 = None if x.state0 is None else x.state0[:, h:h + 1]
    t = time.perf_counter()
    kda_recurrence_fp64(sl(x.q), sl(x.k), sl(x.v), sl(x.g), x.beta[:, :, h:h + 1],
                        state0=s0, scale=x.scale)
    return time.perf_counter() - t


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass


def host_cores():
    """Cores this process may run on, capped at 16 (the host share of one GPU)."""
    avail = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return avail, max(1, min(avail, cap, 16))


def time_oracle(x, budget_s, max_reps, workers):
    """Wall seconds of the whole workload through the oracle, one (sequence, head) block
    per task on `workers` processes (one BLAS thread each), repeated until about
    budget_s seconds of wall time (at least once). Returns (median wall s, reps, summed
    per-block CPU seconds of one rep)."""
    import multiprocessing as mp

    global _ORACLE_X
    _ORACLE_X = x
    ctx = mp.get_context("fork")
    walls, cpu = [], 0.0
    with ctx.Pool(processes=workers, initializer=_one_thread) as pool:
        while not walls or (sum(walls) < budget_s and len(walls) < max_reps):
            t = time.perf_counter()
            per = pool.map(_oracle_block, range(x.H), chunksize=1)
            walls.append(time.perf_counter() - t)
            cpu = sum(per)
    _ORACLE_X = None
    return statistics.median(walls), len(walls), cpu


def cpu_baseline(x, x_full=None, budget_s=10.0, max_reps=30):
    """The FP64 oracle timed on the host's cores: a process pool over the workload's
    (sequence, head) blocks (heads are independent), one thread per process. The bench
    workload is repeated for about budget_s seconds; x_full (the 96-head workload) is
    timed once in full. A one-process run of the same blocks gives the single-core
    figure."""
    avail, cores = host_cores()
    workers = min(cores, x.H)
    wall, reps, cpu_s = time_oracle(x, budget_s, max_reps, workers)
    th = x.tokens() * x.H
    out = dict(value=round(x.tokens() / wall, 1), unit="tokens/s", cores=workers,
               kind="oracle",
               sample=f"whole {x.name} workload ({x.tokens()} tokens x {x.H} heads), FP64 "
                      f"NumPy token recurrence, one (sequence, head) block per task on "
                      f"{workers} processes (one thread each; {avail} host cores visible, "
                      f"{cores} used at most), median wall time of {reps} runs "
                      f"({wall:.3f} s each)",
               wall_s=round(wall, 4), s_per_token_head=cpu_s / th,
               one_core_tokens_per_s=round(x.tokens() / cpu_s, 1),
               host_cores_visible=avail)
    if x_full is not None:
        workers_f = min(cores, x_full.H)
        wall_f, _, cpu_f = time_oracle(x_full, 0.0, 1, workers_f)
        th_f = x_full.tokens() * x_full.H
        out["full_96_heads"] = dict(
            workload=f"{x_full.name}: T={x_full.T} H={x_full.H}, every head",
            wall_s=round(wall_f, 3), tokens_per_s=round(x_full.tokens() / wall_f, 1),
            cores=workers_f, cpu_s=round(cpu_f, 2), s_per_token_head=cpu_f / th_f)
    return out


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def summarize(x, r):
    th = x.tokens() * x.H
    # Element sizes: FP32 configurations move twice the bytes of the BF16 figures.
    es = 2 if x.dtype == "bf16" else 4
    ess = 2 if x.state_dtype == "bf16" else 4
    state_b = (2 if x.state0 is not None else 1) * x.N * x.H * D * D * ess
    prep_us = statistics.mean(r["prep_ms"]) * 1e3
    rec_us = statistics.mean(r["rec_ms"]) * 1e3
    tot_us = r["ms_per_step"] * 1e3
    alg_bytes = th * BYTES_PER_TOKEN_HEAD_BF16 * es // 2 + state_b
    alg_flop = th * (FLOP_REC_PER_TOKEN_HEAD + FLOP_PREP_PER_TOKEN_HEAD)
    if 1 <= x.T <= 8 and x.cu_seqlens is None:
        # Token-loop form (a decode step or a few draft tokens): one kernel (timed between
        # the first two events), bound by the state read and write.
        return dict(
            us=round(tot_us, 2), tokens_per_s=round(x.tokens() / (tot_us * 1e-6), 1),
            decode_kernel_us=round(prep_us, 2), state_bytes=state_b, alg_bytes=alg_bytes,
            hbm_gbs=round(alg_bytes / (tot_us * 1e-6) / 1e9, 1),
            hbm_frac=round(alg_bytes / (tot_us * 1e-6) / (PEAK_HBM_GBS * 1e9), 5),
            event_marker_us=round(r["event_gap_ms"] * 1e3, 2),
            per_call_us=r["per_call_us"],
        )
    return dict(
        us=round(tot_us, 2), tokens_per_s=round(x.tokens() / (tot_us * 1e-6), 1),
        prepare_us=round(prep_us, 2), recurrence_us=round(rec_us, 2),
        hbm_frac=round(alg_bytes / (tot_us * 1e-6) / (PEAK_HBM_GBS * 1e9), 5),
        mfma_frac=round(alg_flop / (tot_us * 1e-6) / (PEAK_BF16_TFLOPS * 1e12), 5),
        alg_bytes=alg_bytes, alg_flop=alg_flop,
        link_ns=round(rec_us * 1e3 / max(1, (x.T + C - 1) // C), 1) if x.cu_seqlens is None
        else None,
        recurrence_phases_us=dict(
            first=round(statistics.mean(r["rec_a_ms"]) * 1e3, 2),
            combine=round(statistics.mean(r["combine_ms"]) * 1e3, 2),
            last=round(statistics.mean(r["rec_c_ms"]) * 1e3, 2)),
        event_marker_us=round(r["event_gap_ms"] * 1e3, 2),
        per_call_us=r["per_call_us"],
    )


def main():
    global WARMUP_MIN_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed calls before each timed pass (the warm-up also lasts at "
                         "least --warmup-ms)")
    ap.add_argument("--warmup-ms", type=float, default=1e3 * WARMUP_MIN_S,
                    help="minimum duration of each untimed warm-up (clock ramp)")
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--extra-configs", default="0,2,3,4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step line")
    ap.add_argument("--no-head-sweep", action="store_true", help="skip the H=24/48 lines")
    ap.add_argument("--no-fused-lines", action="store_true",
                    help="skip the fused-form lines (fuse_prepare=1 at H=6/24/96)")
    ap.add_argument("--fuse-prepare", type=int, default=0,
                    help="0 automatic, 1 chunk preparation fused into the recurrence, -1 a "
                         "separate preparation kernel")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain device copy of this many MiB first (counter "
                         "calibration for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    WARMUP_MIN_S = max(0.0, args.warmup_ms) / 1e3

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA prefill path has no multi-GPU "
              "component (heads would shard across GPUs with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import chunkwise_delta_rule_kda_amd as kda
    import kda_synth

    global FUSE_PREPARE
    FUSE_PREPARE = args.fuse_prepare
    kda.load_library()
    device = torch.device("cuda:0")
    hip = HipEvents()

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # Achievable HBM bandwidth on this machine: a plain 1 GiB device copy (read + write).
    a = torch.empty(1 << 30, dtype=torch.uint8, device=device).fill_(1)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(5):
        b.copy_(a)
    s1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (1 << 30) / (s0.elapsed_time(s1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    # Achievable dense BF16 MFMA rate on this machine: a plain 8192^3 product by the vendor
    # library (contiguous operands), best of five after warm-up.
    a = torch.randn(8192, 8192, device=device).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=device).to(torch.bfloat16).contiguous()
    for _ in range(3):
        torch.mm(a, b)
    gemm = []
    for _ in range(5):
        s0.record()
        torch.mm(a, b)
        s1.record()
        torch.cuda.synchronize()
        gemm.append(2 * 8192 ** 3 / (s0.elapsed_time(s1) * 1e-3) / 1e12)
    gemm_tflops = max(gemm)
    del a, b
    torch.cuda.empty_cache()

    x = kda_synth.config(args.config)
    r = time_config(x, args.steps, args.warmup, device, hip)
    main_s = summarize(x, r)
    main_s["graph_replay_us"] = time_graph(x, args.steps, args.warmup, device)
    progress(f"config{args.config}: {main_s}")

    # Dominant kernel: the first recurrence launch (the serial chain), the longest launch
    # of the call. It runs once per call in the serial form and in the affine-output
    # segmented form (segment 0, and the zero-start and transition runs of the later
    # segments; the carry-and-output pass is another kernel), the form a call without
    # checkpoints takes. `achieved` charges the path's algorithmic recurrence FLOP (every
    # token-head passes through this launch) to this launch alone;
    # `recurrence_all_launches` charges them to all recurrence launches together.
    launches = 1
    kern_us = statistics.mean(r["rec_a_ms"]) * 1e3
    avg_launch_us = kern_us / launches
    th = x.tokens() * x.H
    rec_flop = th * FLOP_REC_PER_TOKEN_HEAD
    achieved = rec_flop / launches / (avg_launch_us * 1e-6) / 1e12
    workload = f"config{args.config}"
    phases = main_s["recurrence_phases_us"]
    rec_all_us = phases["first"] + phases["combine"] + phases["last"]
    rec_all_tflops = rec_flop / (rec_all_us * 1e-6) / 1e12
    traffic = traffic_from_profiles("kda_recurrence", workload)
    traffic_src = (f"profiles/traffic_kda_recurrence_{workload}.txt, FETCH_SIZE + WRITE_SIZE "
                   f"per launch, counted for kernel_source_hash {kernel_hash()}"
                   if traffic is not None else None)
    roofline = dict(bound="mfma", kernel="kda_recurrence (first recurrence launch)",
                    achieved=round(achieved, 3), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 6),
                    traffic=traffic, traffic_source=traffic_src,
                    hbm_frac_of_traffic=(round(traffic / (avg_launch_us * 1e-6) /
                                               (PEAK_HBM_GBS * 1e9), 5)
                                         if traffic is not None else None),
                    avg_launch_us=round(avg_launch_us, 3), launches_per_call=launches,
                    flop_per_launch=rec_flop / launches,
                    recurrence_all_launches=dict(
                        us=round(rec_all_us, 3), achieved=round(rec_all_tflops, 3),
                        unit="TFLOP/s",
                        frac=round(rec_all_tflops / PEAK_BF16_TFLOPS, 6)))

    per_config = {workload: main_s}
    for c in [int(c) for c in args.extra_configs.split(",") if c.strip()]:
        if c == args.config:
            continue
        xc = kda_synth.config(c)
        per_config[f"config{c}"] = summarize(xc, time_config(xc, max(5, args.steps // 5),
                                                             2, device, hip))
        progress(f"config{c}: {per_config[f'config{c}']}")
        del xc
        torch.cuda.empty_cache()
    # Decode step (one token per sequence, the single-token kernel): B=256 sequences,
    # H=32 heads, BF16 state drawn as config 2's; bound by the state's HBM traffic.
    if not args.no_decode:
        xd = kda_synth.config(2, B=256, T=1, H=32)
        per_config["decode_B256_H32"] = summarize(
            xd, time_config(xd, max(10, args.steps // 2), 3, device, hip))
        progress(f"decode: {per_config['decode_B256_H32']}")
        del xd
        torch.cuda.empty_cache()
        # Verification of 4 draft tokens per sequence, same sizes.
        xd = kda_synth.config(2, B=256, T=4, H=32)
        per_config["draft4_B256_H32"] = summarize(
            xd, time_config(xd, max(10, args.steps // 2), 3, device, hip))
        progress(f"draft4: {per_config['draft4_B256_H32']}")
        del xd
        torch.cuda.empty_cache()
    # The pages' other head counts at T=8192 (config 1's recipe), for the scaling curve.
    if not args.no_head_sweep:
        for hh in (24, 48):
            xh = kda_synth.config(1, H=hh)
            per_config[f"H{hh}_T8192"] = summarize(
                xh, time_config(xh, max(5, args.steps // 5), 2, device, hip))
            progress(f"H={hh}: {per_config[f'H{hh}_T8192']}")
            del xh
            torch.cuda.empty_cache()
    # The fused form (fuse_prepare=1: each chunk prepared by producer waves of the
    # recurrence workgroup into its LDS ring, no record through HBM) at H = 6, 24 and 96,
    # next to the automatic two-kernel form measured above.
    if not args.no_fused_lines and args.fuse_prepare <= 0:
        for name, xf in (("fused_H6_T8192", lambda: kda_synth.config(1)),
                         ("fused_H24_T8192", lambda: kda_synth.config(1, H=24)),
                         ("fused_H96_T8192", lambda: kda_synth.config(3))):
            xf = xf()
            per_config[name] = summarize(
                xf, time_config(xf, max(5, args.steps // 5), 2, device, hip, fuse_prepare=1))
            progress(f"{name}: {per_config[name]}")
            del xf
            torch.cuda.empty_cache()
    # Fractions against the rates measured on this machine as well as the published peaks.
    for v in per_config.values():
        if isinstance(v, dict) and "alg_bytes" in v:
            t = v["us"] * 1e-6
            v["hbm_frac_of_measured_copy"] = round(v["alg_bytes"] / t / (copy_gbs * 1e9), 5)
            if "alg_flop" in v:
                v["mfma_frac_of_measured_gemm"] = round(v["alg_flop"] / t / (gemm_tflops * 1e12), 5)
    if "config1" in per_config and "config3" in per_config:
        c1, c3 = per_config["config1"], per_config["config3"]
        # t(H=96) / t(H=6) by step time and by per-call medians: warm, flushed by a 512 MB
        # write, and cold after a 512 MB read (H=6's 63 MB of inputs fit in the MALL when
        # warm).
        per_config["head_scaling_t96_over_t6"] = round(c3["us"] / c1["us"], 3)
        for mode in ("warm", "flushed", "cold"):
            per_config[f"head_scaling_{mode}_per_call"] = round(
                c3["per_call_us"][mode]["median"] / c1["per_call_us"][mode]["median"], 3)

    cpu = None
    if not args.no_cpu_baseline:
        x3 = kda_synth.config(3) if args.config != 3 else None
        cpu = cpu_baseline(x, x3)
        del x3
        progress(f"cpu_baseline: {cpu}")

    line = {
        "metric": "KDA prefill tokens/s at T=8192 (H=6 default; H=12/96 under per_config)",
        "value": round(x.tokens() / (r["ms_per_step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_ms": round(1e3 * WARMUP_MIN_S, 1),
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{workload}: B=1 T={x.T} H={x.H} d=128 chunk=16 "
                               f"bf16 q,k,v,g,beta; bf16 state", "global_batch": x.B,
                   "seq_len": x.T, "heads": x.H, "parallelism": "single-gpu"},
        "roofline": roofline,
        "hbm_copy_measured_gbs": round(copy_gbs, 1),
        "mfma_bf16_gemm_measured_tflops": round(gemm_tflops, 1),
        "cpu_baseline": cpu,
        "per_config": per_config,
        "kernel_source_hash": kernel_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
