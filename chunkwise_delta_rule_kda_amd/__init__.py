"""Python binding of libkda, the MI355X (gfx950) chunkwise KDA prefill library.

Argument marshalling only: every step of the computation runs in the HIP kernels behind
the C ABI of ``include/kda.h``. PyTorch supplies device memory and the stream. If the
library has not been built this module raises on the first call (there is no fallback).

Entry points (same names as the C ABI):
    kda_prefill(q, k, v, g, beta, state_in=None, cu_seqlens=None, ...) -> (o, state_out)
    kda_prefill_no_alloc(...): the same with the library's static device scratch as the
        workspace (no workspace argument; the outputs are still the caller's or torch's)
    kda_prefill_workspace_bytes(...), kda_prefill_check(...), kda_prefill_plan(...)
    kda_status_string(status), kda_last_error(), kda_debug_check_cu_seqlens(cu, T)
"""

import ctypes
import math
import os

__all__ = [
    "KdaError",
    "lib_path",
    "load_library",
    "kda_prefill",
    "kda_prefill_no_alloc",
    "kda_prefill_args",
    "kda_prefill_workspace_bytes",
    "kda_prefill_check",
    "kda_prefill_plan",
    "kda_status_string",
    "kda_last_error",
    "kda_debug_check_cu_seqlens",
    "make_args",
    "KDA_BF16",
    "KDA_FP32",
    "KDA_FLAG_L2NORM_QK",
    "KDA_FLAG_GATE_IN_KERNEL",
    "KDA_FLAG_BETA_IS_LOGIT",
    "KDA_FLAG_KEEP_RECORDS",
    "KDA_WS_RECORD",
    "STATUS",
]

KDA_BF16 = 0
KDA_FP32 = 1
KDA_FLAG_L2NORM_QK = 1 << 0
KDA_FLAG_GATE_IN_KERNEL = 1 << 1
KDA_FLAG_BETA_IS_LOGIT = 1 << 2
KDA_FLAG_KEEP_RECORDS = 1 << 3
KDA_WS_RECORD = 13824
HEAD_DIM = 128

STATUS = {
    0: "KDA_OK",
    1: "KDA_ERR_NULL",
    2: "KDA_ERR_SHAPE",
    3: "KDA_ERR_DTYPE",
    4: "KDA_ERR_FLAGS",
    5: "KDA_ERR_BOUND",
    6: "KDA_ERR_ALIAS",
    7: "KDA_ERR_WORKSPACE",
    8: "KDA_ERR_HIP",
    9: "KDA_ERR_CU_SEQLENS",
    10: "KDA_ERR_CONFIG",
}


class KdaError(RuntimeError):
    def __init__(self, status, detail=""):
        self.status = status
        name = STATUS.get(status, str(status))
        super().__init__(f"{name}: {detail}" if detail else name)


class kda_prefill_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("state_in", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("state_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("state_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("lower_bound", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("rows_per_workgroup", ctypes.c_int32),
        ("segment_chunks", ctypes.c_int32),
        ("checkpoint_every", ctypes.c_int64),
        ("checkpoint_rows", ctypes.c_int64),
        ("state_checkpoints", ctypes.c_void_p),
        ("checkpoint_cu_starts", ctypes.c_void_p),
        ("ssm_state_indices", ctypes.c_void_p),
        ("state_pool_slots", ctypes.c_int64),
        ("state_slot_pitch", ctypes.c_int64),
        ("seq_order", ctypes.c_void_p),
        ("trace_events", ctypes.c_void_p),
        ("n_trace_events", ctypes.c_int32),
        ("fuse_prepare", ctypes.c_int32),
    ]


class kda_plan_info(ctypes.Structure):
    _fields_ = [
        ("rows_per_workgroup", ctypes.c_int32),
        ("waves_per_workgroup", ctypes.c_int32),
        ("recurrence_workgroups", ctypes.c_int64),
        ("prepare_workgroups", ctypes.c_int64),
        ("max_chunks", ctypes.c_int64),
        ("workspace_header_bytes", ctypes.c_size_t),
        ("segment_chunks", ctypes.c_int64),
        ("segments_per_head_bound", ctypes.c_int64),
        ("combine_workgroups", ctypes.c_int64),
        ("scan_c_workgroups", ctypes.c_int64),
        ("scan_state_offset", ctypes.c_size_t),
        ("scan_transition_offset", ctypes.c_size_t),
        ("decode", ctypes.c_int32),
        ("scan_affine_output", ctypes.c_int32),
        ("scan_output_offset", ctypes.c_size_t),
        ("fused", ctypes.c_int32),
        ("has_records", ctypes.c_int32),
        ("records_offset", ctypes.c_size_t),
        ("status_offset", ctypes.c_size_t),
    ]


KDA_NO_ALLOC_SCRATCH_BYTES = 64 << 20  # include/kda.h

ABI_VERSION = 7  # the kda_prefill_args layout above (include/kda.h, KDA_ABI_VERSION)


def lib_path():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")


_LIB = None


def load_library():
    """Load libkda.so (built in-tree by ``__graft_entry__.build()``); raise if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(
            f"libkda.so not found at {path}: build it with `python -c \"import "
            "__graft_entry__ as g; g.build()\"` (there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(kda_prefill_args)
    lib.kda_prefill.argtypes = [P, ctypes.c_void_p]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill_no_alloc.argtypes = [P, ctypes.c_void_p]
    lib.kda_prefill_no_alloc.restype = ctypes.c_int
    lib.kda_prefill_check.argtypes = [P]
    lib.kda_prefill_check.restype = ctypes.c_int
    lib.kda_prefill_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_prefill_workspace_bytes.restype = ctypes.c_int
    lib.kda_prefill_plan.argtypes = [P, ctypes.c_int32, ctypes.POINTER(kda_plan_info)]
    lib.kda_prefill_plan.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_debug_check_cu_seqlens.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_void_p]
    lib.kda_debug_check_cu_seqlens.restype = ctypes.c_int
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int32
    if lib.kda_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.kda_abi_version()}, this binding "
                          f"expects {ABI_VERSION}: rebuild the library")
    _LIB = lib
    return lib


def kda_status_string(status):
    return load_library().kda_status_string(int(status)).decode()


def kda_last_error():
    return load_library().kda_last_error().decode()


def _raise_if(status):
    if status != 0:
        raise KdaError(status, kda_last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dtype_code(dt):
    import torch

    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_FP32
    raise KdaError(3, f"unsupported dtype {dt}")


def make_args(*, q=None, k=None, v=None, g=None, beta=None, state_in=None, cu_seqlens=None,
              A_log=None, dt_bias=None, o=None, state_out=None, workspace=None,
              workspace_bytes=0, B, T, H, N, D=HEAD_DIM, io_dtype=KDA_BF16,
              state_dtype=KDA_BF16, scale=0.0, lower_bound=0.0, flags=0,
              rows_per_workgroup=0, segment_chunks=0, checkpoint_every=0,
              checkpoint_rows=0, state_checkpoints=None, checkpoint_cu_starts=None,
              ssm_state_indices=None, state_pool_slots=0, state_slot_pitch=0, seq_order=None,
              trace_events=None, fuse_prepare=0):
    """Fill a kda_prefill_args from raw pointers (ints), tensors or None."""
    a = kda_prefill_args()
    a.q, a.k, a.v, a.g, a.beta = (_ptr(x) for x in (q, k, v, g, beta))
    a.state_in = _ptr(state_in)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    a.o, a.state_out = _ptr(o), _ptr(state_out)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = int(workspace_bytes)
    a.B, a.T, a.H, a.D, a.N = int(B), int(T), int(H), int(D), int(N)
    a.io_dtype, a.state_dtype = int(io_dtype), int(state_dtype)
    a.scale = float(scale)
    a.lower_bound = float(lower_bound)
    a.flags = int(flags)
    a.rows_per_workgroup = int(rows_per_workgroup)
    a.segment_chunks = int(segment_chunks)
    a.checkpoint_every = int(checkpoint_every)
    a.checkpoint_rows = int(checkpoint_rows)
    a.state_checkpoints = _ptr(state_checkpoints)
    a.checkpoint_cu_starts = _ptr(checkpoint_cu_starts)
    a.ssm_state_indices = _ptr(ssm_state_indices)
    a.state_pool_slots = int(state_pool_slots)
    a.state_slot_pitch = int(state_slot_pitch)
    a.seq_order = _ptr(seq_order)
    a.fuse_prepare = int(fuse_prepare)
    if trace_events is not None:
        arr = (ctypes.c_void_p * len(trace_events))(*trace_events)
        a._trace_keepalive = arr
        a.trace_events = ctypes.cast(arr, ctypes.c_void_p)
        a.n_trace_events = len(trace_events)
    return a


def kda_prefill_workspace_bytes(args):
    n = ctypes.c_size_t(0)
    _raise_if(load_library().kda_prefill_workspace_bytes(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def kda_prefill_check(args):
    """Host-only validation; returns the status code (0 = OK)."""
    return load_library().kda_prefill_check(ctypes.byref(args))


def kda_prefill_plan(args, num_cus=256):
    info = kda_plan_info()
    _raise_if(load_library().kda_prefill_plan(ctypes.byref(args), int(num_cus),
                                              ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in kda_plan_info._fields_}


def kda_debug_check_cu_seqlens(cu_seqlens, T, stream=None):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    return load_library().kda_debug_check_cu_seqlens(
        cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, int(T), s)


def _validate(q, k, v, g, beta, state_in, cu_seqlens, A_log, dt_bias, lower_bound,
              state_dtype, o, state_out, workspace, checkpoint_every, state_checkpoints,
              checkpoint_cu_starts, ssm_state_indices, seq_order):
    """Every check the C layer cannot make (it sees pointers, not sizes or devices),
    before any pointer is passed on. Shapes, dtypes and layouts are checked first and
    devices last. Returns (N, state dtype)."""
    import torch

    def need(cond, status, msg):
        if not cond:
            raise KdaError(status, msg)

    need(isinstance(q, torch.Tensor) and q.dim() == 4, 2, "q must be a [B, T, H, 128] tensor")
    B, T, H, D = q.shape
    need(D == HEAD_DIM, 2, f"head dimension {D}, only {HEAD_DIM} is supported")
    _dtype_code(q.dtype)
    for name, t, shape in (("k", k, q.shape), ("v", v, q.shape), ("g", g, q.shape),
                           ("beta", beta, (B, T, H))):
        need(isinstance(t, torch.Tensor), 2, f"{name} must be a tensor")
        need(tuple(t.shape) == tuple(shape), 2, f"{name} has shape {tuple(t.shape)}, "
             f"expected {tuple(shape)}")
        need(t.dtype == q.dtype, 3, f"{name} is {t.dtype}, q is {q.dtype}")
    if cu_seqlens is not None:
        need(cu_seqlens.dtype == torch.int64, 3, "cu_seqlens must be int64")
        need(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2, 2,
             "cu_seqlens must be a 1-D tensor of N + 1 >= 2 offsets")
        need(B == 1, 2, f"packed varlen needs B = 1 (got {B})")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if (A_log is None) != (dt_bias is None):
        raise KdaError(4, "the in-kernel gate needs both A_log and dt_bias")
    if A_log is not None:
        need(lower_bound is not None, 4, "the in-kernel gate needs lower_bound")
        need(A_log.dtype == torch.float32 and dt_bias.dtype == torch.float32, 3,
             "A_log and dt_bias must be float32")
        need(tuple(A_log.shape) == (H,), 2, f"A_log has shape {tuple(A_log.shape)}, "
             f"expected ({H},)")
        need(tuple(dt_bias.shape) == (H, D), 2, f"dt_bias has shape "
             f"{tuple(dt_bias.shape)}, expected ({H}, {D})")
    if state_dtype is None:
        state_dtype = state_in.dtype if state_in is not None else q.dtype
    _dtype_code(state_dtype)
    if state_in is not None:
        need(state_in.dtype == state_dtype, 3, f"state_in is {state_in.dtype}, the state "
             f"dtype is {state_dtype}")
        if ssm_state_indices is None:
            need(tuple(state_in.shape) == (N, H, D, D), 2, f"state_in has shape "
                 f"{tuple(state_in.shape)}, expected ({N}, {H}, {D}, {D})")
        else:
            need(state_in.dim() == 4 and tuple(state_in.shape[1:]) == (H, D, D), 2,
                 "a state pool needs state_in [N_pool, H, 128, 128]")
            need(state_in.shape[0] >= 1 and state_in[0].is_contiguous(), 2,
                 "each state pool slot must be contiguous")
            need(state_in.stride(0) % 8 == 0, 2, "the state pool's slot pitch must be a "
                 "multiple of 8 elements")
    elif ssm_state_indices is not None:
        raise KdaError(10, "a state pool needs state_in")
    if o is not None:
        need(tuple(o.shape) == tuple(q.shape) and o.dtype == q.dtype, 2,
             f"o must be {tuple(q.shape)} of {q.dtype}")
    if state_out is not None:
        if ssm_state_indices is not None:
            need(state_out is state_in or state_out.data_ptr() == state_in.data_ptr(), 6,
                 "with a state pool, state_out must be None or state_in")
        need(tuple(state_out.shape) == (N, H, D, D) or state_out is state_in, 2,
             f"state_out must be ({N}, {H}, {D}, {D})")
        need(state_out.dtype == state_dtype, 3, f"state_out is {state_out.dtype}, the "
             f"state dtype is {state_dtype}")
    if state_checkpoints is not None:
        need(state_checkpoints.dim() == 4 and tuple(state_checkpoints.shape[1:]) == (H, D, D),
             2, "state_checkpoints must be [rows, H, 128, 128]")
        need(state_checkpoints.dtype == state_dtype, 3, "state_checkpoints must have the "
             "state dtype")
    if checkpoint_cu_starts is not None:
        need(checkpoint_cu_starts.dtype == torch.int64 and
             tuple(checkpoint_cu_starts.shape) == (N + 1,), 2,
             f"checkpoint_cu_starts must be int64 [{N + 1}]")
    if checkpoint_every and checkpoint_every % 16:
        raise KdaError(10, f"checkpoint_every {checkpoint_every} is not a multiple of 16")
    for name, t in (("ssm_state_indices", ssm_state_indices), ("seq_order", seq_order)):
        if t is not None:
            need(t.dtype == torch.int32 and tuple(t.shape) == (N,), 3,
                 f"{name} must be an int32 tensor of N={N} entries")
    tensors = [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
               ("state_in", state_in), ("cu_seqlens", cu_seqlens), ("A_log", A_log),
               ("dt_bias", dt_bias), ("o", o), ("state_out", state_out),
               ("workspace", workspace), ("state_checkpoints", state_checkpoints),
               ("checkpoint_cu_starts", checkpoint_cu_starts),
               ("ssm_state_indices", ssm_state_indices), ("seq_order", seq_order)]
    for name, t in tensors:
        if t is None or (name == "state_in" and ssm_state_indices is not None):
            continue
        need(t.is_contiguous(), 2, f"{name} must be contiguous")
    for name, t in tensors:
        if t is None:
            continue
        need(t.is_cuda and t.device == q.device, 2,
             f"{name} must be a CUDA tensor on {q.device} (got {t.device})")
    return N, state_dtype


def kda_prefill(q, k, v, g, beta, state_in=None, cu_seqlens=None, *, scale=None,
                A_log=None, dt_bias=None, lower_bound=None, l2norm_qk=False,
                beta_is_logit=False, output_final_state=True, state_dtype=None, o=None,
                state_out=None, workspace=None, rows_per_workgroup=0, segment_chunks=0,
                checkpoint_every=0, state_checkpoints=None, checkpoint_cu_starts=None,
                ssm_state_indices=None, seq_order=None, stream=None, trace_events=None,
                fuse_prepare=0, keep_records=False, _no_alloc=False):
    """Chunkwise KDA prefill forward on the current (or given) HIP stream.

    q, k, v, g: [B, T, H, 128] bf16 or fp32 CUDA tensors (contiguous); beta [B, T, H].
    state_in: [N, H, 128, 128] or None. cu_seqlens: int64 [N + 1] (B = 1) or None.
    A_log / dt_bias / lower_bound: enable the in-kernel gate. Pass state_out=state_in for
    an in-place state update. segment_chunks: 0 automatic, negative serial, positive
    the time-segment length in chunks.
    checkpoint_every (tokens, a multiple of 16): also write the state before each
    interval of every sequence (the flashinfer page's checkpoint contract) into
    state_checkpoints [C, H, 128, 128] at rows checkpoint_cu_starts[n] + r. When the
    offsets or the buffer are not given they are derived here from the sequence lengths
    (which reads cu_seqlens back to the host).
    ssm_state_indices (int32 [N]): state_in is a pool [N_pool, H, 128, 128] (its first
    dimension may be padded); sequence n starts from slot ssm_state_indices[n] and its
    final state is written back there (the returned state is the pool).
    seq_order (int32 [N], a permutation): the order in which the sequences' workgroups
    start (decreasing length shortens the last partial wave); results do not change.
    Returns (o, state_out or None), or (o, state_out or None, state_checkpoints) with
    checkpoints.
    """
    import torch

    N, st_dtype = _validate(q, k, v, g, beta, state_in, cu_seqlens, A_log, dt_bias,
                            lower_bound, state_dtype, o, state_out, workspace,
                            checkpoint_every, state_checkpoints, checkpoint_cu_starts,
                            ssm_state_indices, seq_order)
    lib = load_library()
    B, T, H, D = q.shape
    state_dtype = st_dtype
    io = _dtype_code(q.dtype)
    st = _dtype_code(state_dtype)
    flags = 0
    if l2norm_qk:
        flags |= KDA_FLAG_L2NORM_QK
    if beta_is_logit:
        flags |= KDA_FLAG_BETA_IS_LOGIT
    if A_log is not None:
        flags |= KDA_FLAG_GATE_IN_KERNEL
    if keep_records:
        flags |= KDA_FLAG_KEEP_RECORDS
    if o is None:
        o = torch.empty_like(v)
    pool_slots = pool_pitch = 0
    if ssm_state_indices is not None:
        pool_slots, pool_pitch = state_in.shape[0], state_in.stride(0)
        state_out = state_in
    if state_out is None and output_final_state:
        state_out = torch.empty((N, H, D, D), dtype=state_dtype, device=q.device)
    if checkpoint_every:
        if checkpoint_cu_starts is None:
            if cu_seqlens is None:
                lens = [T] * B
            else:
                cu = cu_seqlens.cpu().tolist()
                lens = [b - a for a, b in zip(cu[:-1], cu[1:])]
            every = int(checkpoint_every)
            counts = [(n + every - 1) // every if every > 0 else 0 for n in lens]
            starts = [0]
            for c in counts:
                starts.append(starts[-1] + c)
            checkpoint_cu_starts = torch.tensor(starts, dtype=torch.int64, device=q.device)
        if state_checkpoints is None:
            rows = int(checkpoint_cu_starts[-1].item())
            state_checkpoints = torch.empty((rows, H, D, D), dtype=state_dtype, device=q.device)
    args = make_args(q=q, k=k, v=v, g=g, beta=beta, state_in=state_in,
                     cu_seqlens=cu_seqlens, A_log=A_log, dt_bias=dt_bias, o=o,
                     state_out=state_out, B=B, T=T, H=H, N=N, D=D, io_dtype=io,
                     state_dtype=st, scale=0.0 if scale is None else scale,
                     lower_bound=0.0 if lower_bound is None else lower_bound,
                     flags=flags, rows_per_workgroup=rows_per_workgroup,
                     segment_chunks=segment_chunks, checkpoint_every=checkpoint_every,
                     checkpoint_rows=0 if state_checkpoints is None else state_checkpoints.shape[0],
                     state_checkpoints=state_checkpoints,
                     checkpoint_cu_starts=checkpoint_cu_starts,
                     ssm_state_indices=ssm_state_indices, state_pool_slots=pool_slots,
                     state_slot_pitch=pool_pitch, seq_order=seq_order,
                     trace_events=trace_events, fuse_prepare=fuse_prepare)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if _no_alloc:
        if workspace is not None:
            raise KdaError(7, "kda_prefill_no_alloc takes no workspace")
        _raise_if(lib.kda_prefill_no_alloc(ctypes.byref(args), stream))
    else:
        need = kda_prefill_workspace_bytes(args)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel() * workspace.element_size()
        _raise_if(lib.kda_prefill(ctypes.byref(args), stream))
    if checkpoint_every:
        return o, state_out, state_checkpoints
    return o, state_out


def kda_prefill_no_alloc(q, k, v, g, beta, state_in=None, cu_seqlens=None, **kw):
    """kda_prefill through the C entry point of the same name: the workspace is the
    library's static device scratch (KDA_NO_ALLOC_SCRATCH_BYTES per device), so the
    library allocates nothing. Outputs not passed in (o, state_out) are still allocated
    here with torch; pass them for a call that allocates nothing at all. Calls needing
    more workspace than the scratch holds raise KdaError(KDA_ERR_WORKSPACE)."""
    if kw.get("workspace") is not None:
        raise KdaError(7, "kda_prefill_no_alloc takes no workspace")
    return kda_prefill(q, k, v, g, beta, state_in, cu_seqlens, _no_alloc=True, **kw)
