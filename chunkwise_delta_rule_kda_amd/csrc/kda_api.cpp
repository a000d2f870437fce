// Host side of libkda: argument validation, launch geometry and the extern "C" entry
// points declared in include/kda.h. No allocation, no device synchronisation (except in
// the explicit debug checker), no hidden per-call state.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

// Workspace of kda_prefill_no_alloc: one copy per device, alive until the process ends.
// In host code this name is only a handle for hipGetSymbolAddress; the device address
// it resolves to (per device) is what kernels and copies use.
static __device__ __align__(256) unsigned char scratch[KDA_NO_ALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kda_status fail(kda_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

size_t elem_size(int32_t dt) { return dt == KDA_BF16 ? 2 : 4; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

Range range_of(const void* p, size_t bytes, const char* name) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, p ? lo + bytes : lo, name};
}

int64_t max_chunks_of(const kda_prefill_args* a) {
  if (a->cu_seqlens) return (a->T + (kda::kC - 1) * a->N) / kda::kC;
  return a->N * ((a->T + kda::kC - 1) / kda::kC);
}

// Shape, dtype, flag and bound checks (no pointers beyond what sizing needs).
kda_status check_shape(const kda_prefill_args* a) {
  if (!a) return fail(KDA_ERR_NULL, "args is NULL");
  if (a->D != KDA_HEAD_DIM) return fail(KDA_ERR_SHAPE, "D=%lld, only 128 is supported", (long long)a->D);
  if (a->B < 1 || a->T < 0 || a->H < 1 || a->N < 0)
    return fail(KDA_ERR_SHAPE, "bad B=%lld T=%lld H=%lld N=%lld", (long long)a->B,
                (long long)a->T, (long long)a->H, (long long)a->N);
  if (a->H > 65535) return fail(KDA_ERR_SHAPE, "H=%lld exceeds 65535", (long long)a->H);
  // Bounds under which every size below is computed without overflow.
  if (a->B > (int64_t(1) << 31) || a->N > (int64_t(1) << 31) || a->T > (int64_t(1) << 40))
    return fail(KDA_ERR_SHAPE, "B=%lld N=%lld T=%lld out of range", (long long)a->B,
                (long long)a->N, (long long)a->T);
  if (a->cu_seqlens) {
    if (a->B != 1) return fail(KDA_ERR_SHAPE, "packed varlen needs B=1 (got %lld)", (long long)a->B);
    if (a->N < 1) return fail(KDA_ERR_SHAPE, "packed varlen needs N>=1");
  } else if (a->N != a->B) {
    return fail(KDA_ERR_SHAPE, "fixed layout needs N == B (N=%lld, B=%lld)", (long long)a->N,
                (long long)a->B);
  }
  const int64_t mc = max_chunks_of(a);
  if (mc > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "too many chunks (%lld)", (long long)mc);
  if (a->N * a->H * 8 > 0x7fffffffLL) return fail(KDA_ERR_SHAPE, "N*H too large");
  if (mc * a->H > (int64_t(1) << 40)) return fail(KDA_ERR_SHAPE, "chunks*H too large");
  if (a->io_dtype != KDA_BF16 && a->io_dtype != KDA_FP32)
    return fail(KDA_ERR_DTYPE, "io_dtype %d", a->io_dtype);
  if (a->state_dtype != KDA_BF16 && a->state_dtype != KDA_FP32)
    return fail(KDA_ERR_DTYPE, "state_dtype %d", a->state_dtype);
  const uint32_t known = KDA_FLAG_L2NORM_QK | KDA_FLAG_GATE_IN_KERNEL | KDA_FLAG_BETA_IS_LOGIT |
                         KDA_FLAG_KEEP_RECORDS;
  if (a->flags & ~known) return fail(KDA_ERR_FLAGS, "unknown flag bits 0x%x", a->flags & ~known);
  if (a->flags & KDA_FLAG_GATE_IN_KERNEL) {
    if (!a->A_log || !a->dt_bias)
      return fail(KDA_ERR_FLAGS, "gate in kernel needs A_log and dt_bias");
    if (!(a->lower_bound >= -5.0f && a->lower_bound < 0.0f))
      return fail(KDA_ERR_BOUND, "lower_bound %g outside [-5, 0)", (double)a->lower_bound);
  }
  if (!std::isfinite(a->scale) || a->scale < 0.0f)
    return fail(KDA_ERR_BOUND, "scale %g", (double)a->scale);
  if (a->rows_per_workgroup != 0 && a->rows_per_workgroup != 16 &&
      a->rows_per_workgroup != 32 && a->rows_per_workgroup != 64 &&
      a->rows_per_workgroup != 128)
    return fail(KDA_ERR_CONFIG, "rows_per_workgroup %d", a->rows_per_workgroup);
  if (a->segment_chunks > (1 << 24))
    return fail(KDA_ERR_CONFIG, "segment_chunks %d", a->segment_chunks);
  if (a->checkpoint_every < 0 || a->checkpoint_every > (int64_t(1) << 40) ||
      a->checkpoint_every % KDA_CHUNK != 0)
    return fail(KDA_ERR_CONFIG, "checkpoint_every %lld is not a non-negative multiple of 16",
                (long long)a->checkpoint_every);
  if (a->checkpoint_rows < 0 || a->checkpoint_rows > (int64_t(1) << 40))
    return fail(KDA_ERR_CONFIG, "checkpoint_rows %lld", (long long)a->checkpoint_rows);
  if (a->ssm_state_indices) {
    const int64_t dense = a->H * KDA_HEAD_DIM * KDA_HEAD_DIM;
    if (!a->state_in) return fail(KDA_ERR_CONFIG, "a state pool needs state_in");
    if (a->state_pool_slots < 1 || a->state_pool_slots > (int64_t(1) << 31))
      return fail(KDA_ERR_CONFIG, "state_pool_slots %lld", (long long)a->state_pool_slots);
    if (a->state_slot_pitch != 0 && (a->state_slot_pitch < dense || a->state_slot_pitch % 8 ||
                                     a->state_slot_pitch > (int64_t(1) << 40)))
      return fail(KDA_ERR_CONFIG, "state_slot_pitch %lld", (long long)a->state_slot_pitch);
  }
  return KDA_OK;
}

// Elements of state_in / state_out the call may touch.
size_t state_elems(const kda_prefill_args* a) {
  const size_t dense = static_cast<size_t>(a->H) * KDA_HEAD_DIM * KDA_HEAD_DIM;
  if (!a->ssm_state_indices) return static_cast<size_t>(a->N) * dense;
  const size_t pitch = a->state_slot_pitch ? static_cast<size_t>(a->state_slot_pitch) : dense;
  return (static_cast<size_t>(a->state_pool_slots) - 1) * pitch + dense;
}

int rows_per_wg(const kda_prefill_args* a, int num_cus) {
  if (a->rows_per_workgroup) return a->rows_per_workgroup;
  // Smallest slice that keeps the grid within one workgroup per compute unit
  // (the column-split post's rule, section 3.1), with 16 value rows per wave. When
  // 64-row slices take more than one round of the compute units, whole heads (128
  // rows, BF16 I/O) halve the rounds at ~1.5x the chunk time: the packed 8-sequence,
  // 24-head workload (192 pairs) runs its recurrence in 238 us instead of 255.
  const int64_t tasks = a->N * a->H;
  if (tasks * 8 <= num_cus) return 16;
  if (tasks * 4 <= num_cus) return 32;
  if (tasks * 2 <= num_cus || a->io_dtype != KDA_BF16) return 64;
  return 128;
}

// Later segments per sequence from which the affine-output form uses the
// carry-and-output launch, and from which it does so even when that launch needs more
// than one workgroup per compute unit (see make_plan).
constexpr int64_t kCarryMinLater = 6;
constexpr int64_t kCarryMinLaterShared = 9;

// Compute units the automatic segment rule is tuned for (MI355X). The rule must not
// depend on the device so that the workspace size is a pure function of the arguments.
constexpr int64_t kScanTargetCUs = 256;

// Launch geometry and workspace layout of one call.
struct Plan {
  int64_t max_chunks = 0;
  int64_t seg_len = 0;       // chunks per segment; 0 = serial recurrence
  int64_t segs_per_seq = 0;  // fixed layout
  int64_t seg_stride = 0;    // scan slots per head
  size_t header = 0;         // cu_chunks [N + 1] and cu_segs [N + 1] (varlen)
  size_t records = 0;        // offset of the records
  size_t scan_s = 0;         // offset of the FP32 scan states
  size_t scan_phi = 0;       // offset of the BF16 transitions
  bool affine = false;       // affine-output segmented form (no checkpoints)
  size_t scan_q = 0;         // offset of Qt Phi^T per chunk (affine-output form)
  bool carry = false;        // affine-output form with the carry-and-output launch
  bool fused = false;        // the recurrence prepares its own chunks (no prepare kernel)
  bool has_records = false;  // the workspace holds the records
  size_t status = 0;         // offset of the 256-byte status block
  size_t total = 0;
};

// The fused form (producer waves in the recurrence workgroups prepare the chunks) when
// the caller asks for it. The automatic choice is the separate preparation kernel: on
// MI355X the fused form's producers (one wave per chunk, about 12k cycles of dependent
// work each) leave the compute waves waiting, 1.5-1.8x slower at every head count
// measured (T = 8192, warm per call, H = 6: 112 vs 66 us; H = 24: 353 vs 208 us;
// H = 96: 953 vs 555 us), although it moves only 1.08x the algorithmic bytes at H = 96
// (the two-kernel form 2.4x).
bool fused_form(const kda_prefill_args* a) { return a->fuse_prepare > 0; }

// A few tokens per sequence (fixed layout, 1 <= T <= kDecodeMaxT, no checkpoints,
// automatic geometry): the token-loop kernel, no workspace. An explicit
// rows_per_workgroup or segment_chunks asks for the chunked path.
bool decode_form(const kda_prefill_args* a) {
  return a->T >= 1 && a->T <= kda::kDecodeMaxT && !a->cu_seqlens &&
         a->checkpoint_every == 0 && a->rows_per_workgroup == 0 && a->segment_chunks == 0;
}

// Rows per workgroup of the segmented form: the explicit choice, else 64, or a whole
// head's 128 rows (eight compute waves, BF16 I/O) from kSegRows128MinPairs (sequence,
// head) pairs on. A chunk takes ~0.95 us in a 128-row workgroup against ~0.53 us in a
// 64-row one, but a segment needs half the workgroups, so there are about twice as many
// segments. Measured per step at T = 8192, 64-row against 128-row segments: H = 8 77.7
// vs 81.3 us, H = 9 87.0 vs 89.1, H = 10 104.4 vs 96.6, H = 11 103.3 vs 100.6, H = 12
// 117.3 vs 110.7, H = 13 118.3 vs 113.1, H = 14 123.8 vs 126.9, H = 16 142.9 vs 142.4,
// H = 18 153.8 vs 153.0, H = 20 190.2 vs 178.8, H = 24 205.8 vs 200.4, H = 32 258.7 vs
// 251.7; from 33 pairs on 64-row segments no longer fit at all. The fused form keeps
// 64-row segments up to 32 pairs: its chunk time grows more with the rows (the producer
// waves share the CU with eight compute waves), H = 24 took 523 us per step in 128-row
// segments against 357 us in 64-row ones.
constexpr int64_t kSegRows128MinPairs = 10;
constexpr int64_t kFusedSegRows128MinPairs = 33;
int segmented_rows(const kda_prefill_args* a) {
  if (a->rows_per_workgroup) return a->rows_per_workgroup;
  const int64_t from = fused_form(a) ? kFusedSegRows128MinPairs : kSegRows128MinPairs;
  return a->io_dtype == KDA_BF16 && a->N * a->H >= from ? 128 : 64;
}

Plan make_plan(const kda_prefill_args* a) {
  Plan pl;
  pl.max_chunks = max_chunks_of(a);
  if (decode_form(a)) return pl;
  const int64_t per_seq = a->cu_seqlens ? (a->N > 0 ? pl.max_chunks / a->N : 0)
                                        : (a->T + kda::kC - 1) / kda::kC;
  int64_t L = 0;
  if (a->segment_chunks > 0) {
    L = a->segment_chunks;
  } else if (a->segment_chunks == 0) {
    // Time segments pay off when few (sequence, head) pairs leave compute units idle:
    // with b = 128 / rows workgroups per 128 rows, launch A has b (2 P - 1)
    // (affine-output form) or b (2 P - 3) (with checkpoints) workgroups per pair for P
    // segments; aim for one per compute unit, with segments of at least 16 chunks, and
    // take three segments or more (two when at most 32 pairs).
    const int64_t pairs = a->N * a->H;
    if (pairs > 0) {
      const int64_t b = kda::kD / segmented_rows(a);
      const int64_t P = (kScanTargetCUs / (pairs * b) + (a->checkpoint_every > 0 ? 3 : 1)) / 2;
      if (P >= 3 || (P >= 2 && pairs * 8 <= kScanTargetCUs)) {
        L = (per_seq + P - 1) / P;
        if (L < 16) L = 16;
      }
    }
  }
  if (L > 0) {
    if (a->cu_seqlens) {
      if (per_seq > L || a->segment_chunks > 0) {  // automatic: sequences average > 1 segment
        pl.seg_len = L;
        pl.seg_stride = (pl.max_chunks + L - 1) / L + a->N;
      }
    } else {
      const int64_t P = per_seq > 0 ? (per_seq + L - 1) / L : 1;
      if (P >= 2 || a->segment_chunks > 0) {
        pl.seg_len = L;
        pl.segs_per_seq = P;
        pl.seg_stride = a->N * P;
      }
    }
  }
  // varlen header: cu_chunks and cu_segs (int64 [N + 1] each), then the automatic
  // sequence order (int32 [N])
  pl.header = a->cu_seqlens ? round_up(static_cast<size_t>(a->N + 1) * 16 +
                                           static_cast<size_t>(a->N) * 4, 256)
                            : 0;
  pl.fused = fused_form(a);
  pl.records = pl.header;
  size_t end = pl.records;
  if (!pl.fused || (a->flags & KDA_FLAG_KEEP_RECORDS)) {
    pl.has_records = true;
    end += static_cast<size_t>(pl.max_chunks) * static_cast<size_t>(a->H) *
           static_cast<size_t>(kda::kRecord);
  }
  if (pl.seg_len > 0) {
    const size_t slots = static_cast<size_t>(a->H) * static_cast<size_t>(pl.seg_stride);
    pl.scan_s = round_up(end, 256);
    pl.scan_phi = pl.scan_s + slots * kda::kD * kda::kD * 4;
    end = pl.scan_phi + slots * kda::kD * kda::kD * 2;
    pl.affine = a->checkpoint_every == 0;
    // Many segments per sequence (few heads): one carry-and-output launch in place of the
    // combine and the scan output. Measured per step at T = 8192 (BF16), carry against
    // combine + scan output: 64-row segments H = 6 (10 later segments, 240 workgroups)
    // 65.5 against 68.7 us, H = 8 (7, 224) 77.8 against 80.9; 128-row segments H = 10
    // (12, 480) 96.2 against 96.7, H = 12 (10, 480) 109.5 against 110.5, H = 14 (8, 448)
    // 127.1 against 125.6, H = 16 (7, 448) 140.6 against 139.0, H = 20 (5) 180.4 against
    // 178.4, H = 24 (4) 204.4 against 200.5, H = 32 (3) 264.6 against 257.9. With two of
    // its workgroups per compute unit the chains' operand streams share the unit, and
    // with few long segments the scan output's many small workgroups stream the output
    // terms faster.
    {
      const int64_t later = pl.segs_per_seq - 1;
      pl.carry = pl.affine && !a->cu_seqlens && later >= kCarryMinLater &&
                 (a->H * a->N * later * 4 <= kScanTargetCUs || later >= kCarryMinLaterShared);
    }
    if (pl.affine) {
      pl.scan_q = round_up(end, 256);
      end = pl.scan_q + static_cast<size_t>(pl.max_chunks) * static_cast<size_t>(a->H) * 2048 *
                            elem_size(a->io_dtype);
    }
  }
  pl.status = round_up(end, 256);
  pl.total = pl.status + 256;
  return pl;
}

size_t workspace_need(const kda_prefill_args* a) { return make_plan(a).total; }

// Workgroups of launch A and of the re-run launch C of the segmented form. Fixed
// layout: the active row blocks only (per sequence b0 for segment 0 and 2 b0 for each of
// segments 1 .. P-1 (affine-output form) or 1 .. P-2 (re-run form) in A, b0 for each of
// segments 1 .. P-1 in C, b0 = 128 / rows). Varlen: every scan slot of the bound times
// the row blocks; workgroups past a sequence's segments exit.
int64_t scan_a_workgroups(const kda_prefill_args* a, const Plan& pl, int rows) {
  const int64_t b0 = KDA_HEAD_DIM / rows;
  if (a->cu_seqlens) return a->H * pl.seg_stride * 2 * b0;
  const int64_t P = pl.segs_per_seq;
  const int64_t mid = pl.affine ? P - 1 : P - 2;  // segments with Z and Phi runs
  return a->H * a->N * (P >= 2 ? b0 + 2 * b0 * mid : b0);
}

// Workgroups of the scan-output launch (affine-output form): kScanOutChunks chunks of
// one later segment each.
int64_t scan_out_workgroups(const kda_prefill_args* a, const Plan& pl) {
  const int64_t groups = (pl.seg_len + kda::kScanOutChunks - 1) / kda::kScanOutChunks;
  if (a->cu_seqlens) return a->H * pl.seg_stride * groups;
  return a->H * a->N * (pl.segs_per_seq - 1) * groups;
}

// Workgroups of the carry-and-output launch: four 32-row blocks per later segment.
int64_t carry_out_workgroups(const kda_prefill_args* a, const Plan& pl) {
  return a->H * a->N * (pl.segs_per_seq - 1) * 4;
}

int64_t scan_c_workgroups(const kda_prefill_args* a, const Plan& pl, int rows) {
  const int64_t b0 = KDA_HEAD_DIM / rows;
  if (a->cu_seqlens) return a->H * pl.seg_stride * b0;
  return a->H * a->N * (pl.segs_per_seq - 1) * b0;
}

// Rows per workgroup of the recurrence launches: the explicit choice, else the
// segmented form's (launch A alone has about one workgroup per compute unit) and the
// fill rule in the serial form.
int rows_of(const kda_prefill_args* a, const Plan& pl, int num_cus) {
  if (a->rows_per_workgroup) return a->rows_per_workgroup;
  return pl.seg_len > 0 ? segmented_rows(a) : rows_per_wg(a, num_cus);
}

std::atomic<int> g_cu_count[64];

int cu_count_current(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Device address of `scratch` on the current device, resolved once per device (with
// that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

kda_status scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(KDA_ERR_HIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "shape out of range or inconsistent";
    case KDA_ERR_DTYPE: return "unsupported dtype";
    case KDA_ERR_FLAGS: return "unknown flag or missing flag input";
    case KDA_ERR_BOUND: return "lower_bound or scale out of range";
    case KDA_ERR_ALIAS: return "output overlaps an input";
    case KDA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case KDA_ERR_HIP: return "HIP runtime error";
    case KDA_ERR_CU_SEQLENS: return "cu_seqlens violates its contract";
    case KDA_ERR_CONFIG: return "unsupported launch configuration";
  }
  return "unknown status";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

kda_status kda_prefill_workspace_bytes(const kda_prefill_args* a, size_t* bytes) {
  g_last_error.clear();
  const kda_status s = check_shape(a);
  if (s != KDA_OK) return s;
  if (!bytes) return fail(KDA_ERR_NULL, "bytes is NULL");
  *bytes = workspace_need(a);
  return KDA_OK;
}

kda_status kda_prefill_check(const kda_prefill_args* a) {
  g_last_error.clear();
  kda_status s = check_shape(a);
  if (s != KDA_OK) return s;
  const int64_t tokens = a->B * a->T;
  if (tokens > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o))
    return fail(KDA_ERR_NULL, "q, k, v, g, beta and o are required");
  const size_t es = elem_size(a->io_dtype);
  const size_t tensor = static_cast<size_t>(tokens) * a->H * KDA_HEAD_DIM * es;
  const size_t beta_b = static_cast<size_t>(tokens) * a->H * es;
  const size_t state_b = state_elems(a) * elem_size(a->state_dtype);
  if (a->ssm_state_indices && a->state_out && a->state_out != a->state_in)
    return fail(KDA_ERR_ALIAS, "with a state pool, state_out must be NULL or state_in");
  const size_t need = workspace_need(a);
  if (need > 0) {
    if (!a->workspace) return fail(KDA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (a->workspace_bytes < need)
      return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", a->workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(a->workspace) % 256)
      return fail(KDA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  }
  const bool ckpt = a->checkpoint_every > 0;
  // With no checkpoint rows nothing is ever written, so state_checkpoints may be NULL
  // (the data pointer of a zero-size buffer often is); the row offsets are still read.
  if (ckpt && !a->checkpoint_cu_starts)
    return fail(KDA_ERR_NULL, "checkpoints need checkpoint_cu_starts");
  if (ckpt && a->checkpoint_rows > 0 && !a->state_checkpoints)
    return fail(KDA_ERR_NULL, "checkpoint_rows > 0 needs state_checkpoints");
  // Alignment the kernels' vector accesses rely on.
  const void* vec[] = {a->q, a->k, a->v, a->g, a->o, a->state_in, a->state_out,
                       ckpt ? a->state_checkpoints : nullptr};
  for (const void* p : vec)
    if (reinterpret_cast<uintptr_t>(p) % 16)
      return fail(KDA_ERR_SHAPE, "q, k, v, g, o, state and checkpoint pointers must be 16-byte aligned");

  const Range ins[] = {
      range_of(a->q, tensor, "q"),          range_of(a->k, tensor, "k"),
      range_of(a->v, tensor, "v"),          range_of(a->g, tensor, "g"),
      range_of(a->beta, beta_b, "beta"),    range_of(a->state_in, state_b, "state_in"),
      range_of(a->cu_seqlens, a->cu_seqlens ? (a->N + 1) * 8 : 0, "cu_seqlens"),
      range_of(a->A_log, (a->flags & KDA_FLAG_GATE_IN_KERNEL) ? a->H * 4 : 0, "A_log"),
      range_of(a->dt_bias, (a->flags & KDA_FLAG_GATE_IN_KERNEL) ? a->H * 512 : 0, "dt_bias"),
      range_of(a->checkpoint_cu_starts, ckpt ? (a->N + 1) * 8 : 0, "checkpoint_cu_starts"),
      range_of(a->ssm_state_indices, a->ssm_state_indices ? a->N * 4 : 0, "ssm_state_indices"),
      range_of(a->seq_order, a->seq_order ? a->N * 4 : 0, "seq_order"),
  };
  const Range o = range_of(a->o, tensor, "o");
  const Range so = range_of(a->state_out, state_b, "state_out");
  const Range ws = range_of(a->workspace, need, "workspace");
  const int kStateIn = 5;  // index of state_in in ins[]
  for (int i = 0; i < static_cast<int>(sizeof ins / sizeof ins[0]); ++i) {
    const Range& in = ins[i];
    if (overlap(o, in)) return fail(KDA_ERR_ALIAS, "o overlaps %s", in.name);
    if (overlap(ws, in)) return fail(KDA_ERR_ALIAS, "workspace overlaps %s", in.name);
    const bool inplace = i == kStateIn && a->state_out == a->state_in;
    if (!inplace && overlap(so, in)) return fail(KDA_ERR_ALIAS, "state_out overlaps %s", in.name);
  }
  if (overlap(o, so)) return fail(KDA_ERR_ALIAS, "o overlaps state_out");
  if (overlap(o, ws)) return fail(KDA_ERR_ALIAS, "o overlaps workspace");
  if (overlap(so, ws)) return fail(KDA_ERR_ALIAS, "state_out overlaps workspace");
  if (ckpt) {
    const Range ck = range_of(a->state_checkpoints,
                              static_cast<size_t>(a->checkpoint_rows) * a->H * KDA_HEAD_DIM *
                                  KDA_HEAD_DIM * elem_size(a->state_dtype),
                              "state_checkpoints");
    for (const Range& in : ins)
      if (overlap(ck, in)) return fail(KDA_ERR_ALIAS, "state_checkpoints overlaps %s", in.name);
    if (overlap(ck, o) || overlap(ck, so) || overlap(ck, ws))
      return fail(KDA_ERR_ALIAS, "state_checkpoints overlaps an output or the workspace");
  }
  return KDA_OK;
}

kda_status kda_prefill_plan(const kda_prefill_args* a, int32_t num_cus, kda_plan_info* out) {
  g_last_error.clear();
  const kda_status s = check_shape(a);
  if (s != KDA_OK) return s;
  if (!out) return fail(KDA_ERR_NULL, "out is NULL");
  const Plan pl = make_plan(a);
  const int rows = rows_of(a, pl, num_cus > 0 ? num_cus : 256);
  std::memset(out, 0, sizeof *out);
  out->rows_per_workgroup = rows;
  out->waves_per_workgroup = rows / 16 + kda::recurrence_loader_waves(rows / 16);
  out->max_chunks = pl.max_chunks;
  out->prepare_workgroups = pl.max_chunks * a->H;
  out->workspace_header_bytes = pl.header;
  out->segment_chunks = pl.seg_len;
  out->segments_per_head_bound = pl.seg_stride;
  if (pl.seg_len > 0) {
    out->recurrence_workgroups = scan_a_workgroups(a, pl, rows);
    out->scan_c_workgroups = pl.carry    ? carry_out_workgroups(a, pl)
                             : pl.affine ? scan_out_workgroups(a, pl)
                                         : scan_c_workgroups(a, pl, rows);
    out->combine_workgroups = pl.carry ? 0 : (a->H * a->N + 7) / 8 * 64;
    out->scan_affine_output = pl.affine ? 1 : 0;
    out->scan_output_offset = pl.scan_q;
  } else {
    out->recurrence_workgroups = (a->N * a->H + 7) / 8 * 8 * (KDA_HEAD_DIM / rows);
  }
  out->scan_state_offset = pl.scan_s;
  out->scan_transition_offset = pl.scan_phi;
  out->fused = pl.fused ? 1 : 0;
  out->status_offset = pl.status;
  out->records_offset = pl.has_records ? pl.records : 0;
  out->has_records = pl.has_records ? 1 : 0;
  if (pl.fused) {
    out->prepare_workgroups = 0;
    out->waves_per_workgroup = rows / 16 + 4;
  }
  if (decode_form(a)) {
    out->fused = 0;
    out->status_offset = 0;
    out->records_offset = 0;
    out->has_records = 0;
    out->decode = 1;
    out->prepare_workgroups = 0;
    out->recurrence_workgroups = a->N * a->H;
    out->waves_per_workgroup = 4;
    out->rows_per_workgroup = KDA_HEAD_DIM;
  }
  return KDA_OK;
}

kda_status kda_prefill(const kda_prefill_args* a, void* stream_) {
  kda_status s = kda_prefill_check(a);
  if (s != KDA_OK) return s;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const Plan pl = make_plan(a);
  const int rows = rows_of(a, pl, cu_count_current());
  unsigned char* ws = static_cast<unsigned char*>(a->workspace);

  kda::Params p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.g = a->g;
  p.beta = a->beta;
  p.state_in = a->state_in;
  p.cu_seqlens = a->cu_seqlens;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.o = a->o;
  p.state_out = a->state_out;
  p.cu_chunks = a->cu_seqlens ? reinterpret_cast<int64_t*>(ws) : nullptr;
  p.cu_segs = a->cu_seqlens ? reinterpret_cast<int64_t*>(ws) + (a->N + 1) : nullptr;
  p.records = ws + pl.records;
  p.B = a->B;
  p.T = a->T;
  p.H = a->H;
  p.N = a->N;
  p.max_chunks = pl.max_chunks;
  p.chunks_per_seq = (a->T + kda::kC - 1) / kda::kC;
  p.scale = a->scale > 0.0f ? a->scale : 1.0f / std::sqrt(static_cast<float>(KDA_HEAD_DIM));
  p.lower_bound = a->lower_bound;
  p.flags = a->flags;
  p.waves = rows / 16;
  p.mode = kda::kModeSerial;
  p.seg_len = pl.seg_len;
  p.segs_per_seq = pl.segs_per_seq;
  p.seg_stride = pl.seg_stride;
  if (a->ssm_state_indices) {
    p.state_idx = a->ssm_state_indices;
    p.pool_slots = a->state_pool_slots;
    p.slot_pitch = a->state_slot_pitch ? a->state_slot_pitch
                                        : a->H * KDA_HEAD_DIM * KDA_HEAD_DIM;
    p.state_out = const_cast<void*>(a->state_in);  // the pool is updated in place
  }
  // Without a caller's order, the serial form starts varlen sequences longest first
  // (ordered on the device by the plan kernel; up to kAutoOrderMax sequences).
  int32_t* auto_order = nullptr;
  if (a->cu_seqlens && pl.seg_len == 0 && !a->seq_order && a->N <= kda::kAutoOrderMax)
    auto_order = reinterpret_cast<int32_t*>(ws + static_cast<size_t>(a->N + 1) * 16);
  p.seq_order = a->seq_order ? a->seq_order : auto_order;
  if (a->checkpoint_every > 0) {
    p.ckpt = a->state_checkpoints;
    p.ckpt_cu = a->checkpoint_cu_starts;
    p.ckpt_every = a->checkpoint_every / KDA_CHUNK;
    p.ckpt_rows = a->checkpoint_rows;
  }
  if (pl.fused) {
    p.fused = 1;
    p.keep_records = (a->flags & KDA_FLAG_KEEP_RECORDS) ? 1 : 0;
  }
  p.status = reinterpret_cast<int*>(ws + pl.status);
  if (pl.seg_len > 0) {
    p.scan_s = reinterpret_cast<float*>(ws + pl.scan_s);
    p.scan_phi = reinterpret_cast<unsigned short*>(ws + pl.scan_phi);
    p.affine_out = pl.affine ? 1 : 0;
    if (pl.affine) p.scan_q = ws + pl.scan_q;
  }
  const bool io_bf16 = a->io_dtype == KDA_BF16;
  const bool st_bf16 = a->state_dtype == KDA_BF16;
  auto recurrence = [&](int64_t wgs) {
    return kda::launch_recurrence(p, wgs, io_bf16, st_bf16, stream);
  };
  hipEvent_t* ev = nullptr;
  if (a->trace_events && a->n_trace_events >= 3)
    ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(a->trace_events));
  const bool ev5 = ev && a->n_trace_events >= 5;

  hipError_t e = hipSuccess;
  if (decode_form(a)) {
    if (ev) e = hipEventRecord(ev[0], stream);
    if (e == hipSuccess) e = kda::launch_decode(p, io_bf16, st_bf16, stream);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], stream);
    if (e == hipSuccess && ev5) e = hipEventRecord(ev[3], stream);
    if (e == hipSuccess && ev5) e = hipEventRecord(ev[4], stream);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[2], stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s", hipGetErrorString(e));
    return KDA_OK;
  }
  if (ev) e = hipEventRecord(ev[0], stream);
  if (e == hipSuccess && a->cu_seqlens) e = kda::launch_plan(p, auto_order, stream);
  if (e == hipSuccess && a->T > 0 && !pl.fused) e = kda::launch_prepare(p, io_bf16, stream);
  if (e == hipSuccess && ev) e = hipEventRecord(ev[1], stream);
  if (pl.seg_len == 0) {
    // whole rounds of 8 (sequence, head) pairs over the XCDs, each with its row blocks
    const int64_t wgs = (a->N * a->H + 7) / 8 * 8 * (KDA_HEAD_DIM / rows);
    if (e == hipSuccess) e = recurrence(wgs);
    if (e == hipSuccess && ev5) e = hipEventRecord(ev[3], stream);
    if (e == hipSuccess && ev5) e = hipEventRecord(ev[4], stream);
  } else {
    p.mode = kda::kModeScanA;
    p.blocks = 2 * KDA_HEAD_DIM / rows;
    if (e == hipSuccess) e = recurrence(scan_a_workgroups(a, pl, rows));
    if (e == hipSuccess && ev5) e = hipEventRecord(ev[3], stream);
    if (e == hipSuccess && !pl.carry &&
        (a->cu_seqlens || pl.segs_per_seq >= (pl.affine ? 2 : 3)))
      e = kda::launch_combine(p, st_bf16, stream);
    if (e == hipSuccess && ev5) e = hipEventRecord(ev[4], stream);
    p.mode = kda::kModeScanC;
    p.blocks = KDA_HEAD_DIM / rows;
    if (pl.carry) {
      if (e == hipSuccess)
        e = kda::launch_carry_out(p, carry_out_workgroups(a, pl), io_bf16, st_bf16, stream);
    } else if (pl.affine) {
      if (e == hipSuccess) e = kda::launch_scan_output(p, scan_out_workgroups(a, pl), io_bf16, stream);
    } else {
      if (e == hipSuccess) e = recurrence(scan_c_workgroups(a, pl, rows));
    }
  }
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s", hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_prefill_no_alloc(const kda_prefill_args* a, void* stream) {
  g_last_error.clear();
  kda_status s = check_shape(a);
  if (s != KDA_OK) return s;
  if (a->workspace)
    return fail(KDA_ERR_WORKSPACE, "kda_prefill_no_alloc uses the library's static scratch: "
                                   "pass workspace = NULL");
  const size_t need = workspace_need(a);
  if (need > KDA_NO_ALLOC_SCRATCH_BYTES)
    return fail(KDA_ERR_WORKSPACE,
                "the call needs %zu bytes of workspace, the static scratch holds %llu "
                "(use kda_prefill with a caller-allocated workspace)",
                need, (unsigned long long)KDA_NO_ALLOC_SCRATCH_BYTES);
  kda_prefill_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (need > 0) {
    s = scratch_on_current_device(&b.workspace);
    if (s != KDA_OK) return s;
    b.workspace_bytes = KDA_NO_ALLOC_SCRATCH_BYTES;
  }
  return kda_prefill(&b, stream);
}

kda_status kda_debug_check_cu_seqlens(const int64_t* cu, int64_t N, int64_t T, void* stream) {
  g_last_error.clear();
  if (!cu) return fail(KDA_ERR_NULL, "cu_seqlens is NULL");
  if (N < 1) return fail(KDA_ERR_SHAPE, "N=%lld", (long long)N);
  std::vector<int64_t> h(static_cast<size_t>(N + 1));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * 8, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s", hipGetErrorString(e));
  if (h[0] != 0) return fail(KDA_ERR_CU_SEQLENS, "cu_seqlens[0]=%lld", (long long)h[0]);
  for (int64_t i = 0; i < N; ++i)
    if (h[i + 1] < h[i])
      return fail(KDA_ERR_CU_SEQLENS, "cu_seqlens decreases at %lld", (long long)i);
  if (h[N] != T) return fail(KDA_ERR_CU_SEQLENS, "cu_seqlens[N]=%lld != T=%lld", (long long)h[N], (long long)T);
  return KDA_OK;
}

}  // extern "C"
