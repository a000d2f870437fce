/*
 * kda.h - C ABI of the MI355X (gfx950) chunkwise Kimi Delta Attention prefill library.
 *
 * The operation (one call = the whole prefill forward of every sequence and head):
 * for each sequence n and head h, starting from the state S (values x keys, 128 x 128)
 * given in state_in[n, h] (or zeros), every token t updates
 *
 *     S <- S Diag(exp g_t) ;  S <- S + beta_t (v_t - S k_t) k_t^T ;  o_t = scale * S q_t
 *
 * and the final S is written to state_out[n, h]. This is the token form of the chunk
 * equations of the "FlashKDA column split" post (section 1, "FlashKDA in two kernels"):
 * the library evaluates it chunk by chunk (16 tokens) with a chunk-parallel preparation
 * kernel and a serial recurrence kernel whose 128 value rows are split across compute
 * units (section 3.1 of the same post: value rows never interact).
 *
 * A few tokens per sequence (fixed layout with 1 <= T <= 8, no checkpoints, automatic
 * geometry: rows_per_workgroup = segment_chunks = 0) is a decode step (T = 1) or the
 * verification of draft tokens: a token-loop kernel reads each state once, applies the
 * T token steps in registers and writes it back; such a call needs no workspace
 * (kda_prefill_workspace_bytes returns 0). An explicit rows_per_workgroup or
 * segment_chunks selects the chunked path for any T.
 *
 * The calling contract follows the "flashinfer.kda_prefill" API page (sections
 * "Optimized Blackwell prefill subset", "SM120a prefill subset" and "State and graph
 * semantics"): contiguous [B, T, H, 128] q, k, v, g; [B, T, H] beta; one shared head
 * count; head dimension 128; packed varlen through int64 cu_seqlens with B = 1;
 * state layout [N, H, V, K]; in-place state update allowed; optional in-kernel q/k L2
 * normalisation, beta from logits and the lower-bounded gate with lower_bound in [-5, 0).
 *
 * Ownership: the caller allocates every buffer (inputs, outputs, workspace). The library
 * allocates nothing, keeps no per-call caches and holds no global state besides a
 * per-device compute-unit count and, for kda_prefill_no_alloc, one static device array
 * per device (its scratch, see there). All pointers in kda_prefill_args are device
 * pointers unless stated otherwise.
 *
 * Errors: every entry point returns a kda_status; nothing aborts or throws across the
 * ABI. Host-checkable violations are rejected before any launch. Device-side contract
 * violations (non-monotone cu_seqlens, cu_seqlens[0] != 0, cu_seqlens[N] != T, a
 * precomputed g outside [-5, 0]) are undefined behaviour, as on the flashinfer page;
 * kda_debug_check_cu_seqlens is the explicit (synchronising) checker for tests.
 *
 * Indexing is 64-bit throughout: there is no 2^31 extent limit.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 7
#define KDA_HEAD_DIM 128 /* d_k = d_v = 128 */
#define KDA_CHUNK 16     /* tokens per chunk */

typedef enum kda_dtype {
  KDA_BF16 = 0, /* bfloat16, round-to-nearest-even on output */
  KDA_FP32 = 1  /* IEEE float32 */
} kda_dtype;

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,       /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,      /* B, T, H, N or D out of range, or inconsistent */
  KDA_ERR_DTYPE = 3,      /* io_dtype or state_dtype not a kda_dtype */
  KDA_ERR_FLAGS = 4,      /* unknown flag bit, or a flag's companion input missing */
  KDA_ERR_BOUND = 5,      /* lower_bound outside [-5, 0), or scale not finite */
  KDA_ERR_ALIAS = 6,      /* an output overlaps an input (state_out == state_in is allowed),
                             or a state pool's state_out is neither NULL nor state_in */
  KDA_ERR_WORKSPACE = 7,  /* workspace NULL, too small or not 256-byte aligned */
  KDA_ERR_HIP = 8,        /* a HIP runtime call or kernel launch failed */
  KDA_ERR_CU_SEQLENS = 9, /* kda_debug_check_cu_seqlens found a contract violation */
  KDA_ERR_CONFIG = 10     /* rows_per_workgroup not 0, 16, 32, 64 or 128, segment_chunks
                             above 2^24, checkpoint_every not a multiple of 16 (or
                             negative), checkpoint_rows negative, or a state pool
                             with no slots, a pitch below H * 128 * 128 or not a
                             multiple of 8, or no state_in */
} kda_status;

enum {
  /* q <- q / sqrt(sum q^2 + 1e-6), same for k, per (token, head), before anything else */
  KDA_FLAG_L2NORM_QK = 1u << 0,
  /* g <- lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h, c])); needs A_log,
     dt_bias and lower_bound in [-5, 0) */
  KDA_FLAG_GATE_IN_KERNEL = 1u << 1,
  /* beta <- sigmoid(beta) */
  KDA_FLAG_BETA_IS_LOGIT = 1u << 2,
  /* fused form: also write every prepared record to the workspace's record area (for
     inspection; the workspace then includes that area). The separate preparation
     kernel always writes them. */
  KDA_FLAG_KEEP_RECORDS = 1u << 3
};

typedef struct kda_prefill_args {
  /* Inputs (device, contiguous, read only).
     q, k, v, g: [B, T, H, 128] of io_dtype. beta: [B, T, H] of io_dtype.
     Without KDA_FLAG_GATE_IN_KERNEL, g is the per-channel natural-log decay and must
     lie in [-5, 0] (16 tokens of it must keep exp(+-sum) finite, the K3 decay page's
     range argument); with it, g is the raw gate input. */
  const void *q, *k, *v, *g, *beta;
  /* [N, H, 128 (values), 128 (keys)] of state_dtype, or NULL for a zero initial state. */
  const void *state_in;
  /* int64 [N + 1] packed-varlen offsets (B must be 1, T = total tokens), or NULL for the
     fixed layout (N = B sequences of T tokens). Contract: cu[0] = 0, non-decreasing,
     cu[N] = T. Zero-length sequences are allowed and pass their state through. */
  const int64_t *cu_seqlens;
  /* FP32 [H] and [H, 128]; read only with KDA_FLAG_GATE_IN_KERNEL. */
  const float *A_log, *dt_bias;

  /* Outputs (device). o: [B, T, H, 128] of io_dtype, must not overlap any input.
     state_out: [N, H, 128, 128] of state_dtype, or NULL (no final state written);
     it may be exactly state_in (in-place update) but must not partially overlap it. */
  void *o;
  void *state_out;

  /* Caller-owned scratch of at least kda_prefill_workspace_bytes() bytes, 256-byte
     aligned. After a successful call it holds the prepared per-chunk records whose
     layout is given below. */
  void *workspace;
  size_t workspace_bytes;

  int64_t B, T, H, D, N; /* D must be 128; N = number of sequences */
  int32_t io_dtype;      /* kda_dtype of q, k, v, g, beta and o */
  int32_t state_dtype;   /* kda_dtype of state_in and state_out */
  float scale;           /* output scale s; 0 selects 1/sqrt(128) */
  float lower_bound;     /* gate lower bound, in [-5, 0); used with the gate flag */
  uint32_t flags;        /* KDA_FLAG_* */

  /* Launch geometry: value rows handled by one workgroup of the recurrence (each
     compute wave owns 16 rows). 0 = automatic: in the serial form the smallest of 16,
     32 and 64 that keeps N * H * 128 / rows within the device's compute units, else
     128 for BF16 I/O (64 for FP32); in the segmented form 64, or 128 for BF16 I/O
     from N * H = 10 on (past N * H = 32 in the fused form). 16/32/64/128 force it.
     For a given segment_chunks, results are bitwise identical for every choice. */
  int32_t rows_per_workgroup;

  /* Time segments of the recurrence. The chunk-to-chunk carry is affine in the state,
     so a sequence can be cut into segments of this many chunks that run in parallel:
     each later segment's transition Phi (128 x 128) and zero-start run are computed
     first, and the segment start states are then combined serially (one 128x128x128
     product per segment). Without checkpoints (the affine-output form) the first pass
     also writes each later segment's zero-start output into o and the output of its
     transition run (Qt Phi^T per chunk) into the workspace, the combine's last step
     writes the final state, and a parallel pass adds (Qt Phi^T) S_p^T to o: a critical
     path of about one segment plus the combine. With many segments (fixed layout) one
     carry-and-output launch replaces the combine and that pass: each later segment's
     workgroups form their own start state by the chain of transitions and then add its
     output term (see scan_c_workgroups). With checkpoints every later segment
     is instead re-run from its true start (the states inside it are needed): about two
     segments. Either way about twice or three times the recurrence work buys the
     shorter path, which pays off when few (sequence, head) pairs leave compute units
     idle. 0 = automatic: P segments (of at least 16 chunks) such that the first pass
     has about one workgroup per compute unit of a 256-CU device, with the segmented
     form's automatic rows (see rows_per_workgroup) unless rows_per_workgroup says
     otherwise, taken when P >= 3, or P >= 2 with N * H <= 32; negative = never
     (one serial run per sequence); positive = this many chunks per segment. Results
     differ from the serial form only by rounding. */
  int32_t segment_chunks;

  /* State checkpoints, as in the "flashinfer.kda_prefill" page's contract (section
     "State and graph semantics"). checkpoint_every: the interval in tokens, a positive
     multiple of 16, or 0 (no checkpoints). When set, every non-empty sequence n writes
     ceil(len_n / checkpoint_every) states, the states before each interval: row
     checkpoint_cu_starts[n] + r of state_checkpoints holds the state after
     r * checkpoint_every tokens of the sequence (r = 0: its initial state). An empty
     sequence writes none.
     state_checkpoints: [checkpoint_rows, H, 128 (values), 128 (keys)] of state_dtype,
     device, 16-byte aligned, write only, must not overlap any other buffer; it may be
     NULL when checkpoint_rows is 0 (nothing is written then).
     checkpoint_cu_starts: int64 [N + 1] device, the caller's row offsets (on the page's
     contract, cu[0] = 0 and cu[n + 1] - cu[n] = ceil(len_n / checkpoint_every); they
     are device data and not checked on the host). Rows at or beyond checkpoint_rows are
     never written, whatever the offsets say. */
  int64_t checkpoint_every;
  int64_t checkpoint_rows;
  void *state_checkpoints;
  const int64_t *checkpoint_cu_starts;

  /* State pool (the "flashinfer.kda_prefill" page, section "State and graph
     semantics"). ssm_state_indices: int32 [N] device, or NULL. When set, state_in is a
     caller-owned pool of state_pool_slots slots of [H, 128, 128] (state_dtype), slot j
     starting state_slot_pitch elements after slot j - 1 (0 = H * 128 * 128; otherwise at
     least that and a multiple of 8), and sequence n starts from slot
     ssm_state_indices[n] and writes its final state back to the same slot: state_in is
     required and state_out must be NULL or equal to state_in. Slot ids must be unique
     (caller contract, not checked); an id outside [0, state_pool_slots) makes that
     sequence start from zero and write no state. Checkpoints still go to
     state_checkpoints. */
  const int32_t *ssm_state_indices;
  int64_t state_pool_slots;
  int64_t state_slot_pitch;

  /* Scheduling order (the same page, section "Packed scheduling"): int32 [N] device, a
     permutation of [0, N) (caller contract, not checked), or NULL. The serial form
     starts the sequences' workgroups in this order, so ordering by decreasing length
     shortens the last partial wave. NULL: varlen calls with N <= 256 are ordered that
     way on the device (the plan kernel), other calls keep the natural order. Results do
     not depend on it. */
  const int32_t *seq_order;

  /* Optional timing hooks (host array of hipEvent_t handles, or NULL). When
     n_trace_events >= 3, the library records trace_events[0] before the first kernel,
     trace_events[1] between the preparation and recurrence kernels and
     trace_events[2] after the last recurrence kernel, all on the call's stream. When
     n_trace_events >= 5 it also records trace_events[3] after the first recurrence
     launch and trace_events[4] after the segment combine (both right after the
     recurrence in the serial form; trace_events[4] right after trace_events[3] when
     the carry-and-output launch replaces the combine). */
  void *const *trace_events;
  int32_t n_trace_events;

  /* Where the chunk preparation runs. Positive: fused into the recurrence; four
     producer waves in every recurrence workgroup prepare the chunks of its run from q,
     k, g, beta (and copy its V tile) straight into the LDS ring its compute waves read,
     one chunk per producer wave, handed over through LDS counters with bounded waits
     (the prepared records never go through HBM). 0 (automatic) or negative: a separate
     preparation kernel (one workgroup per chunk and head) writes the records to the
     workspace first and the recurrence streams them back. Results differ only by
     rounding. The fused form is this library's take on the producer / consumer overlap
     of the "CAKE KDA Prefill" page (sections "Owner-helper decomposition" and
     "Fine-grained K1-K2 overlap"); it moves about 1x the algorithmic HBM bytes instead
     of about 2.4x, but on MI355X its producers are slower than the separate kernel at
     every head count measured, which is why it is not the automatic choice. */
  int32_t fuse_prepare;
} kda_prefill_args;

/*
 * Workspace layout (bytes, from the workspace base; kda_prefill_plan reports the
 * offsets):
 *   [0, KDA_WS_HEADER)            varlen only: int64 cu_chunks[N + 1], the exclusive
 *                                 prefix of ceil(len_n / 16) (the flashinfer page's
 *                                 compact chunk prefix, section "Packed scheduling"),
 *                                 then int64 cu_segs[N + 1], the prefix of the segment
 *                                 counts max(1, ceil(chunks_n / segment_chunks)), then
 *                                 int32 order[N]: in the serial form without a caller's
 *                                 seq_order (and N <= 256), the sequences by decreasing
 *                                 chunk count (ties by index), the order in which their
 *                                 work starts.
 *   [KDA_WS_HEADER, ...)          only with the separate preparation kernel or
 *                                 KDA_FLAG_KEEP_RECORDS: one KDA_WS_RECORD-byte record
 *                                 per (chunk c, head h) at index h * max_chunks + c,
 *                                 where c counts chunks over all sequences in order and
 *                                 max_chunks is the plan's bound (kda_prefill_plan):
 *                                 N * ceil(T / 16) for the fixed layout, (T + 15 N) / 16
 *                                 for varlen.
 *   scan_state_offset             segmented form only: FP32 [H][S] slots of 128 x 128,
 *                                 the start state (or zero-start end state) per
 *                                 segment, S = segments_per_head_bound; inside a slot,
 *                                 MFMA fragments [row block 8][key block 8][lane 64][4]
 *                                 with lane 16 g + m holding S[16 rb + m][16 b + 4 g + j].
 *                                 Launch A writes segment 0's end state S_1 into slot
 *                                 1 of the sequence, the zero-start end state Z_p of
 *                                 segment p into slot p + 1 and (affine-output form)
 *                                 the last segment's into the sequence's first slot.
 *                                 The combine then writes each start state S_p over
 *                                 slot p: in the affine-output form packed to BF16
 *                                 (blocks 2 kb and 2 kb + 1 as eight BF16 per lane
 *                                 over the FP32 fragment of block 2 kb). With the
 *                                 carry-and-output launch (combine_workgroups == 0)
 *                                 the slots are only read.
 *   scan_transition_offset        segmented form only: BF16 [H][S] slots of 128 x 128,
 *                                 each later segment's transition Phi, as fragments
 *                                 [key block 8][key group 4][lane 64][8] with lane
 *                                 16 g + m holding Phi[k][16 b + m] for the keys
 *                                 k = 32 kk + 16 (e / 4) + 4 g + e % 4.
 *   scan_output_offset            affine-output form only: [H][max_chunks] pieces of
 *                                 2048 elements of the io dtype, Qt Phi^T of each
 *                                 chunk of a later segment (Phi from the segment start
 *                                 to the chunk start), in the record's Qt layout.
 *   status_offset                 the last 256 bytes: int32 status. Bit 0 is set when a
 *                                 bounded wait of the fused form timed out (an internal
 *                                 failure; that call's outputs are then invalid). The
 *                                 library never clears it: a caller that checks it
 *                                 clears it before the call.
 * KDA_WS_HEADER = round_up((N + 1) * 16 + 4 N, 256) for varlen, 0 for the fixed layout.
 *
 * A record holds, for the chunk's 16 tokens (pad tokens of a short last chunk behave as
 * k = q = v = 0, g = 0, beta = 0), with the page's K_start, Q_start, K_end, D_{0:15},
 * A_kk = (I + R)^{-1} and A_qk and B = Diag(beta):
 *   Mb  = A_kk B                              (16 x 16)
 *   Kn  = -Mb K_start^T                       (16 tokens x 128 keys)
 *   Qt  = s Q_start^T + A_qk Kn               (16 tokens x 128 keys)
 * so that a chunk entering with state S gives U^T = Mb V^T + Kn S^T,
 * O^T = Qt S^T + A_qk Mb V^T and S_next^T = D_{0:15} S^T + K_end^T U^T.
 * Offsets inside a record (tok m, lane L = 16 * grp + m, key index
 * kappa(kb, grp, e) = 32 kb + 16 (e / 4) + 4 grp + (e % 4)):
 *   0      bf16 Kn [kb 4][L 64][e 8]          = Kn[m][kappa(kb, grp, e)]
 *   4096   bf16 Qt [kb 4][L 64][e 8]          = Qt[m][kappa(kb, grp, e)]
 *   8192   bf16 KeT[bp 4][L 64][h 2][j 4]     = K_end[4 grp + j][16 (2 bp + h) + m]
 *   12288  fp32 D  [L 64][c 2]                = D_{0:15}[16 (m / 2) + 4 grp + 2 (m % 2) + c]
 *   12800  bf16 MA [L 64][Mb j 4, A_qk j 4]   = Mb[m][4 grp + j], A_qk[m][4 grp + j]
 * (each lane's operands are one contiguous 8- or 16-byte piece; D is ordered so that
 * the 16 lanes of a row hold the 32 entries each of them needs, exchanged by a row
 * broadcast).
 */
#define KDA_WS_RECORD 13824

/* Host only; no HIP call. Validates shapes, dtypes, flags and bound, and stores the
   workspace size the call needs in *bytes. */
kda_status kda_prefill_workspace_bytes(const kda_prefill_args *a, size_t *bytes);

/* Host only; no HIP call. Every check kda_prefill does before launching (pointers,
   shapes, dtypes, flags, bound, aliasing, workspace size and alignment). */
kda_status kda_prefill_check(const kda_prefill_args *a);

/* Enqueue the whole prefill on `stream` (a hipStream_t; NULL = default stream).
   Asynchronous: no device synchronisation, no device-to-host read of cu_seqlens.
   Launch geometry uses the upper bound (T + 15 N) / 16 on the total chunk count. */
kda_status kda_prefill(const kda_prefill_args *a, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
   serving loops, harnesses that forbid hipMalloc): kda_prefill with the workspace taken
   from a static device array of KDA_NO_ALLOC_SCRATCH_BYTES bytes that the library holds
   on each device it runs on until the process ends (its address is resolved on the
   first call on a device). a->workspace must be NULL; every other argument, and all
   behaviour, is that of kda_prefill. Calls whose kda_prefill_workspace_bytes exceed
   KDA_NO_ALLOC_SCRATCH_BYTES return KDA_ERR_WORKSPACE before any launch. The call makes
   no hipMalloc or hipFree. All calls on one device share its array and nothing in it
   needs clearing between calls; calls that overlap in time on one device (on different
   streams, or from several threads) race on it and must be serialised by the caller. */
#define KDA_NO_ALLOC_SCRATCH_BYTES (64ull << 20)
kda_status kda_prefill_no_alloc(const kda_prefill_args *a, void *stream);

/* Static description of a status code. */
const char *kda_status_string(kda_status s);

/* Detail of the last failure on the calling thread (empty string if none). */
const char *kda_last_error(void);

/* Tests only: copies cu_seqlens to the host (synchronising `stream`) and checks
   cu[0] = 0, non-decreasing entries and cu[N] = T. Returns KDA_OK or KDA_ERR_CU_SEQLENS. */
kda_status kda_debug_check_cu_seqlens(const int64_t *cu_seqlens, int64_t N, int64_t T,
                                      void *stream);

/* Launch geometry the call would use (host only): recurrence rows per workgroup,
   workgroup count of each kernel, the upper bound on the chunk count and the
   segmented form's parameters. num_cus only affects the automatic row choice of the
   serial form (0 = 256). */
typedef struct kda_plan_info {
  int32_t rows_per_workgroup;
  int32_t waves_per_workgroup;     /* compute + loader waves of a recurrence workgroup */
  int64_t recurrence_workgroups;   /* serial launch, or the first segmented launch; the
                                      recurrence launches round their grids up to a
                                      multiple of 8 (one round over the XCDs), and the
                                      extra workgroups exit at once */
  int64_t prepare_workgroups;
  int64_t max_chunks;
  size_t workspace_header_bytes;
  int64_t segment_chunks;          /* 0: serial form */
  int64_t segments_per_head_bound; /* scan slots per head */
  int64_t combine_workgroups;      /* 0 when the carry-and-output launch replaces it */
  int64_t scan_c_workgroups;       /* the re-run launch, or the affine-output form's
                                      scan-output launch, or its carry-and-output launch
                                      (fixed layout, seven or more segments per
                                      sequence, ten or more when H * N * (P - 1) * 4
                                      exceeds 256: four 32-row blocks per later segment,
                                      each forming its start state from S_1 and then
                                      its output term; the last ones also the final
                                      state) */
  size_t scan_state_offset;
  size_t scan_transition_offset;
  int32_t decode;                  /* 1: the token-loop kernel (1 <= T <= 8, see above) */
  int32_t scan_affine_output;      /* 1: the affine-output segmented form */
  size_t scan_output_offset;
  int32_t fused;                   /* 1: the chunk preparation runs in the recurrence */
  int32_t has_records;             /* 1: the workspace holds the records */
  size_t records_offset;           /* where they start (the header's end) */
  size_t status_offset;            /* the 256-byte status block */
} kda_plan_info;
kda_status kda_prefill_plan(const kda_prefill_args *a, int32_t num_cus, kda_plan_info *out);

int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
