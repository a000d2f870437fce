// Launch parameters shared by the host entry points and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;          // head dimension (keys = values = 128)
constexpr int kC = 16;           // tokens per chunk
constexpr int kRecord = 13824;   // bytes of one prepared (chunk, head) record
constexpr int kOffKn = 0;        // bf16 [kb 4][L 64][e 8]
constexpr int kOffQt = 4096;     // bf16 [kb 4][L 64][e 8]
constexpr int kOffKeT = 8192;    // bf16 [bp 4][L 64][half 2][j 4]
constexpr int kOffD = 12288;     // fp32 [L 64][2] (row-broadcast order)
constexpr int kOffMbAq = 12800;  // bf16 [L 64][Mb 4, A_qk 4]

// Recurrence launch modes: one serial run per sequence, or the launches of the
// segmented (time-parallel) form.
constexpr int32_t kModeSerial = 0;
constexpr int32_t kModeScanA = 1;  // segment 0 (true start) + Z_p, Phi_p of later segments
constexpr int32_t kModeScanC = 2;  // segments 1..P-1 again from their true start states

// Longest fixed-layout sequence the token-loop kernel takes (automatic geometry, no
// checkpoints); longer calls use the chunked path, which was faster from 16 tokens on
// at every shape measured (8 tokens: the token loop by 1.2-1.3x).
constexpr int kDecodeMaxT = 8;

// Largest sequence count for which the varlen plan orders the sequences by decreasing
// length (one workgroup, one sequence per thread).
constexpr int kAutoOrderMax = 256;

// Chunks per workgroup of the scan-output launch (affine-output segmented form).
constexpr int kScanOutChunks = 4;

constexpr uint32_t kFlagL2 = 1u << 0;
constexpr uint32_t kFlagGate = 1u << 1;
constexpr uint32_t kFlagBetaLogit = 1u << 2;

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const void* state_in;
  const int64_t* cu_seqlens;  // null: fixed layout
  const float* A_log;
  const float* dt_bias;
  void* o;
  void* state_out;
  int64_t* cu_chunks;         // workspace header (varlen only)
  unsigned char* records;     // workspace records
  int64_t B, T, H, N;
  int64_t max_chunks;         // prepare grid width (upper bound on chunks)
  int64_t chunks_per_seq;     // fixed layout: ceil(T / 16)
  float scale;
  float lower_bound;
  uint32_t flags;
  int32_t waves;              // recurrence compute waves per workgroup (16 rows each)
  // Segmented form (modes A and C and the combine kernel).
  int32_t mode;               // kModeSerial / kModeScanA / kModeScanC
  int32_t blocks;             // row blocks per task of this launch (A: 256 / rows, C: 128 / rows)
  int64_t seg_len;            // chunks per segment
  int64_t segs_per_seq;       // fixed layout: segments per sequence
  int64_t seg_stride;         // scan slots per head (bound on the total segment count)
  int64_t* cu_segs;           // varlen: [N + 1] prefix of segments per sequence
  float* scan_s;              // FP32 [H][seg_stride][128][128]: S_p, Z_p
  unsigned short* scan_phi;   // BF16 [H][seg_stride][128 keys][128 rows]: Phi_p transposed
  // Affine-output form: launch A also runs segment P-1 and writes O of the zero-start
  // runs into o and O of the transition runs (Qt Phi^T per chunk) into scan_q; the
  // combine's last step writes the final state; the scan-output launch then adds
  // (Qt Phi^T) S_p^T to o instead of rerunning the segments.
  int32_t affine_out;
  void* scan_q;               // IO dtype [H][max_chunks][kb 4][lane 64][8]
  // State checkpoints (ckpt_every chunks apart; 0 = none).
  void* ckpt;                 // [ckpt_rows][H][128][128] of the state dtype
  const int64_t* ckpt_cu;     // [N + 1] row offsets
  int64_t ckpt_every;         // chunks between checkpoints
  int64_t ckpt_rows;
  // State pool (null: state n at [n][H][128][128]) and scheduling order.
  const int32_t* state_idx;   // [N] slot of each sequence
  int64_t pool_slots;
  int64_t slot_pitch;         // elements between slots
  const int32_t* seq_order;   // [N] or null
  // Fused form: the recurrence workgroups prepare their own chunks (no records in HBM).
  int32_t fused;
  int32_t keep_records;       // fused: also write each record to `records` (inspection)
  int* status;                // fused: bit 0 set when an internal bounded wait timed out
};

// auto_order: null, or [N] int32 (N <= kAutoOrderMax) for the sequences by decreasing
// chunk count.
hipError_t launch_plan(const Params& p, int32_t* auto_order, hipStream_t stream);
hipError_t launch_prepare(const Params& p, bool io_bf16, hipStream_t stream);
int recurrence_loader_waves(int compute_waves);
hipError_t launch_recurrence(const Params& p, int64_t workgroups, bool io_bf16,
                             bool state_bf16, hipStream_t stream);
// The recurrence launch of the fused form (p.fused): same workgroups, producer waves
// instead of loader waves (kda_fused.hip).
hipError_t launch_fused_recurrence(const Params& p, int64_t workgroups, bool io_bf16,
                                   bool state_bf16, hipStream_t stream);
hipError_t launch_combine(const Params& p, bool state_bf16, hipStream_t stream);
hipError_t launch_scan_output(const Params& p, int64_t workgroups, bool io_bf16,
                              hipStream_t stream);
// The affine-output form's last launch when it replaces the combine and the scan output
// (fixed layout): start states by the chain of transitions, then the output term of
// every later segment, and the final state (kda_recurrence.hip).
hipError_t launch_carry_out(const Params& p, int64_t workgroups, bool io_bf16, bool state_bf16,
                            hipStream_t stream);
hipError_t launch_decode(const Params& p, bool io_bf16, bool state_bf16, hipStream_t stream);

}  // namespace kda
