// kda_recurrence: the state carry across chunks, serial or in time-parallel segments.
//
// The "FlashKDA column split" post, section 3.1 ("Every value column is independent"),
// shows that in the transposed form
//   U^T = A_kk B (V^T - K_start^T S^T),  O^T = s Q_start^T S^T + A_qk U^T,
//   S_{c+1}^T = D_{0:15} S^T + K_end^T U^T
// each value row of S follows its own recurrence, so a head's 128 value rows can be
// split over compute units with no synchronisation between them. Section 3.3
// ("Keeping the state in registers") keeps the state slice in registers for the whole
// sequence; on CDNA the MFMA accumulator layout of a 16x16 block already is the
// B-operand layout (up to a fixed permutation of the key order, which the preparation
// kernel applies to the key-side operands), so no transpose is needed.
//
// With the record folded by kda_prepare (Mb = A_kk B, Kn = -Mb K_start^T,
// Qt = s Q_start^T + A_qk Kn), one chunk for the 16 value rows of one wave is
//   UV    = Mb V^T                      (16x16x16 MFMA)
//   U^T   = Kn S^T + UV                 (4 x 16x16x32 MFMA, the serial chain)
//   S^T   = D (.) S^T + K_end^T U^T     (8 x 16x16x16 MFMA, the serial chain)
//   O     = S_old Qt^T + UV^T A_qk^T    (uses the entering state only)
// State is FP32 in registers; MFMA operands are BF16.
//
// Segments. The carry is affine in the state: over a run of chunks, S_end = S_start Phi
// + Z, where Z is the end state of the run started from zero and Phi (128 x 128, keys x
// keys) the end state of the run started from the identity with V = 0 (rows of S never
// interact, so Phi's rows are computed exactly like value rows). The output is affine
// in the start state too: inside segment p, O_c = O^Z_c + (Qt_c Phi_{p,c}^T) S_p^T, where
// O^Z_c is the zero-start run's output and Qt_c Phi_{p,c}^T what the transition run
// outputs (its V is zero). A sequence cut into segments 0..P-1 of L chunks is evaluated
// in three launches (the affine-output form):
//   A: segment 0 from the true initial state (writing its O and S_1), and, for
//      segments 1..P-1, Z_p and O^Z (into o) and Phi_p and Qt Phi^T (into scan_q);
//   B: S_{p+1} = S_p Phi_p + Z_p for p = 1..P-1 (kda_combine_kernel), the last step
//      giving the final state;
//   C: o += (Qt Phi^T) S_p^T for every chunk of segments 1..P-1, in parallel
//      (kda_scan_output_kernel).
// Calls with state checkpoints need the states inside the later segments and take the
// re-run form instead: A computes Z_p and Phi_p of segments 1..P-2 only, B stops at
// S_{P-1}, and C runs segments 1..P-1 again from S_p with this kernel, writing O, the
// checkpoints and, for the last one, the final state.
// Workgroups of launch A see a 256-row space: rows 0..127 are value rows (Z or the true
// run), rows 128..255 the rows of Phi. Serial mode (one segment per sequence) is the
// single launch of the plain recurrence.
//
// Workgroup. W compute waves (16 value rows each, W = 1, 2, 4, 8) plus NL loader waves.
// The loaders stream each chunk's record and V tile with 16-byte loads, DEPTH chunks
// ahead in registers, into a 4-slot LDS ring; one s_barrier per chunk publishes a slot.
// (LDS-DMA loads deliver only ~16 B/clock.) Compute waves touch LDS and registers only.
//
// Ring protocol, iteration c:
//   loaders: issue the loads of chunk c+1+DEPTH, write chunk c+2 into slot (c+2)%4,
//            wait for their own LDS writes of chunk c+1 (issued in iteration c-1),
//            barrier B_c;
//   compute: barrier B_c, read all of chunk c+1's operands (slot (c+1)%4), compute c
//            (operands read in the previous iteration), store the O of chunk c-1.
// A chunk is written one iteration before the barrier that publishes it, so no wave
// waits for LDS writes it has just issued, and the global loads go out before the LDS
// writes, which queue behind the compute waves' reads (measured: a loader that wrote,
// waited for its writes, then issued its loads set the chunk time). Slot (c+2)%4 last
// held chunk c-2, whose reads were consumed before B_{c-1}; the loaders write it after
// B_{c-1}.

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kSlots = 4;
constexpr int kRecUnits = kRecord / 16;  // 864 sixteen-byte units per record

typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Wait for this wave's LDS operations, then meet the other waves. No fence: global
// loads and stores in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// Meet the other waves without waiting for this wave's own LDS operations. A compute
// wave's reads are consumed, and so complete, before it reaches the barrier after next
// (the first after which their slot is rewritten); a loader waits for its writes at
// the start of its next iteration, before the barrier that publishes them.
__device__ __forceinline__ void read_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

constexpr int loader_waves(int w) { return w < 4 ? 2 : 4; }
constexpr int block_threads(int w) { return 64 * (w + loader_waves(w)); }

template <int V>
struct IntC {
  static constexpr int value = V;
};

// f(IntC<0>), ..., f(IntC<N - 1>), in order.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    unroll<N, I + 1>(f);
  }
}

template <bool BF16IO, int W>
struct Tile {
  static constexpr int NL = loader_waves(W);              // loader waves
  static constexpr int ES = BF16IO ? 2 : 4;
  static constexpr int NT = 64 * (W + NL);                // threads in the workgroup
  static constexpr int LT = 64 * NL;                      // loader threads
  static constexpr int VROW = 16 * W * ES;                // bytes of one V-tile token row
  static constexpr int PARTS = VROW / 16;                 // 16-byte pieces per token row
  static constexpr int REAL = kRecUnits + VROW;           // record + V-tile units (16 B)
  static constexpr int K = (REAL + LT - 1) / LT;          // loads per loader thread per chunk
  static constexpr int DEPTH = K <= 5 ? 4 : 3;            // chunks in flight per loader
  static constexpr int SLOT = K * LT * 16;                // padded ring slot
  static_assert(K * (DEPTH - 1) <= 63, "vmcnt range");
  static_assert(DEPTH >= 2, "loader pipeline");
  static_assert(kSlots * SLOT <= 98304, "LDS ring");  // of gfx950's 160 KB per CU
};

// Scan slots hold MFMA fragments, so that every access to them is one contiguous 1 KB
// piece per wave instruction:
// - states (FP32, 128 x 128): [row block rb 8][key block b 8][lane 64][4], lane
//   L = 16 grp + m holding S[16 rb + m][16 b + 4 grp + j] (the accumulator layout);
// - transitions Phi^T (BF16, 128 x 128): [output key block b 8][key group kk 4][lane
//   64][8], lane L = 16 grp + m holding Phi[k][16 b + m] for the eight keys
//   k = 32 kk + 16 (e / 4) + 4 grp + e % 4 (the 16x16x32 A-operand layout; Phi^T is the
//   A operand of the combine).
__device__ __forceinline__ int64_t state_frag(int rb, int b, int lane) {
  return ((rb * 8 + b) * 64 + lane) * 4;  // in floats
}

// Where one workgroup's run starts, what it reads and what it writes.
enum StartKind : int { kStartIn = 0, kStartZero = 1, kStartIdentity = 2, kStartScan = 3 };

struct Task {
  int64_t tok0;       // first token of the run (row index into [B*T] / packed tokens)
  int64_t tok_end;    // end token of the run's sequence
  int64_t rec_chunk;  // index of the run's first record in the head's record stream
  int64_t nch;        // chunks in the run
  int64_t sh;         // sequence * H + head
  int64_t h;
  int64_t n;          // sequence
  int64_t c0s;        // chunk index of the run's first chunk within its sequence
  int vwg;            // first row of the workgroup within its 128-row space
  int start;          // StartKind
  bool vzero;         // V = 0 (rows of Phi)
  bool out;           // write O
  bool final_state;   // write state_out
  const float* s_src; // kStartScan: FP32 [128][128] start state
  float* s_dst;       // FP32 [128][128] end state (scan), or null
  unsigned short* phi_dst;  // BF16 [128 keys][128 rows] end state transposed, or null
};

__device__ __forceinline__ int64_t task_index() {
  // XCD-aware order: workgroup b runs on XCD b % 8; consecutive tasks (the row blocks of
  // one run, which read the same records) go to the same XCD's L2. The grid is a
  // multiple of 8 (launch_recurrence pads it); tasks past the real count decode to no
  // work.
  const int64_t total = gridDim.x;
  const int64_t bid = blockIdx.x;
  return (bid % 8) * (total / 8) + bid / 8;
}

// Token and chunk range of sequence n (the varlen plan's prefix, or the fixed layout).
__device__ __forceinline__ void seq_range(const Params& p, int64_t n, int64_t& start,
                                          int64_t& end, int64_t& chunk0, int64_t& nch) {
  if (p.cu_seqlens) {
    start = p.cu_seqlens[n];
    end = min(p.cu_seqlens[n + 1], p.T);
    chunk0 = p.cu_chunks[n];
  } else {
    start = n * p.T;
    end = start + p.T;
    chunk0 = n * p.chunks_per_seq;
  }
  nch = end > start ? (end - start + kC - 1) / kC : 0;
  if (chunk0 < 0) nch = 0;
  if (chunk0 + nch > p.max_chunks) nch = p.max_chunks > chunk0 ? p.max_chunks - chunk0 : 0;
}

// Segments of sequence n and the global index of its first one.
__device__ __forceinline__ void seq_segments(const Params& p, int64_t n, int64_t& first,
                                             int64_t& count) {
  if (p.cu_seqlens) {
    first = p.cu_segs[n];
    count = p.cu_segs[n + 1] - first;
  } else {
    first = n * p.segs_per_seq;
    count = p.segs_per_seq;
  }
}

__device__ bool segment_task(const Params& p, Task& t, int64_t h, int64_t n, int64_t seg,
                             int64_t first, int64_t nseg, int vr);

// Element offset of state row r of (sequence n, head h) in state_in / state_out (a pool
// slot with a state pool), or -1 when the sequence's slot id is out of range.
__device__ __forceinline__ int64_t state_row(const Params& p, int64_t n, int64_t h, int r) {
  if (p.state_idx) {
    const int64_t slot = p.state_idx[n];
    if (slot < 0 || slot >= p.pool_slots) return -1;
    return slot * p.slot_pitch + (h * kD + r) * kD;
  }
  return ((n * p.H + h) * kD + r) * kD;
}

__device__ bool decode_task(const Params& p, int rows, Task& t) {
  const int64_t task = task_index();
  const int64_t H = p.H;
  t.vzero = false;
  t.out = true;
  t.final_state = true;
  t.s_src = nullptr;
  t.s_dst = nullptr;
  t.phi_dst = nullptr;
  if (p.mode == kModeSerial) {
    // Pairs (sequence slot s, head h), h fastest, are dispatched round-robin over the
    // XCDs (workgroup b runs on XCD b % 8), so that every XCD gets a share of each
    // sequence; the bpp row blocks of one pair share an XCD (and its L2): pair
    // 8 (b / (8 bpp)) + b % 8, row block (b / 8) % bpp. Slot s runs sequence
    // seq_order[s] when an order is given.
    const int bpp = kD / rows;
    const int64_t b = blockIdx.x;
    const int64_t pair = (b / (8 * bpp)) * 8 + (b % 8);
    const int blk = static_cast<int>((b / 8) % bpp);
    if (pair >= p.N * H) return false;
    const int64_t slot = pair / H;
    const int64_t n = p.seq_order ? static_cast<int64_t>(p.seq_order[slot]) : slot;
    if (n < 0 || n >= p.N) return false;
    const int64_t sh = n * H + (pair - slot * H);
    int64_t start, end, chunk0, nch;
    seq_range(p, n, start, end, chunk0, nch);
    t.tok0 = start;
    t.tok_end = end;
    t.rec_chunk = chunk0;
    t.nch = nch;
    t.sh = sh;
    t.h = sh - n * H;
    t.n = n;
    t.c0s = 0;
    t.vwg = blk * rows;
    t.start = kStartIn;
    return true;
  }
  // Fixed layout: only the active row blocks are launched. Per sequence, launch A has
  // the b0 = 128 / rows value blocks of segment 0, then for segments 1 .. P-2 (1 .. P-1
  // in the affine-output form) the b0 value (Z) and b0 transition (Phi) blocks; launch
  // C the b0 value blocks of segments 1 .. P-1. Varlen: a bound of seg_stride slots x
  // p.blocks per head, decoded below.
  if (!p.cu_seqlens) {
    const int b0 = kD / rows;
    const int64_t P = p.segs_per_seq;
    const int64_t mid = p.affine_out ? P - 1 : P - 2;  // segments with Z and Phi runs
    const int64_t per_seq = p.mode == kModeScanA ? (P >= 2 ? b0 + 2 * b0 * mid : b0)
                                                 : (P - 1) * b0;
    if (per_seq <= 0) return false;
    const int64_t per_head = p.N * per_seq;
    const int64_t h = task / per_head;
    if (h >= H) return false;
    const int64_t rem = task - h * per_head;
    const int64_t n = rem / per_seq;
    int64_t u = rem - n * per_seq;
    int64_t seg;
    int vr;
    if (p.mode == kModeScanA) {
      if (u < b0) {
        seg = 0;
      } else {
        u -= b0;
        seg = 1 + u / (2 * b0);
        u -= (seg - 1) * 2 * b0;
      }
    } else {
      seg = 1 + u / b0;
      u -= (seg - 1) * b0;
    }
    vr = static_cast<int>(u) * rows;
    return segment_task(p, t, h, n, seg, n * P, P, vr);
  }
  const int blocks = p.blocks;
  const int64_t per_head = p.seg_stride * blocks;
  const int64_t h = task / per_head;
  const int64_t rem = task - h * per_head;
  const int64_t gsg = rem / blocks;
  const int blk = static_cast<int>(rem - gsg * blocks);
  if (h >= H) return false;
  int64_t n;
  {
    if (gsg >= p.cu_segs[p.N]) return false;
    int64_t lo = 0, hi = p.N - 1;  // largest n with cu_segs[n] <= gsg
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (p.cu_segs[mid] <= gsg) lo = mid;
      else hi = mid - 1;
    }
    n = lo;
  }
  int64_t first, nseg;
  seq_segments(p, n, first, nseg);
  const int64_t seg = gsg - first;
  const int vr = blk * rows;
  if (p.mode == kModeScanA) {
    if (!p.affine_out && nseg >= 2 && seg == nseg - 1) return false;  // only in the re-run
    if (vr >= kD && seg == 0) return false;           // no transition for segment 0
  } else if (seg == 0) {
    return false;                                     // segment 0: only in launch A
  }
  return segment_task(p, t, h, n, seg, first, nseg, vr);
}

// Task of row block vr (0 .. 255 in launch A: value rows, then the rows of Phi) of
// segment seg of sequence n (global segments first .. first + nseg - 1) of head h.
__device__ bool segment_task(const Params& p, Task& t, int64_t h, int64_t n, int64_t seg,
                             int64_t first, int64_t nseg, int vr) {
  if (seg < 0 || seg >= nseg || first < 0 || first + nseg > p.seg_stride) return false;
  const int64_t gsg = first + seg;
  int64_t start, end, chunk0, nch;
  seq_range(p, n, start, end, chunk0, nch);
  const int64_t H = p.H;
  const int64_t c0 = seg * p.seg_len;
  const int64_t c1 = min(c0 + p.seg_len, nch);
  t.tok0 = start + c0 * kC;
  t.tok_end = end;
  t.rec_chunk = chunk0 + c0;
  t.nch = c1 > c0 ? c1 - c0 : 0;
  t.sh = n * H + h;
  t.h = h;
  t.n = n;
  t.c0s = c0;
  const int64_t slot = h * p.seg_stride + gsg;  // scan slot of this segment
  if (p.mode == kModeScanA) {
    if (vr < kD) {
      t.vwg = vr;
      t.start = seg == 0 ? kStartIn : kStartZero;
      t.out = seg == 0 || p.affine_out;  // affine-output form: O of the zero start
      t.final_state = nseg == 1;
      if (nseg >= 2) {
        // S_1 (segment 0) or Z_seg into slot seg + 1; the last segment's Z (affine-output
        // form only) into the sequence's first slot, which never holds a start state.
        const int64_t zs = seg == nseg - 1 ? h * p.seg_stride + first : slot + 1;
        t.s_dst = p.scan_s + zs * (kD * kD);
      }
    } else {
      t.vwg = vr - kD;
      t.start = kStartIdentity;
      t.vzero = true;
      t.out = p.affine_out;  // affine-output form: Qt Phi^T per chunk into scan_q
      t.final_state = false;
      t.phi_dst = p.scan_phi + slot * (kD * kD);
    }
    return true;
  }
  // launch C of the re-run form
  t.vwg = vr;
  t.start = kStartScan;
  t.s_src = p.scan_s + slot * (kD * kD);
  t.final_state = seg == nseg - 1;
  return true;
}

struct ChainIn {  // operands of the chunk's first products
  bf16x8 kn[4];
  i16x4 mb;
  i16x4 aq;
  i16x4 vv;
};

struct TailIn {  // operands of the state update and the output
  u32x4 ke[4];  // K_end^T blocks 2 bp and 2 bp + 1 (8 bytes each)
  f32x2 dv;     // this lane's pair of D_{0:15} entries (row-broadcast order)
  bf16x8 qt[4];
};

template <bool BF16IO, int W>
__device__ __forceinline__ void read_chain(ChainIn& x, const lds_u8* slot, int lane, int w,
                                           int64_t nvalid) {
  using T = Tile<BF16IO, W>;
  const int m = lane & 15;
  const int grp = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    x.kn[kb] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
        slot + kOffKn + kb * 1024 + lane * 16);
  const u32x4 ma =
      *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(slot + kOffMbAq + lane * 16);
  x.mb = __builtin_bit_cast(i16x4, u32x2{ma[0], ma[1]});
  x.aq = __builtin_bit_cast(i16x4, u32x2{ma[2], ma[3]});
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = 4 * grp + j;
    const lds_u8* q = slot + kRecord + tok * T::VROW + (16 * w + m) * T::ES;
    short s;
    if constexpr (BF16IO)
      s = *reinterpret_cast<const __attribute__((address_space(3))) short*>(q);
    else
      s = static_cast<short>(float_to_bf16_bits(
          *reinterpret_cast<const __attribute__((address_space(3))) float*>(q)));
    x.vv[j] = tok < nvalid ? s : static_cast<short>(0);
  }
}

// OUT: the operands of the output (Qt) are read only by runs that write O.
template <bool OUT>
__device__ __forceinline__ void read_tail(TailIn& x, const lds_u8* slot, int lane) {
#pragma unroll
  for (int bp = 0; bp < 4; ++bp)
    x.ke[bp] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        slot + kOffKeT + bp * 1024 + lane * 16);
  x.dv = *reinterpret_cast<const __attribute__((address_space(3))) f32x2*>(slot + kOffD + lane * 8);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if constexpr (OUT)
      x.qt[kb] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
          slot + kOffQt + kb * 1024 + lane * 16);
    else
      x.qt[kb] = bf16x8{};
  }
}

// Lane N of this lane's 16-lane row (DPP row broadcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}

// State block B (keys 16 B + 4 grp + j) times D: key 16 B + 4 grp + j sits in lane
// 2 B + j / 2 of the row, component j % 2.
template <int B>
__device__ __forceinline__ f32x4 decayed(f32x4 st, f32x2 dv) {
  f32x4 r;
  r[0] = st[0] * row_bcast<2 * B>(dv[0]);
  r[1] = st[1] * row_bcast<2 * B>(dv[1]);
  r[2] = st[2] * row_bcast<2 * B + 1>(dv[0]);
  r[3] = st[3] * row_bcast<2 * B + 1>(dv[1]);
  return r;
}

// S^T block B <- D (.) S^T + K_end^T U^T for B = I .. 7.
template <int I>
__device__ __forceinline__ void state_update(f32x4 (&st)[8], const TailIn& b, i16x4 up) {
  if constexpr (I < 8) {
    const u32x4 kp = b.ke[I / 2];
    const i16x4 ke = __builtin_bit_cast(i16x4, (I % 2) ? u32x2{kp[2], kp[3]} : u32x2{kp[0], kp[1]});
    st[I] = mfma16(ke, up, decayed<I>(st[I], b.dv));
    state_update<I + 1>(st, b, up);
  }
}

// One chunk for one wave: updates the state and returns O[value 4 grp + j][token m]
// (zero when OUT is false: runs that write no O skip its products).
template <bool OUT>
__device__ __forceinline__ f32x4 chunk_step(const ChainIn& a, const TailIn& b, f32x4 (&st)[8],
                                            bf16x8 (&sp)[4]) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // Every MFMA accumulation chain uses one opcode and starts from zero; results of the
  // 16x16x16 products are combined with VALU adds rather than fed to a 16x16x32
  // product as its accumulator input.
  const f32x4 uv = mfma16(a.mb, a.vv, zero);  // UV[token 4 grp + j][value m]
  f32x4 u = zero;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) u = mfma32(a.kn[kb], sp[kb], u);
  u += uv;
  const i16x4 up = pack4(u);
  const bf16x8 s0 = sp[0], s1 = sp[1], s2 = sp[2], s3 = sp[3];  // entering state
  state_update<0>(st, b, up);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) sp[kb] = pack8(st[2 * kb], st[2 * kb + 1]);
  if constexpr (!OUT) return zero;
  // O from the entering state (off the chain)
  f32x4 out = mfma32(s0, b.qt[0], zero);
  out = mfma32(s1, b.qt[1], out);
  out = mfma32(s2, b.qt[2], out);
  out = mfma32(s3, b.qt[3], out);
  out += mfma16(pack4(uv), a.aq, zero);
  return out;
}

// Loader waves: the run's chunks, global -> registers (DEPTH chunks ahead) -> LDS ring.
// Unit u = lt + k * LT of a chunk is record byte 16 u (u < 864), V-tile piece u - 864
// (token row, 16-byte part), or padding (re-reads record unit 0 into the slot's unused
// tail). Chunks past the run's end re-read its last chunk (in bounds, never used).
// OUT false: the record units that hold Qt (whole iterations k of the unit loop, for both
// loader widths) are neither loaded nor written.
// Loader units k of a chunk that a run without O skips (the Qt tile), and the number of
// LDS writes one loader wave issues per chunk.
template <typename T, bool OUT>
constexpr bool unit_skipped(int k) {
  return !OUT && k * T::LT >= kOffQt / 16 && (k + 1) * T::LT <= (kOffQt + 4096) / 16;
}
template <typename T, bool OUT>
constexpr int writes_per_chunk() {
  int n = 0;
  for (int k = 0; k < T::K; ++k) n += unit_skipped<T, OUT>(k) ? 0 : 1;
  return n;
}

// Wait until at most N of this wave's LDS operations are outstanding: as they complete
// in order, all but its N most recent ones are done.
template <int N>
__device__ __forceinline__ void lds_wait_n() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xc07f | (N << 8));  // lgkmcnt(N)
  compiler_fence();
}

template <bool BF16IO, typename T, bool OUT>
__device__ __forceinline__ void loader_loop(const Params& p, const Task& t, lds_u8* ring, int lt) {
  auto skipped = [](int k) { return unit_skipped<T, OUT>(k); };
  constexpr int KW = writes_per_chunk<T, OUT>();
  const int64_t vstride_b = p.H * kD * T::ES;
  const unsigned char* rec0 =
      p.records + (t.h * p.max_chunks + t.rec_chunk) * static_cast<int64_t>(kRecord);
  const int vcol = t.vzero ? 0 : t.vwg;  // Phi rows read no V (any in-bounds address)
  const unsigned char* v0 = static_cast<const unsigned char*>(p.v) +
                            (t.tok0 * p.H * kD + t.h * kD + vcol) * T::ES;
  const int64_t vchunk_b = kC * vstride_b;
  const int64_t nch = t.nch;
  // Per-unit source address of chunk 0 (then of the next chunk to load) and its step per
  // chunk. A V unit of a pad token (past the sequence end, only in a sequence's last
  // chunk) reads token row 0 instead.
  const unsigned char* base[T::K];
  uint32_t inc[T::K];
  int vtok[T::K];       // V token row of the unit, or -1 for a record unit
  int64_t vdrop[T::K];  // bytes back to token row 0 for a V unit
#pragma unroll
  for (int k = 0; k < T::K; ++k) {
    const int u = lt + k * T::LT;
    const int i = u - kRecUnits;
    if (i >= 0 && i < T::VROW && !t.vzero) {
      const int tok = i / T::PARTS;
      vtok[k] = tok;
      vdrop[k] = tok * vstride_b;
      base[k] = v0 + tok * vstride_b + (i - tok * T::PARTS) * 16;
      inc[k] = static_cast<uint32_t>(vchunk_b);
    } else {
      vtok[k] = -1;
      vdrop[k] = 0;
      base[k] = rec0 + (u < kRecUnits ? u * 16 : 0);
      inc[k] = kRecord;
    }
  }
  // Chunk j lives in register set j % NS: one set more than the DEPTH chunks in flight,
  // so that the set reloaded in an iteration held a chunk whose LDS writes were complete
  // before the previous barrier.
  constexpr int NS = T::DEPTH + 1;
  u32x4 r[NS][T::K];
  // Chunks are loaded in order, 0, 1, 2, ...: each unit keeps a running source pointer,
  // which stops at the run's last chunk (later loads re-read it, never used).
  int64_t jn = 0;  // the next chunk to load
  auto issue = [&](u32x4(&dst)[T::K]) {
    const int64_t j = jn < nch - 1 ? jn : nch - 1;
    const int64_t nvalid = t.tok_end - (t.tok0 + j * kC);
    if (nvalid >= kC) {
#pragma unroll
      for (int k = 0; k < T::K; ++k)
        if (!skipped(k)) dst[k] = *reinterpret_cast<const u32x4*>(base[k]);
    } else {
#pragma unroll
      for (int k = 0; k < T::K; ++k) {
        if (skipped(k)) continue;
        const unsigned char* src = base[k];
        if (vtok[k] >= nvalid) src -= vdrop[k];
        dst[k] = *reinterpret_cast<const u32x4*>(src);
      }
    }
    if (jn < nch - 1) {
#pragma unroll
      for (int k = 0; k < T::K; ++k) base[k] += inc[k];
    }
    ++jn;
  };
  // One ds_write_b128 per unit, written out as such, so that the wave's LDS operations
  // per chunk are exactly KW writes (the wait before each barrier counts them).
  const uint32_t ring_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
  auto put = [&](const u32x4(&src)[T::K], int slot) {
    const uint32_t s = ring_addr + static_cast<uint32_t>(slot * T::SLOT + lt * 16);
#pragma unroll
    for (int k = 0; k < T::K; ++k) {
      if (skipped(k)) continue;
      asm volatile("ds_write_b128 %0, %1" ::"v"(s + static_cast<uint32_t>(k * T::LT * 16)),
                   "v"(src[k])
                   : "memory");
    }
  };
#pragma unroll
  for (int d = 0; d < T::DEPTH; ++d) issue(r[d]);  // chunks 0 .. DEPTH - 1
  put(r[0], 0);
  issue(r[T::DEPTH]);  // chunk DEPTH, into the spare set
  put(r[1], 1);
  lds_barrier();  // B_{-1}: chunk 0 visible (chunk 1 written too)
  int slot = 1;  // slot of chunk c + 1
  // Iteration c: the set of chunk c (its writes, iteration c - 2, were complete before
  // B_{c-1}) is reloaded with chunk c + 1 + DEPTH, chunk c + 2 goes into the ring, and
  // once this wave's writes of chunk c + 1 (iteration c - 1) are done, barrier B_c
  // publishes chunk c + 1. No wave waits for the LDS writes it has just issued, which
  // queue behind the compute waves' reads of chunk c + 1, and the global loads go out
  // first (measured: a loader that wrote, waited for those writes, then issued its
  // loads set the chunk time). Whole groups of NS iterations are unrolled without
  // conditions so that the compiler's wait before each LDS write is for the oldest set
  // only (DEPTH - 1 chunks stay in flight). Chunks past the run's last are clamped reads
  // of it, written and never read.
  auto step = [&](auto load_c, auto put_c, int64_t c) {
    constexpr int lset = decltype(load_c)::value;  // set of chunk c
    constexpr int pset = decltype(put_c)::value;   // set of chunk c + 2
    issue(r[lset]);  // chunk c + 1 + DEPTH
    slot = slot + 1 == kSlots ? 0 : slot + 1;  // slot of chunk c + 2
    put(r[pset], slot);
    lds_wait_n<KW>();  // all but the writes just issued
    read_barrier();    // B_c: chunk c + 1 visible; chunk c + 2 at B_{c+1}
  };
  int64_t c0 = 0;
#pragma unroll 1
  for (; c0 + NS <= nch; c0 += NS)
    unroll<NS>([&](auto d) {
      constexpr int i = decltype(d)::value;
      step(IntC<i>{}, IntC<(i + 2) % NS>{}, c0 + i);
    });
  const int64_t rest = nch - c0;  // 0 .. NS - 1
  unroll<NS - 1>([&](auto d) {
    constexpr int i = decltype(d)::value;
    if (rest > i) step(IntC<i>{}, IntC<(i + 2) % NS>{}, c0 + i);
  });
}

// OUT: the run writes O (and carries the true state); CKPT: it also writes state
// checkpoints (a separate instantiation, so that runs without them keep a loop body
// with no checkpoint test in it).
template <bool BF16IO, bool BF16ST, int W, bool OUT, bool CKPT>
__device__ __forceinline__ void compute_loop(const Params& p, const Task& t, lds_u8* ring,
                                             int wave, int lane) {
  using T = Tile<BF16IO, W>;
  const int m = lane & 15;
  const int grp = lane >> 4;
  const int v0 = t.vwg + 16 * wave;  // first row of this wave
  const int64_t nch = t.nch;

  // State rows v0 + m, keys 16 b + 4 grp + j: the 16x16x16 accumulator layout.
  const int64_t srow = state_row(p, t.n, t.h, v0 + m);
  f32x4 st[8];
  bf16x8 sp[4];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int key = 16 * b + 4 * grp;
    if (t.start == kStartIn && p.state_in && srow >= 0) {
      st[b] = load4<BF16ST>(p.state_in, srow + key);
    } else if (t.start == kStartScan) {
      st[b] = load4<false>(t.s_src, state_frag(v0 >> 4, b, lane));
    } else if (t.start == kStartIdentity) {
#pragma unroll
      for (int j = 0; j < 4; ++j) st[b][j] = (v0 + m == key + j) ? 1.f : 0.f;
    } else {
      st[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) sp[kb] = pack8(st[2 * kb], st[2 * kb + 1]);

  const int64_t vstride = p.H * kD;
  auto nvalid_of = [&](int64_t c) -> int64_t {
    return t.vzero ? 0 : t.tok_end - (t.tok0 + c * kC);
  };
  if (nch > 0) {
    read_barrier();  // B_{-1}: chunk 0 visible
    ChainIn cur;
    read_chain<BF16IO, W>(cur, ring, lane, wave, nvalid_of(0));
    int cs = 0;  // slot of chunk c
    // The O of chunk c is stored in iteration c + 1, after that iteration's MFMA work
    // has been issued, so that its wait for chunk c's last products is hidden.
    f32x4 pend = {0.f, 0.f, 0.f, 0.f};
    // O[token m][rows v0 + 4 grp + j] goes to o. A transition run (affine-output form)
    // writes Qt Phi^T instead: its rows v0 + 4 grp + j are the keys of that product,
    // stored per chunk in the Qt operand layout [kb 4][lane 64][e 8] of scan_q (key
    // 32 kb + 16 (e / 4) + 4 grp + e % 4 of token m in lane 16 grp + m), which puts
    // this lane's four values in its own lane, block v0 / 32, elements 4 (v0 / 16 % 2) + j.
    void* obuf = p.o;
    int64_t ooff = (t.tok0 + m) * vstride + t.h * kD + v0 + 4 * grp;
    int64_t ostep = kC * vstride;
    if (t.vzero) {
      obuf = p.scan_q;
      ooff = (t.h * p.max_chunks + t.rec_chunk) * (4 * 64 * 8) + ((v0 >> 5) * 64 + lane) * 8 +
             ((v0 >> 4) & 1) * 4;
      ostep = 4 * 64 * 8;
    }
    auto store_out = [&](int64_t c, f32x4 val) {
      if (m < t.tok_end - (t.tok0 + c * kC)) store4<BF16IO>(obuf, ooff + c * ostep, val);
    };
    TailIn tail;
    read_tail<OUT>(tail, ring, lane);
    // State checkpoints (runs that write O are the runs that carry the true state): the
    // state before every chunk j of the sequence with j % ckpt_every == 0 goes to row
    // ckpt_cu[n] + j / ckpt_every, if that row exists.
    const int64_t ck_q = CKPT ? p.ckpt_every : 1;
    int64_t ck_c = 0, ck_row = 0;
    if constexpr (CKPT) {
      ck_c = (ck_q - t.c0s % ck_q) % ck_q;
      ck_row = p.ckpt_cu[t.n] + (t.c0s + ck_c) / ck_q;
    }
#pragma unroll 1
    for (int64_t c = 0; c < nch; ++c) {
      const int ns = cs + 1 == kSlots ? 0 : cs + 1;  // slot of chunk c + 1
      if constexpr (CKPT) {
        if (c == ck_c) {
          if (ck_row >= 0 && ck_row < p.ckpt_rows) {
            const int64_t crow = ((ck_row * p.H + t.h) * kD + v0 + m) * kD;
#pragma unroll
            for (int b = 0; b < 8; ++b) store4<BF16ST>(p.ckpt, crow + 16 * b + 4 * grp, st[b]);
          }
          ck_c += ck_q;
          ++ck_row;
        }
      }
      read_barrier();  // B_c: chunk c + 1 visible
      // All of chunk c + 1's operands are read here, one chunk ahead, so that their
      // latency (they queue behind the loaders' writes of chunk c + 2) is hidden by
      // chunk c's MFMA work.
      ChainIn nxt;
      TailIn ntail;
      read_chain<BF16IO, W>(nxt, ring + ns * T::SLOT, lane, wave, nvalid_of(c + 1));
      read_tail<OUT>(ntail, ring + ns * T::SLOT, lane);
      const f32x4 prev = pend;
      pend = chunk_step<OUT>(cur, tail, st, sp);
      if (OUT && c > 0) store_out(c - 1, prev);
      // Keep the reads in this iteration: without these uses the compiler sinks them to
      // the top of the next iteration, right before the MFMA chain that needs them.
      asm volatile("" ::"v"(nxt.kn[0]), "v"(nxt.kn[1]), "v"(nxt.kn[2]), "v"(nxt.kn[3]),
                   "v"(nxt.mb), "v"(nxt.aq), "v"(nxt.vv));
      asm volatile("" ::"v"(ntail.ke[0]), "v"(ntail.ke[1]), "v"(ntail.ke[2]), "v"(ntail.ke[3]),
                   "v"(ntail.dv));
      if constexpr (OUT)
        asm volatile("" ::"v"(ntail.qt[0]), "v"(ntail.qt[1]), "v"(ntail.qt[2]), "v"(ntail.qt[3]));
      cur = nxt;
      tail = ntail;
      cs = ns;
    }
    if (OUT) store_out(nch - 1, pend);
  }

  if (t.final_state && p.state_out && srow >= 0) {
#pragma unroll
    for (int b = 0; b < 8; ++b) store4<BF16ST>(p.state_out, srow + 16 * b + 4 * grp, st[b]);
  }
  if (t.s_dst) {
#pragma unroll
    for (int b = 0; b < 8; ++b) store4<false>(t.s_dst, state_frag(v0 >> 4, b, lane), st[b]);
  }
  if (t.phi_dst) {
    // This lane holds Phi[r][16 b + 4 grp + j] for row r = v0 + m: key r of output
    // key 16 b + m' (m' = 4 grp + j) sits in group kk = r / 32, lane 16 grp' + m',
    // element e with r % 32 = 16 (e / 4) + 4 grp' + e % 4. This wave's 16 rows fill
    // elements 4 h .. 4 h + 3 (h = v0 / 16 % 2) of every (b, lane) piece of group kk: the
    // values go through this wave's 2 KB of ring slot nch % 4 ([b 4][lane 64][4]), in two
    // halves of four key blocks, then out as one 8-byte store per lane and b. The
    // loaders last wrote that slot with chunk nch (a clamped copy) and waited for those
    // writes before barrier B_{nch-1}; the compute waves only read it after that barrier
    // (chunk nch, values unused, in this wave's own order before these writes). An empty
    // run never touched the ring.
    static_assert(W * 2048 <= T::SLOT, "Phi staging");
    lds_u8* stage = ring + (nch % kSlots) * T::SLOT + wave * 2048;
    const int r = v0 + m;
    const int kk = r >> 5;
    const int h = (r >> 4) & 1;
    const int grpp = (r & 15) >> 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<__attribute__((address_space(3))) unsigned short*>(
              stage + ((bb * 64 + 16 * grpp + 4 * grp + j) * 4 + (r & 3)) * 2) =
              float_to_bf16_bits(st[4 * half + bb][j]);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int b = 4 * half + bb;
        const u32x2 piece = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
            stage + (bb * 64 + lane) * 8);
        *reinterpret_cast<u32x2*>(t.phi_dst + ((b * 4 + kk) * 64 + lane) * 8 + 4 * h) = piece;
      }
    }
  }
}

// CK: the instantiation that writes state checkpoints, launched only when they are
// asked for (kept apart so that the common kernel's code is unaffected by it).
template <bool BF16IO, bool BF16ST, int W, bool CK>
// At most two waves per SIMD (256 registers each): with more room the compiler keeps
// the state in AGPRs and copies it through VGPRs every chunk for the decay multiply.
// The 128-row workgroup (12 waves) needs three waves per SIMD, 168 registers each.
__global__ __launch_bounds__(block_threads(W), W == 8 ? 3 : 2) void kda_recurrence_kernel(Params p) {
  using T = Tile<BF16IO, W>;
  static_assert(T::NT == block_threads(W), "block size");
  __shared__ __attribute__((aligned(16))) unsigned char ring_[kSlots * T::SLOT];
  lds_u8* ring = (lds_u8*)(ring_);  // address-space cast

  Task t;
  if (!decode_task(p, 16 * W, t)) return;  // uniform over the workgroup
  // The wave index as a scalar, so that the role branch below is uniform per wave.
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int lt = static_cast<int>(threadIdx.x) - 64 * W;
  if (t.out) {
    if (wave < W) compute_loop<BF16IO, BF16ST, W, true, CK>(p, t, ring, wave, lane);
    else if (t.nch > 0) loader_loop<BF16IO, T, true>(p, t, ring, lt);
  } else {
    if (wave < W) compute_loop<BF16IO, BF16ST, W, false, false>(p, t, ring, wave, lane);
    else if (t.nch > 0) loader_loop<BF16IO, T, false>(p, t, ring, lt);
  }
}

// Launch B of the segmented form: S_{p+1} = S_p Phi_p + Z_p, p = 1 .. P-2, for 16 value
// rows of one (sequence, head) per workgroup; in the affine-output form also p = P-1,
// whose result is the final state. In the transposed form S^T_{p+1} =
// Phi_p^T S_p^T + Z_p^T; wave w computes output key blocks 2 w and 2 w + 1 (eight
// 16x16x32 products). Phi_p^T, stored as A-operand fragments by launch A, is the A
// operand: one 1 KB contiguous load per wave and product, and a wave's slice of Phi
// (32 keys x 128) is read by that wave alone, so it goes straight to registers, three
// steps ahead together with Z (state fragments, like S). The new state, packed to BF16, is the B
// operand of the next step; the waves exchange their packed blocks through LDS.
// Per step a workgroup moves 32 KB of Phi, 8 KB of Z and 8 KB of S: the per-CU stream
// rate, not the products, sets the step time, hence 16 rows (8 workgroups) per pair.
constexpr int kCombineDepth = 3;  // steps of Phi and Z in flight per wave

struct CombineIn {
  u32x4 a[2][4];  // Phi^T operands: output block 2 w + i, input key group kk
  f32x4 z[2];     // Z rows v0 + m, keys 16 (2 w + i) + 4 grp + j
};

template <bool BF16ST>
__global__ __launch_bounds__(256) void kda_combine_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) unsigned char xch_[2 * 4 * 64 * 16];
  lds_u8* xbase = (lds_u8*)(xch_);  // address-space cast
  // Workgroup b runs on XCD b % 8. The 8 row blocks of one (sequence, head) pair read
  // the same Phi, so they go to one XCD: pair hn = 8 group + (b % 8), row block
  // (b / 8) % 8, group b / 64. Pairs past H N exit.
  const int64_t b = blockIdx.x;
  const int rb = static_cast<int>((b >> 3) & 7);
  const int64_t hn = (b >> 6) * 8 + (b & 7);
  const int64_t h = hn / p.N;
  const int64_t n = hn - h * p.N;
  if (h >= p.H) return;
  int64_t first, nseg;
  seq_segments(p, n, first, nseg);
  const int64_t last = p.affine_out ? nseg - 1 : nseg - 2;  // steps s = 1 .. last
  if (last < 1 || first < 0 || first + nseg > p.seg_stride) return;  // nothing to combine
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int64_t slot0 = h * p.seg_stride + first;
  float* sbase = p.scan_s + slot0 * (kD * kD);
  const unsigned char* pbase = reinterpret_cast<const unsigned char*>(p.scan_phi + slot0 * (kD * kD));
  // This lane's fragment offsets: output key blocks b = 2 wave + i of row block rb.
  const int64_t koff0 = state_frag(rb, 2 * wave, lane);
  const int64_t koff1 = state_frag(rb, 2 * wave + 1, lane);
  const int aoff = (2 * wave * 4 * 64 + lane) * 16;  // bytes: block 2 wave, group 0
  const int64_t srow = state_row(p, n, h, 16 * rb + (lane & 15));  // final state row

  auto fetch = [&](CombineIn& x, int64_t s) {
    s = s < last ? s : last;  // past the last step: re-read it (in bounds, unused)
    const unsigned char* ph = pbase + s * (kD * kD * 2) + aoff;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        x.a[i][kk] = *reinterpret_cast<const u32x4*>(ph + (i * 4 + kk) * 1024);
    // Z_s lives in slot s + 1; the last segment's (affine-output form) in slot 0.
    const float* z = sbase + (s + 1 < nseg ? s + 1 : 0) * (kD * kD);
    x.z[0] = load4<false>(z, koff0);
    x.z[1] = load4<false>(z, koff1);
  };
  // [parity 2][wave 4][lane 64] packed S^T blocks 2 w, 2 w + 1
  auto xch = [&](int parity, int w) {
    return reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(
        xbase + (parity * 4 + w) * 1024 + lane * 16);
  };

  // In the affine-output form the scan-output launch reads each start state S_p
  // (p = 1 .. P-1) as BF16 operands: the packed blocks 2 w, 2 w + 1 of a wave go over the
  // first of its two FP32 fragments in slot p, bytes this wave alone has read.
  auto put_packed = [&](float* slot, bf16x8 v) {
    *reinterpret_cast<bf16x8*>(slot + koff0) = v;
  };
  f32x4 st[2];
  {
    float* s1 = sbase + 1 * (kD * kD);
    st[0] = load4<false>(s1, koff0);
    st[1] = load4<false>(s1, koff1);
    const bf16x8 v = pack8(st[0], st[1]);
    *xch(1, wave) = v;  // S_1, read by step 1
    if (p.affine_out) put_packed(s1, v);
  }
  CombineIn in[kCombineDepth];
#pragma unroll
  for (int d = 0; d < kCombineDepth; ++d) fetch(in[d], 1 + d);
  lds_barrier();

  // Step s: S_{s+1} = S_s Phi_s + Z_s with operands in set (s - 1) % depth; the set is
  // then refilled with step s + depth. Whole groups of depth steps are unrolled without
  // conditions so that the compiler's wait before each step is for its own set only.
  auto step = [&](auto set_c, int64_t s) {
    constexpr int set = decltype(set_c)::value;
    bf16x8 sp[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sp[kk] = *xch(s & 1, kk);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f32x4 acc = zero;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma32(__builtin_bit_cast(bf16x8, in[set].a[i][kk]), sp[kk], acc);
      st[i] = acc + in[set].z[i];
    }
    const bf16x8 v = pack8(st[0], st[1]);
    *xch((s + 1) & 1, wave) = v;
    if (s + 1 < nseg) {
      float* out = sbase + (s + 1) * (kD * kD);  // S_{s+1} replaces Z_s
      if (p.affine_out) {
        put_packed(out, v);
      } else {
        store4<false>(out, koff0, st[0]);
        store4<false>(out, koff1, st[1]);
      }
    } else if (p.state_out && srow >= 0) {  // S_P: the final state
      store4<BF16ST>(p.state_out, srow + 16 * (2 * wave) + 4 * (lane >> 4), st[0]);
      store4<BF16ST>(p.state_out, srow + 16 * (2 * wave + 1) + 4 * (lane >> 4), st[1]);
    }
    fetch(in[set], s + kCombineDepth);
    lds_barrier();
  };
  int64_t s = 1;
#pragma unroll 1
  for (; s + kCombineDepth - 1 <= last; s += kCombineDepth)
    unroll<kCombineDepth>([&](auto d) { step(d, s + decltype(d)::value); });
  unroll<kCombineDepth - 1>([&](auto d) {
    if (s + decltype(d)::value <= last) step(d, s + decltype(d)::value);
  });
}

// Scan-output launch of the affine-output form. Over segment p the state is affine in
// its start state: S_c = S_p Phi_{p,c} + Z_{p,c}, so the output of chunk c is
// O_c = O^Z_c + (Qt_c Phi_{p,c}^T) S_p^T, where O^Z_c is the output of the zero-start
// run and Qt_c Phi_{p,c}^T the output of the transition run, both written by launch A
// (into o and scan_q). Every chunk of segments 1 .. P-1 is then independent: this
// launch adds the second term to o, kScanOutChunks chunks of one segment per
// workgroup, wave w for values 32 w .. 32 w + 31 (row blocks 2 w, 2 w + 1). Per chunk a
// wave runs eight 16x16x32 products with S_p (BF16, packed by the combine) as the A
// operand and the chunk's Qt Phi^T fragments (four contiguous 1 KB pieces) as the B
// operand. The launch moves little data (the o term is read and written once, Qt Phi^T
// read once), so it is bound by load latency: small workgroups, all resident in one
// round.
template <bool BF16IO>
struct ScanOutIn {
  bf16x8 q[4];  // Qt Phi^T fragments of the chunk
  // O^Z[token m][values 16 rb + 4 grp + j], rb = 2 w + i, as loaded (BF16 pairs are
  // widened when used: two registers per piece instead of four, so that four
  // workgroups fit per CU)
  typename std::conditional<BF16IO, u32x2, f32x4>::type oz[2];
};

template <bool BF16IO>
__device__ __forceinline__ bf16x8 load_frag(const void* base, int64_t idx) {
  if constexpr (BF16IO) {
    return *reinterpret_cast<const bf16x8*>(static_cast<const unsigned short*>(base) + idx);
  } else {
    const f32x4* f = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
    return pack8(f[0], f[1]);
  }
}

template <bool BF16IO>
__global__ __launch_bounds__(256, BF16IO ? 4 : 2) void kda_scan_output_kernel(Params p) {
  const int64_t groups = (p.seg_len + kScanOutChunks - 1) / kScanOutChunks;
  const int64_t task = task_index();  // consecutive tasks (one segment) share an XCD
  const int64_t H = p.H;
  int64_t h, n, seg, gi, first, nseg;
  if (!p.cu_seqlens) {
    const int64_t P = p.segs_per_seq;
    const int64_t per_seq = (P - 1) * groups;
    const int64_t per_head = p.N * per_seq;
    if (per_head <= 0) return;
    h = task / per_head;
    if (h >= H) return;
    int64_t rem = task - h * per_head;
    n = rem / per_seq;
    rem -= n * per_seq;
    seg = 1 + rem / groups;
    gi = rem - (seg - 1) * groups;
    first = n * P;
    nseg = P;
  } else {
    const int64_t per_head = p.seg_stride * groups;
    h = task / per_head;
    if (h >= H) return;
    const int64_t rem = task - h * per_head;
    const int64_t gsg = rem / groups;
    gi = rem - gsg * groups;
    if (gsg >= p.cu_segs[p.N]) return;
    int64_t lo = 0, hi = p.N - 1;  // largest n with cu_segs[n] <= gsg
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (p.cu_segs[mid] <= gsg) lo = mid;
      else hi = mid - 1;
    }
    n = lo;
    seq_segments(p, n, first, nseg);
    seg = gsg - first;
  }
  if (seg < 1 || seg >= nseg || first < 0 || first + nseg > p.seg_stride) return;
  int64_t start, end, chunk0, nch;
  seq_range(p, n, start, end, chunk0, nch);
  const int64_t c0 = seg * p.seg_len + gi * kScanOutChunks;
  const int64_t c1 = min(min(c0 + kScanOutChunks, (seg + 1) * p.seg_len), nch);
  if (c0 >= c1) return;

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int m = lane & 15;
  const int grp = lane >> 4;
  // S_p rows 16 rb + m, packed by the combine as the recurrence packs its state (keys in
  // the 16x16x32 operand order): key group kb of row block rb sits where the FP32
  // fragment of key block 2 kb was.
  const float* sp_src = p.scan_s + (h * p.seg_stride + first + seg) * (kD * kD);
  bf16x8 sa[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      sa[i][kb] = *reinterpret_cast<const bf16x8*>(sp_src + state_frag(2 * wave + i, 2 * kb, lane));

  const int64_t vstride = H * kD;
  const int64_t qbase = (h * p.max_chunks + chunk0) * (4 * 64 * 8) + lane * 8;
  const int64_t obase = (start + m) * vstride + h * kD + 32 * wave + 4 * grp;
  // Every load of the workgroup is issued before the first product: the latency of one
  // round trip, not one per chunk, sets the time. Chunks past c1 re-read chunk c1 - 1
  // (in bounds, never stored).
  ScanOutIn<BF16IO> in[kScanOutChunks];
#pragma unroll
  for (int j = 0; j < kScanOutChunks; ++j) {
    const int64_t c = min(c0 + j, c1 - 1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      in[j].q[kb] = load_frag<BF16IO>(p.scan_q, qbase + c * (4 * 64 * 8) + kb * 64 * 8);
    if (m < end - (start + c * kC)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t idx = obase + c * kC * vstride + 16 * i;
        if constexpr (BF16IO)
          in[j].oz[i] = *reinterpret_cast<const u32x2*>(static_cast<const unsigned short*>(p.o) + idx);
        else
          in[j].oz[i] = load4<false>(p.o, idx);
      }
    }
  }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kScanOutChunks; ++j) {
    const int64_t c = c0 + j;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f32x4 acc = mfma32(sa[i][0], in[j].q[0], zero);
      acc = mfma32(sa[i][1], in[j].q[1], acc);
      acc = mfma32(sa[i][2], in[j].q[2], acc);
      acc = mfma32(sa[i][3], in[j].q[3], acc);
      if (c < c1 && m < end - (start + c * kC)) {
        f32x4 oz;
        if constexpr (BF16IO) {
          const u32x2 w = in[j].oz[i];
          oz = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                     __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
        } else {
          oz = in[j].oz[i];
        }
        store4<BF16IO>(p.o, obase + c * kC * vstride + 16 * i, acc + oz);
      }
    }
  }
}

template <bool BF16IO, bool BF16ST, bool CK>
void launch_waves(const Params& p, dim3 grid, hipStream_t stream) {
  switch (p.waves) {
    case 1:
      hipLaunchKernelGGL((kda_recurrence_kernel<BF16IO, BF16ST, 1, CK>), grid,
                         dim3(Tile<BF16IO, 1>::NT), 0, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((kda_recurrence_kernel<BF16IO, BF16ST, 2, CK>), grid,
                         dim3(Tile<BF16IO, 2>::NT), 0, stream, p);
      break;
    case 4:
      hipLaunchKernelGGL((kda_recurrence_kernel<BF16IO, BF16ST, 4, CK>), grid,
                         dim3(Tile<BF16IO, 4>::NT), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((kda_recurrence_kernel<BF16IO, BF16ST, 8, CK>), grid,
                         dim3(Tile<BF16IO, 8>::NT), 0, stream, p);
      break;
  }
}

template <bool BF16IO, bool BF16ST>
void launch_io(const Params& p, dim3 grid, hipStream_t stream) {
  if (p.ckpt_every > 0) launch_waves<BF16IO, BF16ST, true>(p, grid, stream);
  else launch_waves<BF16IO, BF16ST, false>(p, grid, stream);
}

}  // namespace

int recurrence_loader_waves(int compute_waves) { return loader_waves(compute_waves); }

hipError_t launch_recurrence(const Params& p, int64_t workgroups, bool io_bf16, bool state_bf16,
                             hipStream_t stream) {
  if (workgroups <= 0) return hipSuccess;
  if (p.waves != 1 && p.waves != 2 && p.waves != 4 && p.waves != 8) return hipErrorInvalidValue;
  workgroups = (workgroups + 7) / 8 * 8;  // whole XCD rounds (see task_index)
  if (workgroups > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(workgroups));
  if (io_bf16) {
    if (state_bf16) launch_io<true, true>(p, grid, stream);
    else launch_io<true, false>(p, grid, stream);
  } else {
    if (state_bf16) launch_io<false, true>(p, grid, stream);
    else launch_io<false, false>(p, grid, stream);
  }
  return hipGetLastError();
}

hipError_t launch_scan_output(const Params& p, int64_t workgroups, bool io_bf16,
                              hipStream_t stream) {
  if (workgroups <= 0) return hipSuccess;
  workgroups = (workgroups + 7) / 8 * 8;  // whole XCD rounds (see task_index)
  if (workgroups > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(workgroups));
  if (io_bf16) hipLaunchKernelGGL(kda_scan_output_kernel<true>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(kda_scan_output_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const Params& p, bool state_bf16, hipStream_t stream) {
  const int64_t wgs = (p.H * p.N + 7) / 8 * 64;  // 8 row blocks per pair, pairs by XCD
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(wgs));
  if (state_bf16) hipLaunchKernelGGL(kda_combine_kernel<true>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(kda_combine_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
