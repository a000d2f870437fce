// Device code shared by the two recurrence translation units (kda_recurrence.hip: the
// recurrence with loader waves, the segment combine and the scan output; kda_fused.hip:
// the recurrence with producer waves): the task decoding, the compute waves' chunk step
// and loop, and the loader and producer waves. Everything sits in an anonymous namespace
// inside kda, so each unit has its own copy. The algorithm is described at the top of
// kda_recurrence.hip.
#pragma once

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

#include "kda_producer.h"

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
// FUSED: the ring is filled by producer waves that prepare the chunks (kda_producer.h)
// and published through LDS counters instead of the per-chunk barrier; chunks past the
// run's last are neither produced nor read.
template <bool BF16IO, bool BF16ST, int W, bool OUT, bool CKPT, bool FUSED>
__device__ __forceinline__ void compute_loop(const Params& p, const Task& t, lds_u8* ring,
                                             int wave, int lane,
                                             fused::lds_sync<fused::producers(W)>* sy) {
  using T = Tile<BF16IO, W>;
  constexpr int SLOTB = FUSED ? fused::Tile<BF16IO, W>::SLOT : T::SLOT;
  constexpr int NSL = FUSED ? fused::Tile<BF16IO, W>::NSLOT : kSlots;
  // chunk c + 1 of the run is visible: both halves of it counted in its slot (false: the
  // workgroup gave up, leave)
  auto wait_next = [&](int64_t c, int slot) -> bool {
    if constexpr (FUSED) {
      if (c + 1 >= t.nch) return true;
      return fused::wait_at_least(&sy->abort, &sy->ready[slot],
                                  2 * (static_cast<int>((c + 1) / NSL) + 1), p.status);
    } else {
      read_barrier();
      return true;
    }
  };
  // this wave's reads of the slot are complete: count them for its producer
  auto release = [&](int slot) {
    if constexpr (FUSED) {
      fused::lds_drain();
      if (lane == 0) fused::lds_add(&sy->done[slot], 1);
    }
  };
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
    if (!wait_next(-1, 0)) return;  // B_{-1}: chunk 0 visible
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
    release(0);
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
      const int ns = cs + 1 == NSL ? 0 : cs + 1;  // slot of chunk c + 1
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
      if (!wait_next(c, ns)) return;  // B_c: chunk c + 1 visible
      // All of chunk c + 1's operands are read here, one chunk ahead, so that their
      // latency (they queue behind the loaders' writes of chunk c + 2) is hidden by
      // chunk c's MFMA work. In the fused form the last iteration reads a slot that
      // holds no next chunk (in bounds, values unused): reading unconditionally keeps
      // the loop's register use that of the unfused form.
      ChainIn nxt;
      TailIn ntail;
      read_chain<BF16IO, W>(nxt, ring + ns * SLOTB, lane, wave, nvalid_of(c + 1));
      read_tail<OUT>(ntail, ring + ns * SLOTB, lane);
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
      if constexpr (FUSED) {
        if (c + 1 < nch) release(ns);
      }
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
    static_assert(W * 2048 <= SLOTB, "Phi staging");
    lds_u8* stage = ring + (nch % NSL) * SLOTB + wave * 2048;
    if constexpr (FUSED) {
      // Every compute wave is past its last chunk (and every producer write was read)
      // before a slot is reused for staging.
      fused::lds_drain();
      if (lane == 0) fused::lds_add(&sy->fin, 1);
      if (!fused::wait_at_least(&sy->abort, &sy->fin, W, p.status)) return;
      stage = ring + wave * 2048;
    }
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


}  // namespace
}  // namespace kda
