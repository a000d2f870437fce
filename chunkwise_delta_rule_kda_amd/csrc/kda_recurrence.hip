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
// With many segments per sequence B and C are replaced by one launch
// (kda_carry_out_kernel) in which every later segment forms its own start state from
// S_1 by the chain of B and then adds its output term.
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

#include "kda_recurrence_core.h"

namespace kda {

namespace {

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
    if (wave < W) compute_loop<BF16IO, BF16ST, W, true, CK, false>(p, t, ring, wave, lane, nullptr);
    else if (t.nch > 0) loader_loop<BF16IO, T, true>(p, t, ring, lt);
  } else {
    if (wave < W) compute_loop<BF16IO, BF16ST, W, false, false, false>(p, t, ring, wave, lane, nullptr);
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

// Carry-and-output launch: the affine-output form's alternative to the combine and
// scan-output launches for sequences cut into many segments (the small-head regime).
// S_p follows from segment 0's end state S_1 by S_{s+1} = S_s Phi_s + Z_s; one
// workgroup per (head, later segment p, block of 32 value rows) forms S_p for its rows
// by that chain of p - 1 steps, then adds (Qt_c Phi_{p,c}^T) S_p^T to o for every chunk
// c of segment p (the scan-output term); the last segment's workgroups take one more
// step, to the final state. Each workgroup repeats the chain prefix of the segments
// before its own, so no workgroup waits for another one and there is no combine launch
// in between: the segments with short chains stream their outputs while the long
// chains still run.
// Chain step: wave w computes output key blocks 2 w and 2 w + 1 of both row blocks
// (sixteen 16x16x32 products) with its 32-key slice of Phi_s^T as the A operand and the
// packed state, exchanged through LDS, as the B operand; Z_s is added in FP32. The step
// time is set by the operand stream (32 KB of Phi and 16 KB of Z per step), so those
// loads run kCarryDepth steps ahead. Output: wave w takes chunks c0 + w, c0 + w + 4,
// ...; the loads of its first kCarryOut chunks do not depend on the chain and are issued
// right after the chain's first operands (loads retire in order, so the chain's first
// waits do not include them), then each chunk kCarryOut ahead.
constexpr int kCarryDepth = 2;  // chain steps of Phi and Z in flight per wave

struct CarryIn {
  u32x4 a[2][4];  // Phi^T operands: output key block 2 w + i, input key group kk
  f32x4 z[2][2];  // Z rows 16 (R0 + r) + m, keys 16 (2 w + i) + 4 grp + j
};

// Output chunks in flight per wave (an FP32 chunk holds twice the registers).
template <bool BF16IO>
constexpr int carry_out_depth() { return BF16IO ? 4 : 2; }

template <bool BF16IO, bool BF16ST>
__global__ __launch_bounds__(256, 1) void kda_carry_out_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) unsigned char xch_[2 * 2 * 4 * 64 * 16];
  lds_u8* xbase = (lds_u8*)(xch_);  // address-space cast
  // Tasks (head, sequence, later segment, 32-row block), row blocks fastest: the four
  // row blocks of one segment, which read the same Phi, Z slots and Qt Phi^T, run on one
  // XCD. Fixed layout only.
  const int64_t task = task_index();
  const int64_t later = p.segs_per_seq - 1;
  const int64_t per_head = p.N * later * 4;
  if (per_head <= 0) return;
  const int64_t h = task / per_head;
  if (h >= p.H) return;
  const int64_t rem = task - h * per_head;
  const int rb = static_cast<int>(rem & 3);
  const int64_t n = (rem >> 2) / later;
  const int64_t seg = 1 + ((rem >> 2) - n * later);
  const int64_t first = n * p.segs_per_seq;
  const int64_t nseg = p.segs_per_seq;
  const bool fin = seg == nseg - 1 && p.state_out;  // also forms the final state S_P
  const int64_t lastf = fin ? seg : seg - 1;         // chain steps s = 1 .. lastf

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int m = lane & 15;
  const int grp = lane >> 4;
  const int R0 = 2 * rb;  // first 16-row block of the workgroup

  // ---- the chain's first operands: S_1 and the first kCarryDepth steps --------------
  const int64_t slot0 = h * p.seg_stride + first;
  const float* sbase = p.scan_s + slot0 * (kD * kD);
  const unsigned char* pbase =
      reinterpret_cast<const unsigned char*>(p.scan_phi + slot0 * (kD * kD));
  const int aoff = (2 * wave * 4 * 64 + lane) * 16;  // bytes: block 2 wave, group 0
  int64_t koff[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 2; ++i) koff[r][i] = state_frag(R0 + r, 2 * wave + i, lane);
  auto fetch = [&](CarryIn& x, int64_t s) {
    s = s < lastf ? s : lastf;  // past the last step: re-read it (in bounds, unused)
    const unsigned char* ph = pbase + s * (kD * kD * 2) + aoff;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        x.a[i][kk] = *reinterpret_cast<const u32x4*>(ph + (i * 4 + kk) * 1024);
    // Z_s lives in slot s + 1; the last segment's in the sequence's first slot.
    const float* z = sbase + (s + 1 < nseg ? s + 1 : 0) * (kD * kD);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 2; ++i) x.z[r][i] = load4<false>(z, koff[r][i]);
  };
  f32x4 st[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 2; ++i) st[r][i] = load4<false>(sbase + kD * kD, koff[r][i]);  // S_1
  CarryIn in[kCarryDepth];
  if (lastf >= 1) {
#pragma unroll
    for (int d = 0; d < kCarryDepth; ++d) fetch(in[d], 1 + d);
  }

  // ---- this wave's first output chunks (independent of the chain) ---------------------
  int64_t start, end, chunk0, nch;
  seq_range(p, n, start, end, chunk0, nch);
  const int64_t c0 = seg * p.seg_len;
  const int64_t c1 = min(c0 + p.seg_len, nch);
  const int64_t nj = c1 - c0 > wave ? (c1 - c0 - wave + 3) / 4 : 0;  // this wave's chunks
  const int64_t vstride = p.H * kD;
  const int64_t qbase = (h * p.max_chunks + chunk0) * (4 * 64 * 8) + lane * 8;
  const int64_t ocol = h * kD + 32 * rb + 4 * grp;
  // Element offset of O[token tm of chunk c][values 16 (R0 + r) + 4 grp + j].
  auto oidx = [&](int64_t c, int tm, int r) {
    return (start + c * kC + tm) * vstride + ocol + 16 * r;
  };
  constexpr int kCarryOut = carry_out_depth<BF16IO>();
  ScanOutIn<BF16IO> ob[kCarryOut];
  int64_t jn = 0;  // next of this wave's chunks to load; past the last, re-read the last
  auto issue = [&](ScanOutIn<BF16IO>& x) {
    const int64_t c = c0 + wave + 4 * (jn < nj ? jn : nj - 1);
    const int64_t valid = end - (start + c * kC);
    const int tm = m < valid ? m : static_cast<int>(valid) - 1;  // stay in the sequence
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      x.q[kb] = load_frag<BF16IO>(p.scan_q, qbase + c * (4 * 64 * 8) + kb * 64 * 8);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if constexpr (BF16IO)
        x.oz[r] = *reinterpret_cast<const u32x2*>(static_cast<const unsigned short*>(p.o) +
                                                  oidx(c, tm, r));
      else
        x.oz[r] = load4<false>(p.o, oidx(c, tm, r));
    }
    ++jn;
  };
  if (nj > 0) {
#pragma unroll
    for (int d = 0; d < kCarryOut; ++d) issue(ob[d]);
  }

  // ---- the chain S_1 -> S_p (-> S_P) --------------------------------------------------
  // [parity 2][row block r 2][wave 4][lane 64]: packed S^T key blocks 2 w, 2 w + 1
  auto xch = [&](int parity, int r, int w) {
    return reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(
        xbase + ((parity * 2 + r) * 4 + w) * 1024 + lane * 16);
  };
#pragma unroll
  for (int r = 0; r < 2; ++r) *xch(1, r, wave) = pack8(st[r][0], st[r][1]);
  lds_barrier();
  // Step s: S_{s+1} = S_s Phi_s + Z_s with operands in set (s - 1) % depth; the set is
  // then refilled with step s + depth. Whole groups of depth steps are unrolled without
  // conditions so that the compiler's wait before each step is for its own set only.
  auto step = [&](auto set_c, int64_t s) {
    constexpr int set = decltype(set_c)::value;
    bf16x8 sp[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sp[r][kk] = *xch(s & 1, r, kk);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f32x4 acc = zero;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = mfma32(__builtin_bit_cast(bf16x8, in[set].a[i][kk]), sp[r][kk], acc);
        st[r][i] = acc + in[set].z[r][i];
      }
#pragma unroll
    for (int r = 0; r < 2; ++r) *xch((s + 1) & 1, r, wave) = pack8(st[r][0], st[r][1]);
    fetch(in[set], s + kCarryDepth);
    lds_barrier();
  };
  int64_t s = 1;
#pragma unroll 1
  for (; s + kCarryDepth - 1 <= lastf; s += kCarryDepth)
    unroll<kCarryDepth>([&](auto d) { step(d, s + decltype(d)::value); });
  unroll<kCarryDepth - 1>([&](auto d) {
    if (s + decltype(d)::value <= lastf) step(d, s + decltype(d)::value);
  });
  // S_p (parity p & 1; a final step wrote the other parity) as A operands: key group kb
  // of row block r is wave kb's packed piece.
  bf16x8 sa[2][4];
  const int par = static_cast<int>(seg & 1);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sa[r][kb] = *xch(par, r, kb);
  if (fin) {  // st holds S_P
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t srow = state_row(p, n, h, 16 * (R0 + r) + m);
      if (srow < 0) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        store4<BF16ST>(p.state_out, srow + 16 * (2 * wave + i) + 4 * grp, st[r][i]);
    }
  }

  // ---- output: o += (Qt Phi^T) S_p^T for this wave's chunks ---------------------------
  if (nj <= 0) return;  // no barrier follows
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto body = [&](auto d_c, int64_t j) {
    constexpr int d = decltype(d_c)::value;
    const int64_t c = c0 + wave + 4 * j;
    const bool tv = m < end - (start + c * kC);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      f32x4 acc = mfma32(sa[r][0], ob[d].q[0], zero);
      acc = mfma32(sa[r][1], ob[d].q[1], acc);
      acc = mfma32(sa[r][2], ob[d].q[2], acc);
      acc = mfma32(sa[r][3], ob[d].q[3], acc);
      f32x4 oz;
      if constexpr (BF16IO) {
        const u32x2 w = ob[d].oz[r];
        oz = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                   __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
      } else {
        oz = ob[d].oz[r];
      }
      if (tv) store4<BF16IO>(p.o, oidx(c, m, r), acc + oz);
    }
    issue(ob[d]);
  };
  int64_t j = 0;
#pragma unroll 1
  for (; j + kCarryOut <= nj; j += kCarryOut)
    unroll<kCarryOut>([&](auto d) { body(d, j + decltype(d)::value); });
  unroll<kCarryOut - 1>([&](auto d) {
    if (j + decltype(d)::value < nj) body(d, j + decltype(d)::value);
  });
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
  if (p.fused) return launch_fused_recurrence(p, workgroups, io_bf16, state_bf16, stream);
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

hipError_t launch_carry_out(const Params& p, int64_t workgroups, bool io_bf16, bool state_bf16,
                            hipStream_t stream) {
  if (workgroups <= 0) return hipSuccess;
  workgroups = (workgroups + 7) / 8 * 8;  // whole XCD rounds (see task_index)
  if (workgroups > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(workgroups));
  if (io_bf16) {
    if (state_bf16) hipLaunchKernelGGL((kda_carry_out_kernel<true, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kda_carry_out_kernel<true, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (state_bf16) hipLaunchKernelGGL((kda_carry_out_kernel<false, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kda_carry_out_kernel<false, false>), grid, dim3(256), 0, stream, p);
  }
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
