// kda_recurrence: the serial state carry across chunks.
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
// Workgroup. W compute waves (16 value rows each, W = 1, 2, 4, 8) of one
// (sequence, head) plus L loader waves (L = 4 - W when W < 4). Every chunk's record and
// V tile are fetched once per workgroup by all of its waves together with ordinary
// 16-byte loads (one wave alone streams only ~40 GB/s, four reach the compute unit's
// ~150 GB/s; the LDS-DMA path was measured at ~16 B/clock), two chunks ahead, and
// staged through a 3-slot LDS ring. One raw s_barrier per chunk (after each wave's own
// LDS writes have completed; no memory fence, so the global loads in flight stay in
// flight) publishes the next slot.
//
// Ring protocol, iteration c (all waves):
//   write the registers holding chunk c+1 into slot (c+1)%3     [slot of chunk c-2]
//   issue the loads of chunk c+2 into registers
//   wait for own LDS writes; barrier B_c                         [chunk c+1 visible]
//   compute waves: read chunk c+1's chain inputs (prefetch) and compute chunk c.
// Chunk c-2's slot is rewritten only after B_{c-1}, which every wave reaches after its
// last read of chunk c-2 (made in iteration c-2). Chunk c's operands used after B_c were
// written before B_{c-1}.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kSlots = 3;
constexpr int kRecUnits = kRecord / 16;  // 864 sixteen-byte units per record

// Padded ring-slot bytes for W compute waves (loader waves fill the workgroup to at
// least 4 waves), element size es: ceil((864 + 16 W es) / threads) * threads * 16.
constexpr int slot_bytes(int w, int es) {
  const int nt = 64 * (w < 4 ? 4 : w);
  const int real = kRecUnits + 16 * w * es;
  return (real + nt - 1) / nt * nt * 16;
}
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kMaxSlotBytes =
    cmax(cmax(cmax(slot_bytes(1, 4), slot_bytes(2, 4)), cmax(slot_bytes(4, 4), slot_bytes(8, 4))),
         cmax(cmax(slot_bytes(1, 2), slot_bytes(2, 2)), cmax(slot_bytes(4, 2), slot_bytes(8, 2))));
static_assert(kMaxSlotBytes == 24576, "slot size table");
static_assert(slot_bytes(4, 4) / 16 / 256 <= 5 && slot_bytes(8, 4) / 16 / 512 <= 5,
              "kMaxLoads covers every configuration");

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

template <bool BF16IO, int W>
struct Tile {
  static constexpr int ES = BF16IO ? 2 : 4;
  static constexpr int NT = 64 * (W < 4 ? 4 : W);        // threads in the workgroup
  static constexpr int VROW = 16 * W * ES;                // bytes of one V-tile token row
  static constexpr int PARTS = VROW / 16;                 // 16-byte pieces per token row
  static constexpr int REAL = kRecUnits + VROW;           // record + V-tile units (16 B)
  static constexpr int K = (REAL + NT - 1) / NT;          // loads per thread per chunk
  static constexpr int SLOT = K * NT * 16;                // padded slot: K units per thread
  static_assert(SLOT == slot_bytes(W, ES) && SLOT <= kMaxSlotBytes, "slot table");
};

// One thread's share of a chunk's global -> LDS copy. Unit u = tid + k * NT of a chunk
// is record byte 16 u (u < 864), V-tile piece u - 864 (token row, 16-byte part), or
// padding (re-reads record unit 0 into the slot's unused tail).
template <bool BF16IO, int W>
struct Loader {
  using T = Tile<BF16IO, W>;
  u32x4 r[T::K];

  __device__ __forceinline__ void issue(int tid, const unsigned char* rec,
                                        const unsigned char* vrow0, int64_t vstride_b,
                                        int64_t nvalid) {
#pragma unroll
    for (int k = 0; k < T::K; ++k) {
      const int u = tid + k * T::NT;
      const int i = u - kRecUnits;
      const unsigned char* src;
      if (i >= 0 && i < T::VROW) {
        const int tok = i / T::PARTS;
        const int part = i - tok * T::PARTS;
        src = vrow0 + (tok < nvalid ? tok : 0) * vstride_b + part * 16;  // pad rows: row 0
      } else {
        src = rec + (u < kRecUnits ? u * 16 : 0);
      }
      r[k] = *reinterpret_cast<const u32x4*>(src);
    }
  }

  __device__ __forceinline__ void store(int tid, lds_u8* slot) const {
#pragma unroll
    for (int k = 0; k < T::K; ++k)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(slot + (tid + k * T::NT) * 16) =
          r[k];
  }
};

struct ChainIn {  // needed at the very start of a chunk (read one chunk ahead)
  bf16x8 kn[4];
  i16x4 mb;
  i16x4 vv;
};

struct TailIn {  // needed later in the chunk (read at its start)
  i16x4 ke[8];
  f32x4 d[8];
  bf16x8 qt[4];
  i16x4 aq;
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
  x.mb = *reinterpret_cast<const __attribute__((address_space(3))) i16x4*>(slot + kOffMb +
                                                                          lane * 8);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = 4 * grp + j;
    const lds_u8* p = slot + kRecord + tok * T::VROW + (16 * w + m) * T::ES;
    short s;
    if constexpr (BF16IO)
      s = *reinterpret_cast<const __attribute__((address_space(3))) short*>(p);
    else
      s = static_cast<short>(float_to_bf16_bits(
          *reinterpret_cast<const __attribute__((address_space(3))) float*>(p)));
    x.vv[j] = tok < nvalid ? s : static_cast<short>(0);
  }
}

__device__ __forceinline__ void read_tail(TailIn& x, const lds_u8* slot, int lane) {
  const int grp = lane >> 4;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    x.ke[b] = *reinterpret_cast<const __attribute__((address_space(3))) i16x4*>(
        slot + kOffKeT + b * 512 + lane * 8);
    x.d[b] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
        slot + kOffD + (16 * b + 4 * grp) * 4);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    x.qt[kb] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
        slot + kOffQt + kb * 1024 + lane * 16);
  x.aq = *reinterpret_cast<const __attribute__((address_space(3))) i16x4*>(slot + kOffAqk +
                                                                          lane * 8);
}

// One chunk for one wave: updates the state and returns O[value 4 grp + j][token m].
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
#pragma unroll
  for (int i = 0; i < 8; ++i) st[i] = mfma16(b.ke[i], up, st[i] * b.d[i]);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) sp[kb] = pack8(st[2 * kb], st[2 * kb + 1]);
  // O from the entering state (off the chain)
  f32x4 out = mfma32(s0, b.qt[0], zero);
  out = mfma32(s1, b.qt[1], out);
  out = mfma32(s2, b.qt[2], out);
  out = mfma32(s3, b.qt[3], out);
  out += mfma16(pack4(uv), b.aq, zero);
  return out;
}

template <bool BF16IO, bool BF16ST, int W>
__global__ __launch_bounds__(64 * (W < 4 ? 4 : W)) void kda_recurrence_kernel(Params p) {
  using T = Tile<BF16IO, W>;
  __shared__ __attribute__((aligned(16))) unsigned char ring_[kSlots * T::SLOT];
  lds_u8* ring = (lds_u8*)(ring_);  // address-space cast

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // W compute waves; the rest of the workgroup loads only.
  const int slices = 8 / W;
  // XCD-aware order: workgroup b runs on XCD b % 8, so consecutive tasks (the slices of
  // one head, which read the same records) are mapped to the same XCD's L2.
  const int64_t total = gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t task = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  const int64_t sh = task / slices;
  const int slice = static_cast<int>(task - sh * slices);
  const int64_t H = p.H;
  const int64_t s = sh / H;
  const int64_t h = sh - s * H;
  const int vwg = slice * 16 * W;  // first value row of this workgroup
  const bool compute = wave < W;
  const int v0 = vwg + 16 * wave;
  const int m = lane & 15;
  const int grp = lane >> 4;

  int64_t start, end, chunk0;
  if (p.cu_seqlens) {
    start = p.cu_seqlens[s];
    end = min(p.cu_seqlens[s + 1], p.T);
    chunk0 = p.cu_chunks[s];
  } else {
    start = s * p.T;
    end = start + p.T;
    chunk0 = s * p.chunks_per_seq;
  }
  int64_t nch = end > start ? (end - start + kC - 1) / kC : 0;
  if (chunk0 < 0) nch = 0;
  if (chunk0 + nch > p.max_chunks) nch = p.max_chunks > chunk0 ? p.max_chunks - chunk0 : 0;

  const int64_t vstride = H * kD;
  const int64_t vstride_b = vstride * T::ES;
  const unsigned char* rec0 =
      p.records + (h * p.max_chunks + chunk0) * static_cast<int64_t>(kRecord);
  const unsigned char* vtile0 = static_cast<const unsigned char*>(p.v) +
                                (start * vstride + h * kD + vwg) * T::ES;
  const int64_t vchunk_b = kC * vstride_b;  // bytes between consecutive chunks of V
  Loader<BF16IO, W> ld;
  // Next chunk to fetch (clamped: past the end re-reads the last chunk, in bounds).
  int64_t fetch = 0;
  auto issue_next = [&]() {
    const int64_t j = fetch < nch - 1 ? fetch : nch - 1;
    ld.issue(tid, rec0 + j * kRecord, vtile0 + j * vchunk_b, vstride_b, end - start - j * kC);
    ++fetch;
  };

  // State rows v0 + m, keys 16 b + 4 grp + j: the 16x16x16 accumulator layout.
  const int64_t srow = ((s * H + h) * kD + v0 + m) * kD;
  f32x4 st[8];
  bf16x8 sp[4];
  if (compute) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (p.state_in)
        st[b] = load4<BF16ST>(p.state_in, srow + 16 * b + 4 * grp);
      else
        st[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sp[kb] = pack8(st[2 * kb], st[2 * kb + 1]);
  }

  if (nch > 0) {
    issue_next();            // chunk 0
    ld.store(tid, ring);     // slot 0
    issue_next();            // chunk 1
    lds_barrier();           // chunk 0 visible
    ChainIn cur;
    if (compute) read_chain<BF16IO, W>(cur, ring, lane, wave, end - start);
    int cs = 0;  // slot of chunk c
    // O of chunk c is stored at the start of iteration c + 1, before the next loads are
    // issued: loads and stores retire through one in-order counter, so a wait for a
    // load never waits for a store issued after it.
    f32x4 pend = {0.f, 0.f, 0.f, 0.f};
    const int64_t obase = start * vstride + h * kD + v0;
    auto store_out = [&](int64_t c) {
      if (m < end - start - c * kC)
        store4<BF16IO>(p.o, obase + (c * kC + m) * vstride + 4 * grp, pend);
    };
#pragma unroll 1
    for (int64_t c = 0; c < nch; ++c) {
      const int ns = cs + 1 == kSlots ? 0 : cs + 1;     // slot of chunk c + 1
      const lds_u8* slot = ring + cs * T::SLOT;
      TailIn tail;
      if (compute) read_tail(tail, slot, lane);        // written before B_{c-1}
      ld.store(tid, ring + ns * T::SLOT);              // chunk c + 1 (slot of chunk c - 2)
      if (compute && c > 0) store_out(c - 1);
      issue_next();                                    // chunk c + 2
      lds_barrier();                                   // B_c: chunk c + 1 visible
      if (compute) {
        ChainIn nxt;
        read_chain<BF16IO, W>(nxt, ring + ns * T::SLOT, lane, wave,
                              end - start - (c + 1) * kC);
        pend = chunk_step(cur, tail, st, sp);
        cur = nxt;
      }
      cs = ns;
    }
    if (compute) store_out(nch - 1);
  }

  if (compute && p.state_out) {
#pragma unroll
    for (int b = 0; b < 8; ++b) store4<BF16ST>(p.state_out, srow + 16 * b + 4 * grp, st[b]);
  }
}


template <bool BF16IO, bool BF16ST>
void launch_io(const Params& p, dim3 grid, hipStream_t stream) {
  switch (p.waves) {
    case 1:
      hipLaunchKernelGGL((kda_recurrence_kernel<BF16IO, BF16ST, 1>), grid,
                         dim3(Tile<BF16IO, 1>::NT), 0, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((kda_recurrence_kernel<BF16IO, BF16ST, 2>), grid,
                         dim3(Tile<BF16IO, 2>::NT), 0, stream, p);
      break;
    case 4:
      hipLaunchKernelGGL((kda_recurrence_kernel<BF16IO, BF16ST, 4>), grid,
                         dim3(Tile<BF16IO, 4>::NT), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((kda_recurrence_kernel<BF16IO, BF16ST, 8>), grid,
                         dim3(Tile<BF16IO, 8>::NT), 0, stream, p);
      break;
  }
}

}  // namespace

int recurrence_loader_waves(int compute_waves) {
  return compute_waves < 4 ? 4 - compute_waves : 0;
}

hipError_t launch_recurrence(const Params& p, int64_t workgroups, bool io_bf16, bool state_bf16,
                             hipStream_t stream) {
  if (workgroups <= 0) return hipSuccess;
  if (p.waves != 1 && p.waves != 2 && p.waves != 4 && p.waves != 8) return hipErrorInvalidValue;
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

}  // namespace kda
