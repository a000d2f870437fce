// kda_recurrence: the serial state carry across chunks.
//
// The "FlashKDA column split" post, section 3.1 ("Every value column is independent"),
// shows that in the transposed form
//   U^T = A_kk B (V^T - K_start^T S^T),  O^T = s Q_start^T S^T + A_qk U^T,
//   S_{c+1}^T = D_{0:15} S^T + K_end^T U^T
// each value row of S follows its own recurrence, so a head's 128 value rows can be
// split over compute units with no synchronisation at all. Here each wave owns 16 value
// rows and a workgroup holds 1, 2 or 4 waves; the grid covers (sequence, head, slice).
// Section 3.3 ("Keeping the state in registers") keeps the state slice in registers
// for the whole sequence; on CDNA the MFMA accumulator layout of a 16x16 block already
// is the B-operand layout (up to a fixed permutation of the key order, which the
// preparation kernel applies to the key-side operands), so no transpose is needed.
//
// With the record folded by kda_prepare (Mb = A_kk B, Kn = -Mb K_start^T,
// Qt = s Q_start^T + A_qk Kn) one chunk for one wave is:
//   UV    = Mb V^T                      (16x16x16 MFMA, off the chain)
//   U^T   = UV + Kn S^T                 (4 x 16x16x32 MFMA, on the chain)
//   O     = UV^T A_qk^T + S Qt^T        (off the chain: uses the entering state)
//   S^T   = D (.) S^T + K_end^T U^T     (8 x 16x16x16 MFMA, on the chain)
// State is FP32 in registers; MFMA operands are BF16.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

struct ChunkRegs {
  bf16x8 kn[4];
  bf16x8 qt[4];
  i16x4 ke[8];
  f32x4 d[8];
  i16x4 mb;
  i16x4 aq;
  i16x4 vv;
};

template <bool BF16IO>
__device__ __forceinline__ void load_chunk(ChunkRegs& c, const unsigned char* __restrict__ rec,
                                           const void* __restrict__ v, int64_t vbase,
                                           int64_t vstride, int64_t nvalid, int lane) {
  const int m = lane & 15;
  const int grp = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    c.kn[kb] = *reinterpret_cast<const bf16x8*>(rec + kOffKn + kb * 1024 + lane * 16);
    c.qt[kb] = *reinterpret_cast<const bf16x8*>(rec + kOffQt + kb * 1024 + lane * 16);
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    c.ke[b] = *reinterpret_cast<const i16x4*>(rec + kOffKeT + b * 512 + lane * 8);
    c.d[b] = *reinterpret_cast<const f32x4*>(rec + kOffD + (16 * b + 4 * grp) * 4);
  }
  c.mb = *reinterpret_cast<const i16x4*>(rec + kOffMb + lane * 8);
  c.aq = *reinterpret_cast<const i16x4*>(rec + kOffAqk + lane * 8);
  // V^T operand: lane holds v[token 4 grp + j][value m] of this wave's 16 values.
  // Pad tokens of a short last chunk read token 0 of the chunk (always valid) and are
  // zeroed, so no load leaves the chunk's own rows.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * grp + j;
    const bool ok = t < nvalid;
    const int64_t idx = vbase + (ok ? t : 0) * vstride + m;
    short x;
    if constexpr (BF16IO)
      x = static_cast<const short*>(v)[idx];
    else
      x = static_cast<short>(float_to_bf16_bits(static_cast<const float*>(v)[idx]));
    c.vv[j] = ok ? x : static_cast<short>(0);
  }
}

template <bool BF16IO>
__device__ __forceinline__ void chunk_step(const ChunkRegs& c, f32x4 (&st)[8], bf16x8 (&sp)[4],
                                           void* __restrict__ o, int64_t obase, int64_t ostride,
                                           int64_t nvalid, int lane) {
  const int m = lane & 15;
  const int grp = lane >> 4;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // Every MFMA accumulation chain below uses one opcode and starts from zero; results
  // of the 16x16x16 products are combined with VALU adds rather than fed to a
  // 16x16x32 product as its accumulator input.
  // UV[token 4 grp + j][value m]
  const f32x4 uv = mfma16(c.mb, c.vv, zero);
  // U^T = UV + Kn S^T (the chain)
  f32x4 u = zero;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) u = mfma32(c.kn[kb], sp[kb], u);
  u += uv;
  // O[value 4 grp + j][token m] from the entering state (independent of U)
  f32x4 out = zero;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) out = mfma32(sp[kb], c.qt[kb], out);
  out += mfma16(pack4(uv), c.aq, zero);
  // S^T = D (.) S^T + K_end^T U^T
  const i16x4 up = pack4(u);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    f32x4 x = st[b] * c.d[b];
    st[b] = mfma16(c.ke[b], up, x);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) sp[kb] = pack8(st[2 * kb], st[2 * kb + 1]);
  if (m < nvalid) store4<BF16IO>(o, obase + m * ostride + 4 * grp, out);
}

template <bool BF16IO, bool BF16ST>
__global__ __launch_bounds__(256) void kda_recurrence_kernel(Params p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves = p.waves;
  const int slices = 8 / waves;
  // XCD-aware order: workgroup b runs on XCD b % 8, so consecutive tasks (the slices
  // of one head, which read the same records) are mapped to the same XCD's L2.
  const int64_t total = gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t task = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  const int64_t sh = task / slices;
  const int slice = static_cast<int>(task - sh * slices);
  const int64_t H = p.H;
  const int64_t s = sh / H;
  const int64_t h = sh - s * H;
  const int v0 = (slice * waves + wave) * 16;
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

  // State rows v0 + m, keys 16 b + 4 grp + j: the 16x16x16 accumulator layout.
  const int64_t srow = ((s * H + h) * kD + v0 + m) * kD;
  f32x4 st[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (p.state_in)
      st[b] = load4<BF16ST>(p.state_in, srow + 16 * b + 4 * grp);
    else
      st[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 sp[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) sp[kb] = pack8(st[2 * kb], st[2 * kb + 1]);

  const int64_t vstride = H * kD;
  const int64_t rec_stride = H * static_cast<int64_t>(kRecord);
  const unsigned char* rec = p.records + (chunk0 * H + h) * static_cast<int64_t>(kRecord);
  const int64_t base0 = start * vstride + h * kD + v0;

  // Two register stages: chunk c + 1 loads while chunk c computes. Loads past the last
  // chunk re-read the last chunk (in bounds) so the loop body has no branches.
  ChunkRegs A, B;
  const int64_t last = nch - 1;
  auto load_at = [&](ChunkRegs& R, int64_t c) {
    const int64_t cc = c < last ? c : last;
    load_chunk<BF16IO>(R, rec + cc * rec_stride, p.v, base0 + cc * kC * vstride, vstride,
                       end - start - cc * kC, lane);
  };
  if (nch > 0) load_at(A, 0);
  for (int64_t c = 0; c < nch; c += 2) {
    const int64_t t0 = start + c * kC;
    load_at(B, c + 1);
    chunk_step<BF16IO>(A, st, sp, p.o, base0 + c * kC * vstride, vstride, end - t0, lane);
    if (c + 1 >= nch) break;
    load_at(A, c + 2);
    chunk_step<BF16IO>(B, st, sp, p.o, base0 + (c + 1) * kC * vstride, vstride,
                       end - t0 - kC, lane);
  }

  if (p.state_out) {
#pragma unroll
    for (int b = 0; b < 8; ++b) store4<BF16ST>(p.state_out, srow + 16 * b + 4 * grp, st[b]);
  }
}

}  // namespace

hipError_t launch_recurrence(const Params& p, int64_t workgroups, bool io_bf16, bool state_bf16,
                             hipStream_t stream) {
  if (workgroups <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(workgroups));
  const dim3 block(64 * p.waves);
  if (io_bf16) {
    if (state_bf16)
      hipLaunchKernelGGL((kda_recurrence_kernel<true, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((kda_recurrence_kernel<true, false>), grid, block, 0, stream, p);
  } else {
    if (state_bf16)
      hipLaunchKernelGGL((kda_recurrence_kernel<false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((kda_recurrence_kernel<false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace kda
