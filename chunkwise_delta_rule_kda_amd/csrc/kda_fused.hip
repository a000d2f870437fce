// kda_fused: the recurrence launch in its fused form. The workgroup of a run (a sequence,
// a segment, or a transition run, decoded as in kda_recurrence.hip) has W compute waves,
// exactly as there, and producer waves that prepare every chunk of the run from q, k, g,
// beta and v themselves (kda_producer.h) into the LDS ring the compute waves read: no
// preparation kernel runs and no record goes through HBM. The preparation is that of the
// "FlashKDA column split" post, section 1 (the chunk quantities), in the folded record
// layout of include/kda.h.

#include "kda_recurrence_core.h"

namespace kda {

namespace {

// The fused form of the recurrence launch: W compute waves, fed by producer
// waves that prepare each chunk from q, k, g, beta and v themselves (kda_producer.h), so
// no preparation kernel runs and no record goes through HBM. Each workgroup prepares
// every chunk of its run (the row blocks of one run each do so, on their own compute
// units).
template <bool BF16IO, bool BF16ST, int W, bool CK, bool XFORM>
__global__ __launch_bounds__(fused::block_threads(W), fused::waves_per_simd(W)) void kda_fused_kernel(Params p) {
  using F = fused::Tile<BF16IO, W>;
  static_assert(F::NT == fused::block_threads(W), "block size");
  __shared__ __attribute__((aligned(16))) unsigned char ring_[F::NSLOT * F::SLOT];
  __shared__ __attribute__((aligned(16))) fused::Sync<F::NP> sync_;
  lds_u8* ring = (lds_u8*)(ring_);                       // address-space casts
  fused::lds_sync<F::NP>* sy = (fused::lds_sync<F::NP>*)(&sync_);

  Task t;
  if (!decode_task(p, 16 * W, t)) return;  // uniform over the workgroup
  const int tid = static_cast<int>(threadIdx.x);
  if (tid < 8) {
    sy->ready[tid] = 0;
    sy->done[tid] = 0;
  }
  if (tid < F::NPAIR) sy->pair[tid] = 0;
  if (tid == 0) {
    sy->fin = 0;
    sy->abort = 0;
  }
  if (XFORM && (p.flags & kFlagGate) && tid < kD) sy->dtb[tid] = p.dt_bias[t.h * kD + tid];
  __syncthreads();  // the only workgroup barrier: every later wait is on LDS counters
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  if (t.out) {
    if (wave < W) compute_loop<BF16IO, BF16ST, W, true, CK, true>(p, t, ring, wave, lane, sy);
    else if (t.nch > 0) fused::producer_loop<BF16IO, W, true, XFORM>(p, t, ring, sy, wave - W, lane);
  } else {
    if (wave < W) compute_loop<BF16IO, BF16ST, W, false, false, true>(p, t, ring, wave, lane, sy);
    else if (t.nch > 0) fused::producer_loop<BF16IO, W, false, XFORM>(p, t, ring, sy, wave - W, lane);
  }
}

template <bool BF16IO, bool BF16ST, bool CK, bool XFORM>
void launch_fused_xform(const Params& p, dim3 grid, hipStream_t stream) {
  switch (p.waves) {
    case 1:
      hipLaunchKernelGGL((kda_fused_kernel<BF16IO, BF16ST, 1, CK, XFORM>), grid,
                         dim3(fused::Tile<BF16IO, 1>::NT), 0, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((kda_fused_kernel<BF16IO, BF16ST, 2, CK, XFORM>), grid,
                         dim3(fused::Tile<BF16IO, 2>::NT), 0, stream, p);
      break;
    case 4:
      hipLaunchKernelGGL((kda_fused_kernel<BF16IO, BF16ST, 4, CK, XFORM>), grid,
                         dim3(fused::Tile<BF16IO, 4>::NT), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((kda_fused_kernel<BF16IO, BF16ST, 8, CK, XFORM>), grid,
                         dim3(fused::Tile<BF16IO, 8>::NT), 0, stream, p);
      break;
  }
}

template <bool BF16IO, bool BF16ST, bool CK>
void launch_fused_waves(const Params& p, dim3 grid, hipStream_t stream) {
  if (p.flags & (kFlagL2 | kFlagGate | kFlagBetaLogit))
    launch_fused_xform<BF16IO, BF16ST, CK, true>(p, grid, stream);
  else
    launch_fused_xform<BF16IO, BF16ST, CK, false>(p, grid, stream);
}

}  // namespace

hipError_t launch_fused_recurrence(const Params& p, int64_t workgroups, bool io_bf16,
                                   bool state_bf16, hipStream_t stream) {
  if (workgroups <= 0) return hipSuccess;
  if (p.waves != 1 && p.waves != 2 && p.waves != 4 && p.waves != 8) return hipErrorInvalidValue;
  workgroups = (workgroups + 7) / 8 * 8;  // whole XCD rounds (see task_index)
  if (workgroups > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(workgroups));
  const bool ck = p.ckpt_every > 0;
  if (io_bf16) {
    if (state_bf16) {
      if (ck) launch_fused_waves<true, true, true>(p, grid, stream);
      else launch_fused_waves<true, true, false>(p, grid, stream);
    } else {
      if (ck) launch_fused_waves<true, false, true>(p, grid, stream);
      else launch_fused_waves<true, false, false>(p, grid, stream);
    }
  } else {
    if (state_bf16) {
      if (ck) launch_fused_waves<false, true, true>(p, grid, stream);
      else launch_fused_waves<false, true, false>(p, grid, stream);
    } else {
      if (ck) launch_fused_waves<false, false, true>(p, grid, stream);
      else launch_fused_waves<false, false, false>(p, grid, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace kda
