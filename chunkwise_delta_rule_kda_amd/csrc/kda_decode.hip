// kda_decode: one token per sequence (T = 1), the token step itself:
//   S <- S Diag(exp g) ; u = beta (v - S k) ; S <- S + u k^T ; o = s S q
// (the one-token case of the chunk equations of the "FlashKDA column split" post,
// section 1). With one token the chunk machinery has nothing to amortise: this kernel
// reads each (sequence, head) state once, updates it in registers and writes it back,
// so it is bound by the 2 x 32 KB (BF16) of state traffic per head.
//
// One 256-thread workgroup per (sequence, head). Thread t holds the 16-byte state
// pieces t + 256 i (i = 0..7): row r = t / 16 + 16 i, keys 8 (t % 16) .. + 7, so that one
// wave instruction reads four whole 256-byte rows, and the 16 lanes of a DPP row hold
// one state row; row sums (S k, S q) are 16-lane DPP reductions.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of this lane's DPP row, in every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x124>(x);  // row_ror 4
  x += dpp_mov<0x128>(x);  // row_ror 8
  return x;
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t idx, const float (&x)[8]) {
  if constexpr (BF16) {
    const f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
    *reinterpret_cast<bf16x8*>(static_cast<unsigned short*>(base) + idx) = pack8(lo, hi);
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx);
    p[0] = f32x4{x[0], x[1], x[2], x[3]};
    p[1] = f32x4{x[4], x[5], x[6], x[7]};
  }
}

template <bool BF16IO, bool BF16ST>
__global__ __launch_bounds__(256) void kda_decode_kernel(Params p) {
  const int64_t task = blockIdx.x;  // n * H + h
  const int64_t n = task / p.H;
  const int64_t h = task - n * p.H;
  if (n >= p.N) return;
  const int t = threadIdx.x;
  const int cb = t & 15;  // keys 8 cb .. 8 cb + 7
  const int r0 = t >> 4;  // rows r0 + 16 i
  const int64_t tok = n * p.H + h;  // token row of (n, h): B = N sequences of one token

  float q[8], k[8], g[8];
  load8<BF16IO>(p.q, tok * kD + 8 * cb, q);
  load8<BF16IO>(p.k, tok * kD + 8 * cb, k);
  load8<BF16IO>(p.g, tok * kD + 8 * cb, g);
  float beta = load1<BF16IO>(p.beta, tok);
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = load1<BF16IO>(p.v, tok * kD + r0 + 16 * i);

  if (p.flags & kFlagL2) {  // uniform
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq += q[e] * q[e];
      sk += k[e] * k[e];
    }
    const float iq = 1.0f / sqrtf(row_sum16(sq) + 1e-6f);
    const float ik = 1.0f / sqrtf(row_sum16(sk) + 1e-6f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q[e] *= iq;
      k[e] *= ik;
    }
  }
  if (p.flags & kFlagGate) {
    const float a = __expf(p.A_log[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      g[e] = p.lower_bound * sigmoidf_(a * (g[e] + p.dt_bias[h * kD + 8 * cb + e]));
  }
  if (p.flags & kFlagBetaLogit) beta = sigmoidf_(beta);

  float dk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dk[e] = __expf(g[e]);

  // State rows of this (sequence, head); a pool slot out of range starts from zero and
  // writes nothing.
  int64_t sbase = ((n * p.H + h) * kD) * kD;
  bool has_state = true;
  if (p.state_idx) {
    const int64_t slot = p.state_idx[n];
    has_state = slot >= 0 && slot < p.pool_slots;
    sbase = has_state ? slot * p.slot_pitch + h * kD * kD : 0;
  }
  float s[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (p.state_in && has_state) {
      load8<BF16ST>(p.state_in, sbase + (r0 + 16 * i) * kD + 8 * cb, s[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) s[i][e] = 0.f;
    }
  }
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float pk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[i][e] *= dk[e];  // decay every key channel
      pk += s[i][e] * k[e];
    }
    const float u = beta * (v[i] - row_sum16(pk));  // delta-rule error of the prediction
    float pq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[i][e] += u * k[e];  // write
      pq += s[i][e] * q[e];
    }
    o[i] = p.scale * row_sum16(pq);  // read with the updated state
  }
  if (p.state_out && has_state) {
#pragma unroll
    for (int i = 0; i < 8; ++i) store8<BF16ST>(p.state_out, sbase + (r0 + 16 * i) * kD + 8 * cb, s[i]);
  }
  // Lane cb of each row stores o for row r0 + 16 cb (cb < 8).
  float mine = o[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mine = cb == i ? o[i] : mine;
  if (cb < 8) {
    const int64_t at = tok * kD + r0 + 16 * cb;
    if constexpr (BF16IO)
      static_cast<unsigned short*>(p.o)[at] = float_to_bf16_bits(mine);
    else
      static_cast<float*>(p.o)[at] = mine;
  }
}

}  // namespace

hipError_t launch_decode(const Params& p, bool io_bf16, bool state_bf16, hipStream_t stream) {
  const int64_t wgs = p.N * p.H;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(wgs));
  if (io_bf16) {
    if (state_bf16) hipLaunchKernelGGL((kda_decode_kernel<true, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kda_decode_kernel<true, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (state_bf16) hipLaunchKernelGGL((kda_decode_kernel<false, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kda_decode_kernel<false, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace kda
