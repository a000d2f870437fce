// kda_decode: a few tokens per sequence (T <= kDecodeMaxT = 8, fixed layout), the token
// step itself, token after token:
//   S <- S Diag(exp g) ; u = beta (v - S k) ; S <- S + u k^T ; o = s S q
// (the one-token case of the chunk equations of the "FlashKDA column split" post,
// section 1; with T = 1 a decode step, with a few tokens the verification of draft
// tokens). With so few tokens the chunk machinery has nothing to amortise: this kernel
// reads each (sequence, head) state once, applies the T token steps in registers and
// writes it back, so it is bound by the 2 x 32 KB (BF16) of state traffic per head plus
// the tokens' own rows.
//
// One 256-thread workgroup per (sequence, head). Thread t holds the 16-byte state
// pieces t + 256 i (i = 0..7): row r = t / 16 + 16 i, keys 8 (t % 16) .. + 7, so that one
// wave instruction reads four whole 256-byte rows, and the 16 lanes of a DPP row hold
// one state row; row sums (S k, S q) are 16-lane DPP reductions. The next token's rows
// are loaded (as raw bits) while the current one is applied.

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

// One token's inputs for this thread, as loaded: q, k, g channels 8 cb .. 8 cb + 7,
// v rows r0 + 16 i, beta.
template <bool BF16IO>
struct TokenIn {
  u32x4 q[BF16IO ? 1 : 2], k[BF16IO ? 1 : 2], g[BF16IO ? 1 : 2];
  float v[8];
  float beta;
};

template <bool BF16IO>
__device__ __forceinline__ void load_token(TokenIn<BF16IO>& x, const Params& p, int64_t tok,
                                           int cb, int r0) {
  constexpr int W = BF16IO ? 1 : 2;  // 16-byte pieces per 8 channels
  const int64_t c = tok * kD + 8 * cb;
  const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const char*>(p.q) + c * (BF16IO ? 2 : 4));
  const u32x4* k = reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k) + c * (BF16IO ? 2 : 4));
  const u32x4* g = reinterpret_cast<const u32x4*>(static_cast<const char*>(p.g) + c * (BF16IO ? 2 : 4));
#pragma unroll
  for (int w = 0; w < W; ++w) {
    x.q[w] = q[w];
    x.k[w] = k[w];
    x.g[w] = g[w];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x.v[i] = load1<BF16IO>(p.v, tok * kD + r0 + 16 * i);
  x.beta = load1<BF16IO>(p.beta, tok);
}

template <bool BF16IO>
__device__ __forceinline__ void unpack8(const u32x4 (&w)[BF16IO ? 1 : 2], float (&out)[8]) {
  if constexpr (BF16IO) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[0][i] << 16);
      out[2 * i + 1] = __uint_as_float(w[0][i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = __uint_as_float(w[0][i]);
      out[4 + i] = __uint_as_float(w[1][i]);
    }
  }
}

// MULTI: T > 1 (the next token's rows are prefetched during the current one); a single
// token keeps the registers of that prefetch free, for more resident waves.
template <bool BF16IO, bool BF16ST, bool MULTI>
__global__ __launch_bounds__(256) void kda_decode_kernel(Params p) {
  const int64_t task = blockIdx.x;  // n * H + h
  const int64_t n = task / p.H;
  const int64_t h = task - n * p.H;
  if (n >= p.N) return;
  const int t = threadIdx.x;
  const int cb = t & 15;  // keys 8 cb .. 8 cb + 7
  const int r0 = t >> 4;  // rows r0 + 16 i
  const int64_t T = MULTI ? p.T : 1;

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
  // Per-head gate parameters (the in-kernel gate), loaded once.
  float gate_a = 0.f, dtb[8];
  if (p.flags & kFlagGate) {
    gate_a = __expf(p.A_log[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) dtb[e] = p.dt_bias[h * kD + 8 * cb + e];
  }

  TokenIn<BF16IO> cur, nxt;
  if (T > 0) load_token<BF16IO>(cur, p, (n * T) * p.H + h, cb, r0);
#pragma unroll 1
  for (int64_t tt = 0; tt < T; ++tt) {
    const int64_t tok = (n * T + tt) * p.H + h;  // token row of (n, tt, h)
    if (MULTI && tt + 1 < T) load_token<BF16IO>(nxt, p, tok + p.H, cb, r0);
    float q[8], k[8], g[8];
    unpack8<BF16IO>(cur.q, q);
    unpack8<BF16IO>(cur.k, k);
    unpack8<BF16IO>(cur.g, g);
    float beta = cur.beta;
    if (p.flags & kFlagL2) {  // uniform
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq += q[e] * q[e];
        sk += k[e] * k[e];
      }
      const float iq = rsqrtf(row_sum16(sq) + 1e-6f);
      const float ik = rsqrtf(row_sum16(sk) + 1e-6f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        q[e] *= iq;
        k[e] *= ik;
      }
    }
    if (p.flags & kFlagGate) {
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = p.lower_bound * sigmoidf_(gate_a * (g[e] + dtb[e]));
    }
    if (p.flags & kFlagBetaLogit) beta = sigmoidf_(beta);

    float dk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dk[e] = __expf(g[e]);
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float pk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[i][e] *= dk[e];  // decay every key channel
        pk += s[i][e] * k[e];
      }
      const float u = beta * (cur.v[i] - row_sum16(pk));  // delta-rule error of the prediction
      float pq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[i][e] += u * k[e];  // write
        pq += s[i][e] * q[e];
      }
      o[i] = p.scale * row_sum16(pq);  // read with the updated state
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
    if constexpr (MULTI) cur = nxt;
  }
  if (p.state_out && has_state) {
#pragma unroll
    for (int i = 0; i < 8; ++i) store8<BF16ST>(p.state_out, sbase + (r0 + 16 * i) * kD + 8 * cb, s[i]);
  }
}

}  // namespace

template <bool BF16IO, bool BF16ST>
void launch_decode_io(const Params& p, dim3 grid, hipStream_t stream) {
  if (p.T > 1)
    hipLaunchKernelGGL((kda_decode_kernel<BF16IO, BF16ST, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((kda_decode_kernel<BF16IO, BF16ST, false>), grid, dim3(256), 0, stream, p);
}

hipError_t launch_decode(const Params& p, bool io_bf16, bool state_bf16, hipStream_t stream) {
  const int64_t wgs = p.N * p.H;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(wgs));
  if (io_bf16) {
    if (state_bf16) launch_decode_io<true, true>(p, grid, stream);
    else launch_decode_io<true, false>(p, grid, stream);
  } else {
    if (state_bf16) launch_decode_io<false, true>(p, grid, stream);
    else launch_decode_io<false, false>(p, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace kda
