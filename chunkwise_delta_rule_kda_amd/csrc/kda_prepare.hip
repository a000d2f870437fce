// kda_prepare: one workgroup (256 threads) per (16-token chunk, head).
//
// Builds the per-chunk quantities of the "FlashKDA column split" post, section 1
// ("FlashKDA in two kernels"): K_start (column i = D_{0:i} k_i), Q_start, K_end
// (row i = k_i^T D_{i+1:15}), D_{0:15}, R_ij = beta_i <k_j|D_{j+1:i}|k_i> (j < i),
// A_kk = (I + R)^{-1} and A_qk_ij = s <k_j|D_{j+1:i}|q_i> (j <= i). The decayed products
// use the split-exponent form of the K3 decay page (section "How the per-channel decay
// factor exp(G) enters tile computation"): with G_i the prefix sum of g through token i,
// <k_j|D_{j+1:i}|k_i> = sum_c (exp(G_i) k_i)[c] (exp(-G_j) k_j)[c], one dense 16x16x128
// product on MFMA. The lower bound g >= -5 keeps exp(+-G) inside FP32/BF16 range over 16
// tokens (same page, "Why a diagonal tile needs lower-bounded decay").
//
// The record it writes folds A_kk, B and A_qk into the key-side operands so the serial
// recurrence has one K=128 contraction and one K=16 update on its critical path:
//   Mb = A_kk B, Kn = -Mb K_start^T, Qt = s Q_start^T + A_qk Kn  (layout: include/kda.h).
// All math is FP32; MFMA operands are BF16 with FP32 accumulation.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Exclusive prefixes over the packed sequences: cu_chunks[0..N] of ceil(len_n / 16),
// and, when seg_len > 0, cu_segs[0..N] of max(1, ceil(chunks_n / seg_len)) (the number
// of time segments of sequence n; a zero-length sequence keeps one empty segment so its
// state passes through).
__global__ __launch_bounds__(256) void kda_plan_kernel(const int64_t* __restrict__ cu,
                                                        int64_t N, int64_t seg_len,
                                                        int64_t* __restrict__ cu_chunks,
                                                        int64_t* __restrict__ cu_segs) {
  __shared__ int64_t buf[2][256];
  __shared__ int64_t carry[2];
  const int t = threadIdx.x;
  if (t == 0) {
    carry[0] = carry[1] = 0;
    cu_chunks[0] = 0;
    if (seg_len > 0) cu_segs[0] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < N; base += 256) {
    const int64_t i = base + t;
    int64_t c = 0, sg = 0;
    if (i < N) {
      const int64_t len = cu[i + 1] - cu[i];
      c = len > 0 ? (len + kC - 1) / kC : 0;
      if (seg_len > 0) sg = c > 0 ? (c + seg_len - 1) / seg_len : 1;
    }
    buf[0][t] = c;
    buf[1][t] = sg;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int64_t x0 = t >= off ? buf[0][t - off] : 0;
      const int64_t x1 = t >= off ? buf[1][t - off] : 0;
      __syncthreads();
      buf[0][t] += x0;
      buf[1][t] += x1;
      __syncthreads();
    }
    if (i < N) {
      cu_chunks[i + 1] = carry[0] + buf[0][t];
      if (seg_len > 0) cu_segs[i + 1] = carry[1] + buf[1][t];
    }
    __syncthreads();
    if (t == 0) {
      carry[0] += buf[0][255];
      carry[1] += buf[1][255];
    }
    __syncthreads();
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void kda_prepare_kernel(Params p) {
  // fp32 tiles [token][channel]; sG is reused for Kn and sQf ends up holding Qt.
  __shared__ __attribute__((aligned(16))) float sG[kC][kD];
  __shared__ __attribute__((aligned(16))) float sQf[kC][kD];
  // bf16 tiles [token][channel]
  __shared__ __attribute__((aligned(16))) unsigned short sKs[kC][kD];
  __shared__ __attribute__((aligned(16))) unsigned short sQs[kC][kD];
  __shared__ __attribute__((aligned(16))) unsigned short sKi[kC][kD];
  __shared__ __attribute__((aligned(16))) unsigned short sKe[kC][kD];
  __shared__ float sBeta[kC];
  __shared__ float sR[kC][kC + 1];
  __shared__ float sA[kC][kC + 1];
  __shared__ float sM[kC][kC + 1];
  __shared__ __attribute__((aligned(16))) unsigned short sNM[kC][kC];
  __shared__ __attribute__((aligned(16))) unsigned short sNP[kC][kC];

  const int tid = threadIdx.x;
  const int64_t gc = blockIdx.x;
  const int64_t h = blockIdx.y;
  const int64_t H = p.H;

  int64_t tok0, valid;
  if (p.cu_seqlens) {
    const int64_t total = p.cu_chunks[p.N];
    if (gc >= total) return;  // uniform over the workgroup
    int64_t lo = 0, hi = p.N;  // first index with cu_chunks[idx] > gc
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (p.cu_chunks[mid] > gc) hi = mid; else lo = mid + 1;
    }
    const int64_t s = lo > 0 ? lo - 1 : 0;
    const int64_t end = min(p.cu_seqlens[s + 1], p.T);
    tok0 = p.cu_seqlens[s] + kC * (gc - p.cu_chunks[s]);
    valid = min<int64_t>(kC, end - tok0);
  } else {
    const int64_t s = gc / p.chunks_per_seq;
    const int64_t lc = gc - s * p.chunks_per_seq;
    tok0 = s * p.T + kC * lc;
    valid = min<int64_t>(kC, p.T - kC * lc);
  }
  if (tok0 < 0) valid = 0;
  unsigned char* rec = p.records + (h * p.max_chunks + gc) * (int64_t)kRecord;

  // ---- load the chunk's rows and apply the optional transforms -------------------
  const int r = tid >> 4;         // token of the chunk
  const int cq = (tid & 15) * 8;  // first of this thread's 8 channels
  const bool tv = r < valid;
  const int64_t row = (tok0 + r) * H + h;
  float q[8], k[8], g[8];
  if (tv) {
    load8<BF16>(p.q, row * kD + cq, q);
    load8<BF16>(p.k, row * kD + cq, k);
    load8<BF16>(p.g, row * kD + cq, g);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = k[e] = g[e] = 0.f;
  }
  if (p.flags & kFlagL2) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq += q[e] * q[e];
      sk += k[e] * k[e];
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      sq += __shfl_xor(sq, off, 16);
      sk += __shfl_xor(sk, off, 16);
    }
    const float iq = 1.0f / sqrtf(sq + 1e-6f);
    const float ik = 1.0f / sqrtf(sk + 1e-6f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q[e] *= iq;
      k[e] *= ik;
    }
  }
  if ((p.flags & kFlagGate) && tv) {
    const float a = __expf(p.A_log[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      g[e] = p.lower_bound * sigmoidf_(a * (g[e] + p.dt_bias[h * kD + cq + e]));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sG[r][cq + e] = g[e];
  if ((tid & 15) == 0) {
    float b = tv ? load1<BF16>(p.beta, row) : 0.f;
    if ((p.flags & kFlagBetaLogit) && tv) b = sigmoidf_(b);
    sBeta[r] = b;
  }
  __syncthreads();

  // ---- prefix decay and the decayed key/query rows --------------------------------
  float G[8], G15[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) G[e] = G15[e] = 0.f;
#pragma unroll
  for (int t = 0; t < kC; ++t) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = sG[t][cq + e];
      G15[e] += x;
      if (t <= r) G[e] += x;
    }
  }
  unsigned short bks[8], bqs[8], bki[8], bke[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float gam = __expf(G[e]);
    const float igam = __expf(-G[e]);
    const float tail = __expf(G15[e] - G[e]);
    const float ks = gam * k[e];
    const float qs = gam * q[e];
    sQf[r][cq + e] = p.scale * qs;
    bks[e] = float_to_bf16_bits(ks);
    bqs[e] = float_to_bf16_bits(qs);
    bki[e] = float_to_bf16_bits(igam * k[e]);
    bke[e] = float_to_bf16_bits(tail * k[e]);
  }
  *reinterpret_cast<u32x4*>(&sKs[r][cq]) = *reinterpret_cast<const u32x4*>(bks);
  *reinterpret_cast<u32x4*>(&sQs[r][cq]) = *reinterpret_cast<const u32x4*>(bqs);
  *reinterpret_cast<u32x4*>(&sKi[r][cq]) = *reinterpret_cast<const u32x4*>(bki);
  *reinterpret_cast<u32x4*>(&sKe[r][cq]) = *reinterpret_cast<const u32x4*>(bke);
  if (r == 0) {
    // D_{0:15}, ordered for a row broadcast: lane L = 16 g + m holds the pair of keys
    // 16 (m / 2) + 4 g + 2 (m % 2) + {0, 1}, so that the 16 lanes of row g together hold
    // the 32 keys 16 b + 4 g + j that each of them needs.
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int key = cq + e;
      const int b = key >> 4, g = (key >> 2) & 3, hh = (key >> 1) & 1;
      const int L = 16 * g + 2 * b + hh;
      f32x2 v;
      v[0] = __expf(G15[e]);
      v[1] = __expf(G15[e + 1]);
      *reinterpret_cast<f32x2*>(rec + kOffD + L * 8) = v;
    }
  }
  __syncthreads();

  // ---- R and A_qk on MFMA (waves 0, 1); K_end record (all threads) ----------------
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 15;
  const int grp = lane >> 4;
  if (wave < 2) {
    const unsigned short(*Arows)[kD] = wave == 0 ? sKs : sQs;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Arows[m][32 * kb + 8 * grp]);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sKi[m][32 * kb + 8 * grp]);
      acc = mfma32(a, b, acc);
    }
    // lane holds the product for row i = 4 grp + j (token i) and column m (token j).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * grp + j;
      if (wave == 0)
        sR[i][m] = m < i ? sBeta[i] * acc[j] : 0.f;
      else
        sA[i][m] = m <= i ? p.scale * acc[j] : 0.f;
    }
  }
  {
    // K_end^T record, [bp 4][L 64][half 2][j 4] = K_end[4 grp(L) + j][16 (2 bp + half) +
    // m(L)]: one 16-byte piece per (block pair, lane), one per thread.
    const int bp = tid >> 6;
    const int L = tid & 63;
    unsigned short out[8];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        out[4 * half + j] = sKe[4 * (L >> 4) + j][16 * (2 * bp + half) + (L & 15)];
    *reinterpret_cast<u32x4*>(rec + kOffKeT + 16 * tid) = *reinterpret_cast<const u32x4*>(out);
  }
  __syncthreads();

  // ---- A_kk = (I + R)^{-1} by forward substitution, one column per thread ----------
  if (tid < kC) {
    const int c = tid;
    float x[kC];
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      float acc = i == c ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) acc -= sR[i][j] * x[j];
      x[i] = acc;
    }
    const float bc = sBeta[c];
#pragma unroll
    for (int i = 0; i < kC; ++i) sM[i][c] = x[i] * bc;  // Mb = A_kk B
  }
  __syncthreads();

  // ---- -Mb and -(A_qk Mb) as BF16 MFMA operands; Mb / A_qk records ----------------
  {
    const int mi = tid >> 4;
    const int c = tid & 15;
    float P = 0.f;
#pragma unroll
    for (int i = 0; i < kC; ++i) P += sA[mi][i] * sM[i][c];
    sNP[mi][c] = float_to_bf16_bits(-P);
    sNM[mi][c] = float_to_bf16_bits(-sM[mi][c]);
    if (tid < 64) {  // [L 64][Mb j 4, A_qk j 4]
      const int L = tid;
      const int mm = L & 15, g2 = L >> 4;
      unsigned short out[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[j] = float_to_bf16_bits(sM[mm][4 * g2 + j]);
        out[4 + j] = float_to_bf16_bits(sA[mm][4 * g2 + j]);
      }
      *reinterpret_cast<u32x4*>(rec + kOffMbAq + 16 * L) = *reinterpret_cast<const u32x4*>(out);
    }
  }
  __syncthreads();

  // ---- Kn = -Mb K_start^T and Qt = s Q_start^T - (A_qk Mb) K_start^T on MFMA --------
  {
    const i16x4 aM = *reinterpret_cast<const i16x4*>(&sNM[m][4 * grp]);
    const i16x4 aP = *reinterpret_cast<const i16x4*>(&sNP[m][4 * grp]);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * wave + bb;  // 16-key block
      i16x4 bk;
#pragma unroll
      for (int j = 0; j < 4; ++j) bk[j] = static_cast<short>(sKs[4 * grp + j][16 * b + m]);
      f32x4 qt;
#pragma unroll
      for (int j = 0; j < 4; ++j) qt[j] = sQf[4 * grp + j][16 * b + m];
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 kn = mfma16(aM, bk, zero);
      qt = mfma16(aP, bk, qt);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sG[4 * grp + j][16 * b + m] = kn[j];
        sQf[4 * grp + j][16 * b + m] = qt[j];
      }
    }
  }
  __syncthreads();

  // ---- Kn and Qt records in the recurrence's operand order --------------------------
  {
    const int f0 = 8 * tid;  // [kb 4][L 64][e 8]
    const int kb = f0 >> 9;
    const int L = (f0 >> 3) & 63;
    const int mm = L & 15, g2 = L >> 4;
    unsigned short a[8], b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = 32 * kb + 16 * (e >> 2) + 4 * g2 + (e & 3);
      a[e] = float_to_bf16_bits(sG[mm][key]);
      b[e] = float_to_bf16_bits(sQf[mm][key]);
    }
    *reinterpret_cast<u32x4*>(rec + kOffKn + 16 * tid) = *reinterpret_cast<const u32x4*>(a);
    *reinterpret_cast<u32x4*>(rec + kOffQt + 16 * tid) = *reinterpret_cast<const u32x4*>(b);
  }
}

hipError_t launch_plan(const Params& p, hipStream_t stream) {
  const int64_t seg_len = p.seg_len;  // 0: serial recurrence, no segment prefix
  hipLaunchKernelGGL(kda_plan_kernel, dim3(1), dim3(256), 0, stream, p.cu_seqlens, p.N,
                     seg_len, p.cu_chunks, p.cu_segs);
  return hipGetLastError();
}

hipError_t launch_prepare(const Params& p, bool io_bf16, hipStream_t stream) {
  if (p.max_chunks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.max_chunks), static_cast<unsigned>(p.H));
  if (io_bf16)
    hipLaunchKernelGGL(kda_prepare_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(kda_prepare_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
