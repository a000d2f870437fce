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
// state passes through). When order is given (N <= kAutoOrderMax), also the sequences
// by decreasing chunk count, ties by index: the order in which the serial recurrence
// starts them, so that the longest do not start last.
__global__ __launch_bounds__(256) void kda_plan_kernel(const int64_t* __restrict__ cu,
                                                        int64_t N, int64_t seg_len,
                                                        int64_t* __restrict__ cu_chunks,
                                                        int64_t* __restrict__ cu_segs,
                                                        int32_t* __restrict__ order) {
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
  if (order && N <= kAutoOrderMax) {  // uniform
    __shared__ int64_t cnt[kAutoOrderMax];
    int64_t c = 0;
    if (t < N) {
      const int64_t len = cu[t + 1] - cu[t];
      c = len > 0 ? (len + kC - 1) / kC : 0;
      cnt[t] = c;
    }
    __syncthreads();
    if (t < N) {
      // rank = sequences that come first: more chunks, or as many with a lower index
      int rank = 0;
      for (int j = 0; j < N; ++j) rank += (cnt[j] > c) || (cnt[j] == c && j < t);
      order[rank] = t;
    }
  }
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations, not for its
// global stores (the record stores are never read back by this kernel, and waiting for
// them at every barrier would add an HBM write round trip each time).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Record tiles are stored non-temporally: a record is read once, by the recurrence
// launch, long after it is written. Measured against plain stores (bitwise the same
// results): the recurrence at T = 8192 took 286 instead of 303 us at H=96, 133 instead
// of 147 us at H=24, and a whole H=6 call 72 instead of 74 us (H=12 alone lost ~2 us),
// because dirty record lines no longer wait in L2 to be written back while the
// recurrence streams.
template <typename V>
__device__ __forceinline__ void store_record(unsigned char* at, V v) {
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(at));
}

// DPP within 16-lane rows: lane r receives lane r - N of its row (0 past the row start),
// or lane N of its row.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}

// Token range of chunk gc (over all sequences, in order): first token and the number
// of real tokens (0..16). False past the last chunk (varlen: the plan's count).
struct ChunkSpan {
  int64_t tok0;
  int64_t valid;
};

__device__ __forceinline__ bool chunk_span(const Params& p, int64_t gc, ChunkSpan& sp) {
  if (p.cu_seqlens) {
    const int64_t total = p.cu_chunks[p.N];
    if (gc >= total) return false;
    int64_t lo = 0, hi = p.N;  // first index with cu_chunks[idx] > gc
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (p.cu_chunks[mid] > gc) hi = mid; else lo = mid + 1;
    }
    const int64_t s = lo > 0 ? lo - 1 : 0;
    const int64_t end = min(p.cu_seqlens[s + 1], p.T);
    sp.tok0 = p.cu_seqlens[s] + kC * (gc - p.cu_chunks[s]);
    sp.valid = min<int64_t>(kC, end - sp.tok0);
  } else {
    const int64_t s = gc / p.chunks_per_seq;
    const int64_t lc = gc - s * p.chunks_per_seq;
    sp.tok0 = s * p.T + kC * lc;
    sp.valid = min<int64_t>(kC, p.T - kC * lc);
  }
  if (sp.tok0 < 0) sp.valid = 0;
  return true;
}

// 8 consecutive elements of one row as loaded (BF16: one 16-byte piece; FP32: two).
template <bool BF16>
struct RawRow {
  u32x4 w[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ void to_float(const RawRow<BF16>& x, float* out) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(x.w[0][i] << 16);
      out[2 * i + 1] = __uint_as_float(x.w[0][i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = __uint_as_float(x.w[0][i]);
      out[4 + i] = __uint_as_float(x.w[1][i]);
    }
  }
}

// This thread's q, k, g pieces (token r, channels cq .. cq + 7) of a chunk, zeros past its
// valid tokens; beta of token tid for tid < 16.
template <bool BF16>
__device__ __forceinline__ void load_rows(const Params& p, const ChunkSpan& sp, int64_t h, int r,
                                          int cq, int tid, RawRow<BF16>& q, RawRow<BF16>& k,
                                          RawRow<BF16>& g, float& beta) {
  constexpr int ES = BF16 ? 2 : 4;
  if (r < sp.valid) {
    const int64_t off = (((sp.tok0 + r) * p.H + h) * kD + cq) * ES;
#pragma unroll
    for (int i = 0; i < (BF16 ? 1 : 2); ++i) {
      q.w[i] = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.q) + off + 16 * i);
      k.w[i] = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.k) + off + 16 * i);
      g.w[i] = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.g) + off + 16 * i);
    }
  } else {
#pragma unroll
    for (int i = 0; i < (BF16 ? 1 : 2); ++i) q.w[i] = k.w[i] = g.w[i] = u32x4{0u, 0u, 0u, 0u};
  }
  beta = 0.f;
  if (tid < kC && tid < sp.valid) beta = load1<BF16>(p.beta, (sp.tok0 + tid) * p.H + h);
}

// At most 64 registers and 20 KB of LDS, so that eight workgroups (32 waves) share a
// compute unit: the kernel is bound by the latency of its arithmetic and barrier
// chains, which only more resident waves hide.
template <bool BF16, bool HEADS_FAST>
__global__ __launch_bounds__(256, 8) void kda_prepare_kernel(Params p) {
  // bf16 tiles [token][channel]: MFMA operands and the K_end^T record gather.
  __shared__ __attribute__((aligned(16))) unsigned short sKs[kC][kD];  // K_start rows
  __shared__ __attribute__((aligned(16))) unsigned short sQs[kC][kD];  // Q_start rows
  __shared__ __attribute__((aligned(16))) unsigned short sKi[kC][kD];  // k / Gamma rows
  __shared__ __attribute__((aligned(16))) unsigned short sKe[kC][kD];  // K_end rows
  __shared__ __attribute__((aligned(16))) float sR[kC][kC];
  __shared__ __attribute__((aligned(16))) float sA[kC][kC];
  __shared__ __attribute__((aligned(16))) float sM[kC][kC];
  __shared__ __attribute__((aligned(16))) float sP[kC][kC];
  // The L2 norm partials (first phase) and beta (read last by the solve) live in the P
  // tile, which is written only after the solve: 20 KB per workgroup, eight per CU.
  float(*sNorm)[4][kC] = reinterpret_cast<float(*)[4][kC]>(&sP[0][0]);  // [2][4][16]
  float* sBeta = &sP[8][0];

  const int tid = threadIdx.x;
  // HEADS_FAST: workgroup (x, y) prepares head x % H of chunk y * cb + x / H (cb =
  // gridDim.x / H chunks per grid row), so the workgroups resident at a time read whole
  // token rows of q, k and g. Otherwise workgroup (x, y) is chunk x of head y, and
  // consecutive workgroups write consecutive records of a head.
  int64_t h, gc;
  if constexpr (HEADS_FAST) {
    const int64_t cb = static_cast<int64_t>(gridDim.x) / p.H;
    h = static_cast<int64_t>(blockIdx.x) % p.H;
    gc = static_cast<int64_t>(blockIdx.y) * cb + static_cast<int64_t>(blockIdx.x) / p.H;
    if (gc >= p.max_chunks) return;  // the last grid row's tail (uniform)
  } else {
    h = blockIdx.y;
    gc = blockIdx.x;
  }
  // Thread (r, c8): token r = tid % 16, channels 8 c8 .. 8 c8 + 7, c8 = tid / 16, so the
  // 16 tokens of a channel group form one 16-lane row (the prefix over tokens is a
  // row scan).
  const int r = tid & 15;
  const int cq = (tid >> 4) * 8;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  ChunkSpan span;
  if (!chunk_span(p, gc, span)) return;  // uniform over the workgroup
  RawRow<BF16> rq, rk, rg;
  float rbeta;
  load_rows<BF16>(p, span, h, r, cq, tid, rq, rk, rg, rbeta);
  // The gate's per-head parameters, loaded with the rows (independent of them).
  float gate_a = 0.f, dtb[8];
  if (p.flags & kFlagGate) {
    gate_a = p.A_log[h];
#pragma unroll
    for (int e = 0; e < 8; ++e) dtb[e] = p.dt_bias[h * kD + cq + e];
  }
  const int64_t valid = span.valid;
  unsigned char* rec = p.records + (h * p.max_chunks + gc) * (int64_t)kRecord;

  // ---- this chunk's rows and the optional transforms -------------------------------
  const bool tv = r < valid;
  float q[8], k[8], g[8];
  to_float<BF16>(rq, q);
  to_float<BF16>(rk, k);
  to_float<BF16>(rg, g);
  if (tid < kC) {
    float b = rbeta;
    if ((p.flags & kFlagBetaLogit) && tid < valid) b = sigmoidf_(b);
    sBeta[tid] = b;
  }
  if (p.flags & kFlagL2) {  // uniform branch
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq += q[e] * q[e];
      sk += k[e] * k[e];
    }
    // the 4 channel groups of this wave, then the 4 waves
    sq += __shfl_xor(sq, 16);
    sk += __shfl_xor(sk, 16);
    sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 32);
    if (lane < 16) {
      sNorm[0][wave][r] = sq;
      sNorm[1][wave][r] = sk;
    }
    lds_barrier();
    sq = sNorm[0][0][r] + sNorm[0][1][r] + sNorm[0][2][r] + sNorm[0][3][r];
    sk = sNorm[1][0][r] + sNorm[1][1][r] + sNorm[1][2][r] + sNorm[1][3][r];
    const float iq = rsqrtf(sq + 1e-6f);
    const float ik = rsqrtf(sk + 1e-6f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q[e] *= iq;
      k[e] *= ik;
    }
  }
  if ((p.flags & kFlagGate) && tv) {
    const float a = __expf(gate_a);
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = p.lower_bound * sigmoidf_(a * (g[e] + dtb[e]));
  }

  // ---- prefix decay (row scan over tokens) and the decayed key/query rows ----------
  float G[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = g[e];
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    G[e] = x;
  }
  // exp(G_15) is token 15's exp(G): a row broadcast instead of a third exponential.
  // Over one chunk G >= -80 (g >= -5), so exp(+-G) and their product stay in FP32 range.
  float gam[8], E15[8];
  unsigned short bks[8], bqs[8], bki[8], bke[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    gam[e] = __expf(G[e]);
    E15[e] = row_bcast<15>(gam[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float igam = __expf(-G[e]);
    bks[e] = float_to_bf16_bits(gam[e] * k[e]);
    bqs[e] = float_to_bf16_bits(gam[e] * q[e]);
    bki[e] = float_to_bf16_bits(igam * k[e]);
    bke[e] = float_to_bf16_bits(E15[e] * igam * k[e]);
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
      const int b = key >> 4, gg = (key >> 2) & 3, hh = (key >> 1) & 1;
      const int L = 16 * gg + 2 * b + hh;
      f32x2 v;
      v[0] = E15[e];
      v[1] = E15[e + 1];
      // (8-byte pieces stay ordinary stores: non-temporal ones write partial lines)
      *reinterpret_cast<f32x2*>(rec + kOffD + L * 8) = v;
    }
  }
  lds_barrier();

  // ---- R and A_qk on MFMA (waves 0, 1); K_end record (all threads) ----------------
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
    store_record(rec + kOffKeT + 16 * tid, *reinterpret_cast<const u32x4*>(out));
  }
  lds_barrier();

  // ---- Mb = (I + R)^{-1} B by forward substitution, one column per thread ----------
  if (tid < kC) {
    const int c = tid;
    float x[kC];
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      float acc = i == c ? 1.f : 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        if (4 * q4 < i) {
          const f32x4 rv = *reinterpret_cast<const f32x4*>(&sR[i][4 * q4]);  // broadcast
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (4 * q4 + t < i) acc -= rv[t] * x[4 * q4 + t];
        }
      }
      x[i] = acc;
    }
    const float bc = sBeta[c];
#pragma unroll
    for (int i = 0; i < kC; ++i) sM[i][c] = x[i] * bc;
  }
  lds_barrier();

  // ---- P = A_qk Mb ---------------------------------------------------------------
  {
    const int mi = tid >> 4;
    const int c = tid & 15;
    float acc = 0.f;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(&sA[mi][4 * i4]);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc += av[t] * sM[4 * i4 + t][c];
    }
    sP[mi][c] = acc;
  }
  lds_barrier();

  // ---- Kn^T = -K_start^T Mb^T and Qt^T = s Q_start^T - K_start^T P^T on MFMA --------
  // With the key blocks as MFMA rows, lane (grp, m) of block b ends up holding
  // Kn[m][16 b + 4 grp + j], which is the record's operand order: wave kb writes the
  // pieces of key blocks 2 kb and 2 kb + 1 directly.
  {
    const int kb = wave;
    const f32x4 mrow = *reinterpret_cast<const f32x4*>(&sM[m][4 * grp]);
    const f32x4 prow = *reinterpret_cast<const f32x4*>(&sP[m][4 * grp]);
    const i16x4 bM = pack4(-mrow);  // B[token 4 grp + j][token m] = -Mb[m][4 grp + j]
    const i16x4 bP = pack4(-prow);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    i16x4 kn[2], qt[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int b = 2 * kb + half;
      i16x4 a;  // A[key 16 b + m][token 4 grp + j] = K_start[4 grp + j][16 b + m]
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = static_cast<short>(sKs[4 * grp + j][16 * b + m]);
      // s Q_start^T enters as the accumulator, from the BF16 Q_start tile.
      const u32x2 qs = *reinterpret_cast<const u32x2*>(&sQs[m][16 * b + 4 * grp]);
      f32x4 qinit;
      qinit[0] = p.scale * __uint_as_float(qs[0] << 16);
      qinit[1] = p.scale * __uint_as_float(qs[0] & 0xffff0000u);
      qinit[2] = p.scale * __uint_as_float(qs[1] << 16);
      qinit[3] = p.scale * __uint_as_float(qs[1] & 0xffff0000u);
      kn[half] = pack4(mfma16(a, bM, zero));
      qt[half] = pack4(mfma16(a, bP, qinit));
    }
    const u32x2 k0 = __builtin_bit_cast(u32x2, kn[0]), k1 = __builtin_bit_cast(u32x2, kn[1]);
    const u32x2 q0 = __builtin_bit_cast(u32x2, qt[0]), q1 = __builtin_bit_cast(u32x2, qt[1]);
    store_record(rec + kOffKn + kb * 1024 + lane * 16, u32x4{k0[0], k0[1], k1[0], k1[1]});
    store_record(rec + kOffQt + kb * 1024 + lane * 16, u32x4{q0[0], q0[1], q1[0], q1[1]});
    if (wave == 0) {  // [L 64][Mb j 4, A_qk j 4]
      const f32x4 arow = *reinterpret_cast<const f32x4*>(&sA[m][4 * grp]);
      const u32x2 mb = __builtin_bit_cast(u32x2, pack4(mrow));
      const u32x2 aq = __builtin_bit_cast(u32x2, pack4(arow));
      store_record(rec + kOffMbAq + 16 * lane, u32x4{mb[0], mb[1], aq[0], aq[1]});
    }
  }
}

hipError_t launch_plan(const Params& p, int32_t* auto_order, hipStream_t stream) {
  const int64_t seg_len = p.seg_len;  // 0: serial recurrence, no segment prefix
  hipLaunchKernelGGL(kda_plan_kernel, dim3(1), dim3(256), 0, stream, p.cu_seqlens, p.N,
                     seg_len, p.cu_chunks, p.cu_segs, auto_order);
  return hipGetLastError();
}

hipError_t launch_prepare(const Params& p, bool io_bf16, hipStream_t stream) {
  if (p.max_chunks <= 0 || p.H <= 0) return hipSuccess;
  // Which neighbours in dispatch order share a workgroup's memory pages: with many heads
  // the input reads from HBM dominate and the heads of a chunk go together (one token
  // row of q, k and g is H * 256 contiguous bytes); with few heads the inputs mostly sit
  // in the last-level cache and the record writes dominate, and a head's consecutive
  // chunks go together. Measured per prepare (T = 8192, same box): H = 96 259.2 -> 254.9
  // us and H = 48 132.5 -> 129.5 us with heads fastest; H = 24 even; H = 6 17.8 -> 18.6
  // us and the 8-sequence H = 24 varlen workload 223.2 -> 226.8 us the other way.
  const bool heads_fast = p.H >= 32;
  dim3 grid;
  if (heads_fast) {
    // Grid rows of cb chunks: 64, more when the chunk count would need more than 65535
    // rows.
    int64_t cb = p.max_chunks < 64 ? p.max_chunks : 64;
    if ((p.max_chunks + cb - 1) / cb > 65535) cb = (p.max_chunks + 65534) / 65535;
    const int64_t gx = cb * p.H;
    const int64_t gy = (p.max_chunks + cb - 1) / cb;
    if (gx * 256 > 0xffffffffLL || gy > 65535) return hipErrorInvalidValue;
    grid = dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
  } else {
    if (p.max_chunks * 256 > 0xffffffffLL || p.H > 65535) return hipErrorInvalidValue;
    grid = dim3(static_cast<unsigned>(p.max_chunks), static_cast<unsigned>(p.H));
  }
  if (heads_fast) {
    if (io_bf16) hipLaunchKernelGGL((kda_prepare_kernel<true, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kda_prepare_kernel<false, true>), grid, dim3(256), 0, stream, p);
  } else {
    if (io_bf16) hipLaunchKernelGGL((kda_prepare_kernel<true, false>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kda_prepare_kernel<false, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace kda
