// Producer waves of the fused recurrence: the chunk preparation of the "FlashKDA column
// split" post, section 1 ("FlashKDA in two kernels": K_start, Q_start, K_end, D_{0:15},
// A_kk = (I + R)^{-1}, A_qk), computed by the recurrence workgroup itself, one chunk per
// producer wave (four producer waves take the run's chunks in turn), straight into the
// LDS ring its compute waves read. The record an LDS slot receives is the folded record
// of include/kda.h (Mb = A_kk B, Kn = -Mb K_start^T, Qt = s Q_start^T + A_qk Kn, K_end^T,
// D), in the same lane layout, followed by the chunk's V tile; nothing of it goes
// through HBM. (kPaired below selects the other arrangement, measured and not taken: two
// waves per chunk, 64 keys each, exchanging partial sums.)
//
// Included by kda_recurrence_core.h inside namespace kda (anonymous namespace), after the
// Params / Task / MFMA helpers it uses.
//
// Lane layout of a producer wave (lane L = 16 grp + m): token m of the chunk, keys
// kappa(kb, grp, e) = 32 kb + 16 (e / 4) + 4 grp + e % 4 for its key groups kb, e = 0..7
// (the record's key order). The 16 tokens of a key set form one 16-lane row, so the
// prefix of g over the chunk is a DPP row scan and D_{0:15} = exp(G_15) a row
// broadcast, as in kda_prepare. Then:
// - R and A_qk are 16x16x32 MFMA products over the keys, with the scaled rows as
//   operands straight from registers (the K3 decay page's split-exponent form: decayed
//   key rows exp(G_i) k_i against exp(-G_j) k_j, safe because g >= -5 keeps |G| <= 80);
// - (I + R)^{-1} is a 16-step forward substitution in FP32 over 16 lanes (one column
//   each) with R's rows broadcast from a 1 KB LDS scratch, and P = A_qk Mb four FP32
//   16x16x4 MFMA products;
// - the key-major tiles the record needs (K_start^T as an MFMA operand, K_end^T) are
//   16x16 transposes done by a 16x16x16 MFMA against the identity in the operands' own
//   k order: exact (one BF16 term per output) and independent of how the hardware
//   assigns k to lanes;
// - Kn^T and Qt^T are 16x16x16 MFMA products, as in kda_prepare.
//
// Synchronisation is by counters in LDS, not by the workgroup barrier: a producer waits
// until every compute wave has read the slot's previous chunk (done[s] counts reads),
// writes the slot, waits for its writes and adds two to ready[s] (one per half of the
// slot, the count a pair of waves would reach); a compute wave waits until ready[s]
// counts both halves of its chunk, reads, and adds to done.
// Every wait is bounded: past kSpinLimit polls the wave sets the workgroup's abort flag
// and the call's status word (a device int the host can read) and every wave of the
// workgroup leaves its loop, so the kernel always ends.
#pragma once

namespace fused {

// Keys a producer wave covers: all 128 (kPaired false: one wave per chunk, one producer
// per SIMD, up to 256 registers) or 64 (kPaired true: two waves per chunk exchanging
// partial sums, two producers per SIMD next to each compute wave, at most 168 registers).
// Measured at T = 8192 (H = 96, serial form, 64-row workgroups) with an earlier state of
// the producer code: one wave per chunk 811 us, pairs 1192 us (the one-wave form as it
// stands takes about 970 us).
constexpr bool kPaired = false;
constexpr int producers(int w) { return kPaired && w < 8 ? 8 : 4; }
constexpr int kHalvesPerWave = kPaired ? 1 : 2;
constexpr int kSpinLimit = 1 << 22;    // polls of one bounded wait (~0.1 s with sleeps)
constexpr int kStatusTimeout = 1;      // status bit: an LDS wait timed out

constexpr int block_threads(int w) { return 64 * (w + producers(w)); }
// The ring takes most of the LDS, so one workgroup runs per compute unit: its own waves
// per SIMD are the occupancy the register budget is sized for.
constexpr int waves_per_simd(int w) { return (w + producers(w) + 3) / 4; }

template <bool BF16IO, int W>
struct Tile {
  static constexpr int ES = BF16IO ? 2 : 4;
  static constexpr int VROW = 16 * W * ES;          // bytes of one V-tile token row
  static constexpr int PARTS = VROW / 16;           // 16-byte pieces per token row
  static constexpr int SLOT = kRecord + kC * VROW;  // record + V tile
  static constexpr int NSLOT = W == 8 ? 5 : (BF16IO ? 6 : 5);  // ring depth
  static constexpr int NP = producers(W);
  static constexpr int NPAIR = NP / 2;
  static constexpr int NT = 64 * (W + NP);
  static constexpr int VPIECES = kC * PARTS;        // 16-byte pieces of the V tile
  static constexpr int VWAVE = VPIECES * kHalvesPerWave / 2;  // copied by one wave
  static constexpr int VPL = (VWAVE + 63) / 64;     // per producer lane
  static_assert(SLOT % 16 == 0, "slot alignment");
  static_assert(W * 2048 <= SLOT, "Phi staging fits one slot");
};

template <int NP>
struct Sync {
  int ready[8];                         // per slot: halves published, cumulative
  int done[8];                          // per slot: compute-wave reads, cumulative
  int pair[NP / 2 > 0 ? NP / 2 : 1];    // per pair: waves at the exchange, cumulative
  int fin;                              // compute waves past their last chunk
  int abort;                            // a bounded wait timed out
  float dtb[kD];                        // gate bias of the head (in-kernel gate)
  // per pair: [buffer (chunk parity)][half][R', A'] partial sums, [row 16][column 16]
  float part[kPaired ? NP / 2 : 1][2][2][2][kC][kC];
  float rows[NP][2][kC][kC];            // per producer: R rows, then Mb transposed
};

template <int NP>
using lds_sync = __attribute__((address_space(3))) Sync<NP>;

__device__ __forceinline__ int lds_load(const __attribute__((address_space(3))) int* p) {
  return *reinterpret_cast<const volatile __attribute__((address_space(3))) int*>(p);
}

__device__ __forceinline__ void lds_add(__attribute__((address_space(3))) int* p, int v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Leave after a timeout: raise the workgroup's abort flag and the call's status bit.
__device__ __noinline__ void give_up(__attribute__((address_space(3))) int* abort, int* status) {
  *reinterpret_cast<volatile __attribute__((address_space(3))) int*>(abort) = 1;
  if (status) __hip_atomic_fetch_or(status, kStatusTimeout, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
}

// Poll until *p >= target (false: abort raised or time limit; the caller leaves).
__device__ __forceinline__ bool wait_at_least(__attribute__((address_space(3))) int* abort,
                                              const __attribute__((address_space(3))) int* p,
                                              int target, int* status) {
  int spins = 0;
  while (lds_load(p) < target) {
    if (lds_load(abort)) return false;
    if (++spins > kSpinLimit) {
      give_up(abort, status);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// This wave's LDS operations are all complete.
__device__ __forceinline__ void lds_drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// DPP within 16-lane rows: lane r receives lane r - N of its row (0 past the row start).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}

// Lane N of this lane's 16-lane row (DPP row broadcast). Every lane is written, so no
// old value is needed and the move folds into the instruction that uses it.
template <int N>
__device__ __forceinline__ float bcast16(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}

// Raw inputs of one chunk for one producer lane (token m) of one half of the keys.
template <bool BF16IO, int VPL, bool XFORM>
struct Raw {
  typedef typename std::conditional<BF16IO, u32x2, u32x4>::type piece;
  // q, k, g: piece i = 2 kk + half holds keys 32 kb(kk) + 16 half + 4 grp + (0..3)
  piece q[4 * kHalvesPerWave], k[4 * kHalvesPerWave], g[4 * kHalvesPerWave];
  // with the in-kernel L2 norm, the other half's q and k (for the row norms only)
  piece qo[XFORM && kPaired ? 4 : 1], ko[XFORM && kPaired ? 4 : 1];
  float beta;
  u32x4 v[VPL];  // V-tile pieces hh VWAVE + lane + 64 i
};

template <bool BF16IO>
__device__ __forceinline__ f32x4 widen(u32x2 w) {
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
               __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
}
template <bool BF16IO>
__device__ __forceinline__ f32x4 widen(u32x4 w) {
  return __builtin_bit_cast(f32x4, w);
}

// Issue the loads of chunk j (of the run) for this lane and half hh of the keys: q, k, g
// and beta, and this half's V-tile pieces (rows t.vwg .. t.vwg + 16 W). Pad tokens read
// the chunk's first token (in bounds) and are zeroed (q = k = g = 0, beta = 0: the state
// passes through); the compute waves mask pad tokens of V, and lanes past the half-tile
// read its first piece (never stored).
template <bool BF16IO, int W, bool XFORM, typename R>
__device__ __forceinline__ void load_chunk(const Params& p, const Task& t, int64_t j, int lane,
                                           int hh, R& x) {
  using F = Tile<BF16IO, W>;
  constexpr int ES = F::ES;
  typedef typename R::piece piece;
  const int m = lane & 15;
  const int grp = lane >> 4;
  const int64_t c0 = t.tok0 + j * kC;
  const int64_t nvalid = t.tok_end - c0;  // >= 1 for a chunk of the run
  const bool tv = m < nvalid;
  const int64_t tok = c0 + (tv ? m : 0);
  const int64_t row = (tok * p.H + t.h) * kD;
  const unsigned char* q = static_cast<const unsigned char*>(p.q);
  const unsigned char* k = static_cast<const unsigned char*>(p.k);
  const unsigned char* g = static_cast<const unsigned char*>(p.g);
#pragma unroll
  for (int i = 0; i < 4 * kHalvesPerWave; ++i) {
    const int key = 32 * (kPaired ? 2 * hh + (i >> 1) : (i >> 1)) + 16 * (i & 1) + 4 * grp;
    const int64_t off = (row + key) * ES;
    const piece a = *reinterpret_cast<const piece*>(q + off);
    const piece b = *reinterpret_cast<const piece*>(k + off);
    const piece c = *reinterpret_cast<const piece*>(g + off);
    x.q[i] = tv ? a : piece{};
    x.k[i] = tv ? b : piece{};
    x.g[i] = tv ? c : piece{};
    if constexpr (XFORM && kPaired) {
      const int64_t oo = (row + key + 64 - 128 * hh) * ES;  // the other half's keys
      const piece a2 = *reinterpret_cast<const piece*>(q + oo);
      const piece b2 = *reinterpret_cast<const piece*>(k + oo);
      x.qo[i] = tv ? a2 : piece{};
      x.ko[i] = tv ? b2 : piece{};
    }
  }
  const float bt = load1<BF16IO>(p.beta, tok * p.H + t.h);
  x.beta = tv ? bt : 0.f;
  if (!t.vzero) {
    const unsigned char* v = static_cast<const unsigned char*>(p.v) + (t.h * kD + t.vwg) * ES;
#pragma unroll
    for (int i = 0; i < F::VPL; ++i) {
      const int pl = lane + 64 * i;
      const int pc = hh * F::VWAVE + (pl < F::VWAVE ? pl : 0);
      const int vt = pc / F::PARTS;
      const int64_t vtok = c0 + (vt < nvalid ? vt : 0);
      x.v[i] = *reinterpret_cast<const u32x4*>(v + vtok * p.H * kD * ES + (pc - vt * F::PARTS) * 16);
    }
  }
}

typedef __attribute__((address_space(3))) float lds_f;
typedef __attribute__((address_space(3))) f32x4 lds_f4;
typedef __attribute__((address_space(3))) u32x4 lds_v4;

__device__ __forceinline__ u32x4 join(i16x4 a, i16x4 b) {
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  return u32x4{x[0], x[1], y[0], y[1]};
}

// Producer wave pw: with pairs, half hh = pw % 2 of pair pp = pw / 2, chunks pp,
// pp + NPAIR, ... of the run, keys 64 hh .. 64 hh + 63; otherwise chunks pw, pw + NP, ...
// and all keys. Per chunk j:
//  1. the element-wise part of its two key groups (rows loaded one chunk of the pair
//     earlier) and its partial R', A' products, then the loads of chunk j + NPAIR;
//  2. with pairs, the exchange of partial sums with the other half (double-buffered by
//     chunk parity); then R, A_qk, Mb = (I + R)^{-1} B and P = A_qk Mb;
//  3. wait until the slot's previous chunk has been read, then the transposes and
//     products of its key groups, each piece stored to the slot as soon as it is formed,
//     its D entries, its V pieces (and Mb, A_qk from half 0);
//  4. wait for the stores, count its halves in ready[s].
// OUT: the record's Qt is needed (runs that write O). XFORM: the call has in-kernel
// transforms (a separate instantiation, so that the common one has no branch in its
// element-wise part).
template <bool BF16IO, int W, bool OUT, bool XFORM>
__device__ void producer_loop(const Params& p, const Task& t, lds_u8* ring,
                              lds_sync<producers(W)>* sy, int pw, int lane) {
  using F = Tile<BF16IO, W>;
  const int64_t nch = t.nch;
  constexpr int NKB = 2 * kHalvesPerWave;  // 32-key groups of this wave
  constexpr int STRIDE = kPaired ? F::NPAIR : F::NP;  // chunks between this wave's chunks
  const int pp = kPaired ? pw >> 1 : pw;
  const int hh = kPaired ? pw & 1 : 0;
  auto kb_of = [&](int kk) { return kPaired ? 2 * hh + kk : kk; };
  lds_f* sR = &sy->rows[pw][0][0][0];
  lds_f* sA = &sy->rows[pw][1][0][0];
  const bool gate = XFORM && (p.flags & kFlagGate);
  const bool l2 = XFORM && (p.flags & kFlagL2);
  const float gate_a = gate ? __expf(p.A_log[t.h]) : 0.f;
  // One row block of a run that carries the value rows writes the records out when
  // asked (they are the same for every row block).
  const bool keep = p.keep_records && OUT && !t.vzero && t.vwg == 0;
  constexpr float kLog2e = 1.4426950408889634f;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  Raw<BF16IO, F::VPL, XFORM> x;
  int64_t j = pp;
  if (j < nch) load_chunk<BF16IO, W, XFORM>(p, t, j, lane, hh, x);
  for (int gen = 0; j < nch; j += STRIDE, ++gen) {
    // The lane index, opaque to the compiler inside the loop: values derived from it
    // (masks, the identity operand, the unit row) are formed per chunk instead of being
    // hoisted out of the loop and held in registers across it.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int m = ln & 15;
    const int grp = ln >> 4;
    const int64_t nvalid = t.tok_end - (t.tok0 + j * kC);
    const bool tv = m < nvalid;
    // ---- 1. element-wise part -------------------------------------------------------
    float iq = 1.f, ik = 1.f;
    if (l2) {  // uniform branch
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int i = 0; i < 2 * NKB; ++i) {
        const f32x4 a = widen<BF16IO>(x.q[i]), b = widen<BF16IO>(x.k[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sq += a[e] * a[e];
          sk += b[e] * b[e];
        }
        if constexpr (kPaired) {
          const f32x4 a2 = widen<BF16IO>(x.qo[i]), b2 = widen<BF16IO>(x.ko[i]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sq += a2[e] * a2[e];
            sk += b2[e] * b2[e];
          }
        }
      }
      sq += __shfl_xor(sq, 16);
      sk += __shfl_xor(sk, 16);
      sq += __shfl_xor(sq, 32);
      sk += __shfl_xor(sk, 32);
      iq = rsqrtf(sq + 1e-6f);
      ik = rsqrtf(sk + 1e-6f);
    }
    float beta = x.beta;
    if (XFORM && (p.flags & kFlagBetaLogit)) beta = tv ? sigmoidf_(beta) : 0.f;
    // With the in-kernel gate the decays are formed first (one uniform branch; pad
    // tokens keep g = 0).
    f32x4 gx[XFORM ? 2 * NKB : 1];
    if constexpr (XFORM) {
#pragma unroll
      for (int i = 0; i < 2 * NKB; ++i) gx[i] = widen<BF16IO>(x.g[i]);
      if (gate) {
#pragma unroll
        for (int i = 0; i < 2 * NKB; ++i) {
          const int key = 32 * kb_of(i >> 1) + 16 * (i & 1) + 4 * grp;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = gate_a * (gx[i][e] + sy->dtb[key + e]);
            const float gv = p.lower_bound * __builtin_amdgcn_rcpf(1.f + __expf(-z));
            gx[i][e] = tv ? gv : 0.f;
          }
        }
      }
    }
    bf16x8 ks[NKB], qs[NKB], ke[NKB];
    f32x4 accR = zero, accA = zero;
    f32x2 dpair = {0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      f32x4 vks[2], vqs[2], vki[2], vke[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int i = 2 * kk + hf;
        f32x4 q = widen<BF16IO>(x.q[i]), k = widen<BF16IO>(x.k[i]);
        f32x4 g;
        if constexpr (XFORM) {
          g = gx[i];
          q *= iq;
          k *= ik;
        } else {
          g = widen<BF16IO>(x.g[i]);
        }
        f32x4 e15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float G = g[e];
          G += row_shr<1>(G);
          G += row_shr<2>(G);
          G += row_shr<4>(G);
          G += row_shr<8>(G);
          // Over one chunk G >= -80 (g >= -5): 2^(+-G log2 e) stays a normal FP32 number.
          const float tt = G * kLog2e;
          const float gam = __builtin_amdgcn_exp2f(tt);
          const float igam = __builtin_amdgcn_exp2f(-tt);
          e15[e] = bcast16<15>(gam);
          vks[hf][e] = gam * k[e];
          vqs[hf][e] = gam * q[e];
          vki[hf][e] = igam * k[e];
          vke[hf][e] = e15[e] * vki[hf][e];
        }
        // D_{0:15} pair of this lane: keys 16 (m / 2) + 4 grp + 2 (m % 2) + {0, 1}, i.e.
        // group m / 4, half (m / 2) % 2, elements 2 (m % 2) + {0, 1}.
        if ((m >> 2) == kb_of(kk) && ((m >> 1) & 1) == hf)
          dpair = (m & 1) ? f32x2{e15[2], e15[3]} : f32x2{e15[0], e15[1]};
      }
      ks[kk] = pack8(vks[0], vks[1]);
      qs[kk] = pack8(vqs[0], vqs[1]);
      ke[kk] = pack8(vke[0], vke[1]);
      const bf16x8 ki = pack8(vki[0], vki[1]);
      // lane (grp, m) accumulates R'[m][4 grp + j] = <K_start row m, K_inv row 4 grp + j>
      // and the same with Q_start: row m, column 4 grp + j (over this half's keys).
      accR = mfma32(ki, ks[kk], accR);
      accA = mfma32(ki, qs[kk], accA);
    }
    u32x4 vcur[F::VPL];  // V pieces of chunk j (x is reloaded with chunk j + NPAIR)
#pragma unroll
    for (int i = 0; i < F::VPL; ++i) vcur[i] = x.v[i];
    if (j + STRIDE < nch) load_chunk<BF16IO, W, XFORM>(p, t, j + STRIDE, lane, hh, x);

    // ---- 2. exchange, R, A_qk, Mb = (I + R)^{-1} B, P = A_qk Mb ---------------------
    if constexpr (kPaired) {
      const int b = gen & 1;
      lds_f* mine = &sy->part[pp][b][hh][0][0][0];
      lds_f* theirs = &sy->part[pp][b][hh ^ 1][0][0][0];
      *reinterpret_cast<lds_f4*>(mine + m * kC + 4 * grp) = accR;
      *reinterpret_cast<lds_f4*>(mine + kC * kC + m * kC + 4 * grp) = accA;
      lds_drain();
      if (lane == 0) lds_add(&sy->pair[pp], 1);
      if (!wait_at_least(&sy->abort, &sy->pair[pp], 2 * (gen + 1), p.status)) return;
      // the sum in the same order in both halves: half 0's part first
      const f32x4 oR = *reinterpret_cast<const lds_f4*>(theirs + m * kC + 4 * grp);
      const f32x4 oA = *reinterpret_cast<const lds_f4*>(theirs + kC * kC + m * kC + 4 * grp);
      accR = hh ? oR + accR : accR + oR;
      accA = hh ? oA + accA : accA + oA;
    }
    // R strictly lower, scaled by beta of its row; A_qk lower with the diagonal; row m,
    // columns 4 grp + j.
    f32x4 r, aq;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int col = 4 * grp + jj;
      r[jj] = col < m ? beta * accR[jj] : 0.f;
      aq[jj] = col <= m ? p.scale * accA[jj] : 0.f;
    }
    *reinterpret_cast<lds_f4*>(sR + m * kC + 4 * grp) = r;
    // Mb = (I + R)^{-1} Diag(beta): lane c < 16 solves column c by forward substitution
    // (its token's beta scales it) with the rows of R broadcast from the scratch, and
    // writes it as row c of Mb^T (over the R rows, which it no longer needs: the wave's
    // LDS operations are in order, and every lane's last read of R comes first).
    if (ln < kC) {
      const int c = ln;
      float xs[kC];
#pragma unroll
      for (int i = 0; i < kC; ++i) {
        float acc = i == c ? 1.f : 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          if (4 * q4 < i) {
            const f32x4 rv = *reinterpret_cast<const lds_f4*>(sR + i * kC + 4 * q4);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
              if (4 * q4 + tt < i) acc -= rv[tt] * xs[4 * q4 + tt];
          }
        }
        xs[i] = acc;
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<lds_f4*>(sA + c * kC + 4 * i4) =
            f32x4{xs[4 * i4] * beta, xs[4 * i4 + 1] * beta, xs[4 * i4 + 2] * beta,
                  xs[4 * i4 + 3] * beta};
    }
    // Mb[4 grp + j][m] (column m) and Mb[m][4 grp + j] (row m).
    const f32x4 mbc = *reinterpret_cast<const lds_f4*>(sA + m * kC + 4 * grp);
    f32x4 mbr;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) mbr[jj] = sA[(4 * grp + jj) * kC + m];
    // P row m, columns 4 grp + j: the sum over t of Mb[t][col] A_qk[m][t], lane (grp, m)
    // giving Mb[4 grp + kk][m] and A_qk[m][4 grp + kk] for k step kk of a 16x16x4 FP32
    // product.
    f32x4 pr = zero;
    if (OUT) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        pr = __builtin_amdgcn_mfma_f32_16x16x4f32(mbc[kk], aq[kk], pr, 0, 0, 0);
    }
    // Identity in the 16x16x16 operands' k order: the B operand of lane (grp, m) is
    // I[4 grp + j][m], so A Id = A for any assignment of k to (grp, j).
    i16x4 ident;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) ident[jj] = (4 * grp + jj == m) ? static_cast<short>(0x3F80) : 0;
    const i16x4 bM = pack4(-mbr);  // B[token 4 grp + j][token m] = -Mb[m][4 grp + j]
    const i16x4 bP = pack4(-pr);   // B[token 4 grp + j][token m] = -P[m][4 grp + j]

    // ---- 3. the slot: this half's record pieces as they are formed, then V ----------
    const int s = static_cast<int>(j % F::NSLOT);
    // the slot's previous chunk, j - NSLOT, has been read by all W compute waves
    if (!wait_at_least(&sy->abort, &sy->done[s], W * static_cast<int>(j / F::NSLOT), p.status))
      return;
    lds_u8* slot = ring + s * F::SLOT;
    auto put = [&](int off, u32x4 v) { *reinterpret_cast<lds_v4*>(slot + off + lane * 16) = v; };
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const int kb = kb_of(kk);
      const u32x4 ksw = __builtin_bit_cast(u32x4, ks[kk]);
      const u32x4 kew = __builtin_bit_cast(u32x4, ke[kk]);
      const u32x4 qsw = __builtin_bit_cast(u32x4, qs[kk]);
      i16x4 kn2[2], qt2[2], ke2[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const i16x4 aks = __builtin_bit_cast(i16x4, hf ? u32x2{ksw[2], ksw[3]} : u32x2{ksw[0], ksw[1]});
        const i16x4 ake = __builtin_bit_cast(i16x4, hf ? u32x2{kew[2], kew[3]} : u32x2{kew[0], kew[1]});
        // lane (grp, m): K_start[token 4 grp + j][key 16 b + m] (b = 2 kb + hf), the A
        // operand of Kn^T and Qt^T
        const i16x4 at = pack4(mfma16(aks, ident, zero));
        kn2[hf] = pack4(mfma16(at, bM, zero));  // Kn[m][16 b + 4 grp + j]
        if (OUT) {
          const u32x2 qh = hf ? u32x2{qsw[2], qsw[3]} : u32x2{qsw[0], qsw[1]};
          const f32x4 qinit = p.scale * widen<true>(qh);  // s Q_start[m][16 b + 4 grp + j]
          qt2[hf] = pack4(mfma16(at, bP, qinit));          // Qt[m][16 b + 4 grp + j]
        }
        ke2[hf] = pack4(mfma16(ake, ident, zero));  // K_end[token 4 grp + j][key 16 b + m]
      }
      put(kOffKn + kb * 1024, join(kn2[0], kn2[1]));
      if (OUT) put(kOffQt + kb * 1024, join(qt2[0], qt2[1]));
      put(kOffKeT + kb * 1024, join(ke2[0], ke2[1]));
    }
    if (!kPaired || (m >> 3) == hh)  // the D entries of this wave's keys
      *reinterpret_cast<__attribute__((address_space(3))) f32x2*>(slot + kOffD + lane * 8) = dpair;
    if (hh == 0) put(kOffMbAq, join(pack4(mbr), pack4(aq)));
    if (!t.vzero) {
#pragma unroll
      for (int i = 0; i < F::VPL; ++i) {
        const int pl = lane + 64 * i;
        if (pl < F::VWAVE)
          *reinterpret_cast<lds_v4*>(slot + kRecord + (hh * F::VWAVE + pl) * 16) = vcur[i];
      }
    }
    // ---- 4. publish this half ----------------------------------------------------------
    lds_drain();
    const int whole = 2 * (static_cast<int>(j / F::NSLOT) + 1);  // both halves counted
    if (keep && hh == kHalvesPerWave % 2) {
      // Inspection copy of the record, before the chunk is published (so no reader can
      // free the slot); with pairs by the second half once the first has written.
      if (kPaired && !wait_at_least(&sy->abort, &sy->ready[s], whole - 1, p.status)) return;
      unsigned char* rec =
          p.records + (t.h * p.max_chunks + t.rec_chunk + j) * static_cast<int64_t>(kRecord);
      for (int u = lane; u < kRecord / 16; u += 64)
        *reinterpret_cast<u32x4*>(rec + 16 * u) = *reinterpret_cast<const lds_v4*>(slot + 16 * u);
    }
    if (lane == 0) lds_add(&sy->ready[s], kHalvesPerWave);
  }
}

}  // namespace fused
