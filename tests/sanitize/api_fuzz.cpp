// Host-side fuzz driver for the C ABI's argument handling (kda_api.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host pass: thousands of
// argument sets, valid and invalid (null, misaligned and overlapping pointers, extreme
// sizes, unknown dtypes and flags), go through kda_prefill_workspace_bytes,
// kda_prefill_check, kda_prefill_plan and kda_prefill. The device launches are replaced
// by stubs that fail (no GPU is touched); pointers are never dereferenced by the host
// code, only compared. Any sanitizer report ends the run with a non-zero status.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "kda.h"
#include "kda_internal.h"

namespace kda {
hipError_t launch_plan(const Params&, int32_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prepare(const Params&, bool, hipStream_t) { return hipErrorInvalidValue; }
int recurrence_loader_waves(int w) { return w < 4 ? 2 : 4; }
hipError_t launch_recurrence(const Params&, int64_t, bool, bool, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_fused_recurrence(const Params&, int64_t, bool, bool, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_combine(const Params&, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_scan_output(const Params&, int64_t, bool, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_carry_out(const Params&, int64_t, bool, bool, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_decode(const Params&, bool, bool, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace kda

namespace {

std::mt19937_64 rng(12345);

int64_t pick(std::initializer_list<int64_t> v) {
  return *(v.begin() + static_cast<size_t>(rng() % v.size()));
}

bool g_sane = false;  // this argument set: valid pointers only

// A fake, never dereferenced device address: regions 1 TiB apart, 256-byte aligned,
// optionally misaligned or null.
void* fake(int i) {
  if (g_sane) return reinterpret_cast<void*>(uintptr_t(i + 1) << 40);
  switch (rng() % 16) {
    case 0: return nullptr;
    case 1: return reinterpret_cast<void*>((uintptr_t(i + 1) << 40) + 8);
    case 2: return reinterpret_cast<void*>(uintptr_t(1) << 40);  // shared: overlaps
    default: return reinterpret_cast<void*>(uintptr_t(i + 1) << 40);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  int ok = 0, rejected = 0;
  for (int it = 0; it < iters; ++it) {
    kda_prefill_args a;
    std::memset(&a, 0, sizeof a);
    g_sane = rng() % 2 == 0;  // half the sets keep every pointer valid
    const bool varlen = rng() % 3 == 0;
    a.D = rng() % 50 ? KDA_HEAD_DIM : pick({0, 64, 256, -1});
    a.B = varlen ? pick({1, 1, 1, 2}) : pick({1, 2, 3, 16, 256, 0, -1, int64_t(1) << 40, INT64_MAX});
    a.T = pick({0, 1, 4, 8, 15, 16, 17, 100, 256, 8192, 65536, -1, int64_t(1) << 35, INT64_MAX});
    a.H = pick({1, 2, 6, 12, 24, 96, 65535, 65536, 0, -3, INT64_MAX});
    a.N = varlen ? pick({1, 2, 8, 300, 0, -1, int64_t(1) << 40, INT64_MAX})
                 : (rng() % 10 ? a.B : pick({0, 5, INT64_MAX}));
    a.q = fake(0); a.k = fake(1); a.v = fake(2); a.g = fake(3); a.beta = fake(4);
    a.o = fake(5);
    a.state_in = rng() % 2 ? fake(6) : nullptr;
    a.state_out = rng() % 4 == 0 ? const_cast<void*>(a.state_in) : (rng() % 2 ? fake(7) : nullptr);
    a.workspace = fake(8);
    a.workspace_bytes = static_cast<size_t>(pick({0, 256, 1 << 20, int64_t(1) << 40, INT64_MAX}));
    a.cu_seqlens = varlen ? static_cast<const int64_t*>(fake(9)) : nullptr;
    a.io_dtype = static_cast<int32_t>(rng() % 20 ? rng() % 2 : pick({2, -1}));
    a.state_dtype = static_cast<int32_t>(rng() % 20 ? rng() % 2 : pick({7}));
    a.scale = static_cast<float>(pick({0, 1, -1})) * 0.088f;
    a.flags = static_cast<uint32_t>(rng() % 16) | (rng() % 40 == 0 ? 0x100u : 0u);
    if (a.flags & KDA_FLAG_GATE_IN_KERNEL) {
      a.A_log = rng() % 8 ? static_cast<const float*>(fake(10)) : nullptr;
      a.dt_bias = static_cast<const float*>(fake(11));
      a.lower_bound = static_cast<float>(pick({-5, -1, 0, 3}));
    }
    a.rows_per_workgroup = static_cast<int32_t>(pick({0, 16, 32, 64, 128, 8, -16}));
    a.segment_chunks = static_cast<int32_t>(pick({0, 0, -1, 1, 2, 47, 1 << 25, INT32_MIN}));
    if (rng() % 4 == 0) {
      a.checkpoint_every = pick({16, 1024, 17, -16, int64_t(1) << 40});
      a.checkpoint_rows = pick({0, 1, 100, -1});
      a.state_checkpoints = fake(12);
      a.checkpoint_cu_starts = static_cast<const int64_t*>(fake(13));
    }
    if (rng() % 5 == 0) {
      a.ssm_state_indices = static_cast<const int32_t*>(fake(14));
      a.state_pool_slots = pick({1, 4, 0, INT64_MAX});
      a.state_slot_pitch = pick({0, 8, a.H > 0 && a.H < 65536 ? a.H * 16384 : 0, INT64_MAX});
    }
    if (rng() % 6 == 0) a.seq_order = static_cast<const int32_t*>(fake(15));
    a.fuse_prepare = static_cast<int32_t>(pick({0, 0, 1, -1}));

    if (g_sane) {  // sizes, dtypes and flags in range too
      a.D = KDA_HEAD_DIM;
      a.B = varlen ? 1 : pick({1, 2, 3, 16, 256});
      a.T = pick({0, 1, 4, 8, 15, 16, 17, 100, 256, 8192});
      a.H = pick({1, 2, 6, 12, 24, 96});
      a.N = varlen ? pick({1, 2, 8, 300}) : a.B;
      a.io_dtype = static_cast<int32_t>(rng() % 2);
      a.state_dtype = static_cast<int32_t>(rng() % 2);
      a.flags &= 0xfu;
      if (a.flags & KDA_FLAG_GATE_IN_KERNEL) {
        a.A_log = static_cast<const float*>(fake(10));
        a.lower_bound = -5.0f;
      }
      if (a.checkpoint_every) {
        a.checkpoint_every = pick({16, 1024});
        a.checkpoint_rows = pick({0, 1, 100});
      }
      if (a.ssm_state_indices) {
        a.state_pool_slots = pick({1, 4, 1000});
        a.state_slot_pitch = pick({0, a.H * 16384 + 8});
      }
      if (a.segment_chunks > (1 << 24) || a.segment_chunks == INT32_MIN) a.segment_chunks = 0;
      if (a.rows_per_workgroup < 0 || a.rows_per_workgroup == 8) a.rows_per_workgroup = 0;
      if (a.scale < 0) a.scale = 0.f;
    }
    size_t bytes = 0;
    const kda_status s0 = kda_prefill_workspace_bytes(&a, &bytes);
    if (s0 == KDA_OK && rng() % 2) a.workspace_bytes = bytes;  // often exactly enough
    kda_plan_info info;
    (void)kda_prefill_plan(&a, static_cast<int32_t>(pick({0, 80, 256, 304})), &info);
    const kda_status s1 = kda_prefill_check(&a);
    if (s1 == KDA_OK) {
      ++ok;
      (void)kda_prefill(&a, nullptr);  // stub launches: reports a HIP error, no GPU work
      kda_prefill_args b = a;
      b.workspace = nullptr;
      b.workspace_bytes = 0;
      (void)kda_prefill_no_alloc(&b, nullptr);
    } else {
      ++rejected;
    }
    (void)kda_status_string(s1);
    (void)kda_last_error();
  }
  std::printf("fuzz: %d argument sets accepted, %d rejected\n", ok, rejected);
  return ok > 0 && rejected > 0 ? 0 : 2;
}
