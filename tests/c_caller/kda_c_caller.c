/* A C client of the library: no Python and no PyTorch, only the HIP runtime and
 * include/kda.h. Reads q, k, v, g (BF16 [1, T, H, 128]), beta (BF16 [1, T, H]) and
 * state_in (BF16 [1, H, 128, 128]) as raw little-endian files from DIR, sizes and
 * allocates the workspace, runs kda_prefill on a stream of its own, and writes o and
 * state_out back to DIR. Exit status 0 on success; on a library error it prints the
 * status and kda_last_error() and exits with 1.
 *
 * usage: kda_c_caller DIR T H
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

#define CHECK_HIP(x)                                                           \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      exit(2);                                                                 \
    }                                                                          \
  } while (0)

static void *read_file(const char *dir, const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) { perror(path); exit(2); }
  void *buf = malloc(bytes);
  if (!buf || fread(buf, 1, bytes, f) != bytes) { fprintf(stderr, "short read: %s\n", path); exit(2); }
  fclose(f);
  return buf;
}

static void write_file(const char *dir, const char *name, const void *buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) { perror(path); exit(2); }
  fclose(f);
}

static void *to_device(const void *host, size_t bytes) {
  void *d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes));
  CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char **argv) {
  if (argc != 4) {
    fprintf(stderr, "usage: %s DIR T H\n", argv[0]);
    return 2;
  }
  const char *dir = argv[1];
  const int64_t T = atoll(argv[2]), H = atoll(argv[3]);
  if (kda_abi_version() != KDA_ABI_VERSION) {
    fprintf(stderr, "library ABI %d, header %d\n", kda_abi_version(), KDA_ABI_VERSION);
    return 2;
  }
  const size_t tensor = (size_t)T * H * KDA_HEAD_DIM * 2, beta_b = (size_t)T * H * 2;
  const size_t state_b = (size_t)H * KDA_HEAD_DIM * KDA_HEAD_DIM * 2;

  kda_prefill_args a;
  memset(&a, 0, sizeof a);
  a.q = to_device(read_file(dir, "q.bin", tensor), tensor);
  a.k = to_device(read_file(dir, "k.bin", tensor), tensor);
  a.v = to_device(read_file(dir, "v.bin", tensor), tensor);
  a.g = to_device(read_file(dir, "g.bin", tensor), tensor);
  a.beta = to_device(read_file(dir, "beta.bin", beta_b), beta_b);
  a.state_in = to_device(read_file(dir, "state_in.bin", state_b), state_b);
  void *o = NULL, *state_out = NULL;
  CHECK_HIP(hipMalloc(&o, tensor));
  CHECK_HIP(hipMalloc(&state_out, state_b));
  a.o = o;
  a.state_out = state_out;
  a.B = 1;
  a.T = T;
  a.H = H;
  a.D = KDA_HEAD_DIM;
  a.N = 1;
  a.io_dtype = KDA_BF16;
  a.state_dtype = KDA_BF16;

  size_t ws_bytes = 0;
  kda_status st = kda_prefill_workspace_bytes(&a, &ws_bytes);
  if (st != KDA_OK) {
    fprintf(stderr, "workspace query: %s: %s\n", kda_status_string(st), kda_last_error());
    return 1;
  }
  void *ws = NULL;
  if (ws_bytes) CHECK_HIP(hipMalloc(&ws, ws_bytes));
  a.workspace = ws;
  a.workspace_bytes = ws_bytes;

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  st = kda_prefill(&a, stream);
  if (st != KDA_OK) {
    fprintf(stderr, "kda_prefill: %s: %s\n", kda_status_string(st), kda_last_error());
    return 1;
  }
  CHECK_HIP(hipStreamSynchronize(stream));

  void *ho = malloc(tensor), *hs = malloc(state_b);
  CHECK_HIP(hipMemcpy(ho, o, tensor, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hs, state_out, state_b, hipMemcpyDeviceToHost));
  write_file(dir, "o.bin", ho, tensor);
  write_file(dir, "state_out.bin", hs, state_b);
  printf("kda_c_caller: T=%lld H=%lld workspace %zu bytes: ok\n", (long long)T, (long long)H,
         ws_bytes);
  return 0;
}
