/*
 * A plain-C client of libra.so (include/ra.h): no C++, no Python, no torch.
 *
 *   ring_forward_c check
 *       No GPU work: prints the library version and checks that invalid
 *       arguments are rejected with a status and a message.
 *   ring_forward_c run B H N d P q.bin k.bin v.bin out.bin
 *       Reads bf16 Q, K, V ([B, H, N, d], contiguous, raw 16-bit words) from
 *       files, runs the whole ring (ra_ring_forward, all P query blocks
 *       resident, default scale, internal workspace, default stream) and
 *       writes O the same way.
 *
 * Exit status 0 on success; otherwise a message on stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ra.h"

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

static int check(void) {
  printf("libra %s\n", ra_version());
  const int64_t st[3] = {16 * 1024 * 128, 1024 * 128, 128};
  void* fake = (void*)(uintptr_t)0x10000; /* never dereferenced: the call fails its checks first */
  ra_status_t s = ra_ring_forward(fake, st, fake, st, fake, st, fake, st, RA_DTYPE_BF16, 1, 16, 1024, 128, 0,
                                  NULL, 0, 0.0f, NULL, 0, NULL);
  if (s != RA_E_INVALID_ARG || ra_last_error()[0] == '\0') {
    fprintf(stderr, "P = 0 was not rejected (status %d)\n", (int)s);
    return 1;
  }
  printf("P = 0 rejected: %s\n", ra_last_error());
  s = ra_ring_forward(fake, st, fake, st, fake, st, fake, st, RA_DTYPE_BF16, 1, 16, 1024, 96, 4, NULL, 4, 0.0f, NULL,
                      0, NULL);
  if (s != RA_E_UNSUPPORTED) {
    fprintf(stderr, "d = 96 was not rejected (status %d)\n", (int)s);
    return 1;
  }
  printf("d = 96 rejected: %s\n", ra_last_error());
  return 0;
}

static int read_file(const char* path, void* dst, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return 1;
  }
  const size_t got = fread(dst, 1, bytes, f);
  fclose(f);
  if (got != bytes) {
    fprintf(stderr, "%s: read %zu of %zu bytes\n", path, got, bytes);
    return 1;
  }
  return 0;
}

static int run(int64_t B, int64_t H, int64_t N, int64_t d, int32_t P, const char* qp, const char* kp, const char* vp,
               const char* op) {
  const size_t bytes = (size_t)(B * H * N * d) * 2;
  uint16_t* host = (uint16_t*)malloc(bytes);
  if (!host) return 1;
  void *q = NULL, *k = NULL, *v = NULL, *out = NULL;
  HIP_OK(hipMalloc(&q, bytes));
  HIP_OK(hipMalloc(&k, bytes));
  HIP_OK(hipMalloc(&v, bytes));
  HIP_OK(hipMalloc(&out, bytes));
  const char* ins[3] = {qp, kp, vp};
  void* devs[3] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    if (read_file(ins[i], host, bytes)) return 1;
    HIP_OK(hipMemcpy(devs[i], host, bytes, hipMemcpyHostToDevice));
  }
  const int64_t st[3] = {H * N * d, N * d, d};
  const ra_status_t s =
      ra_ring_forward(q, st, k, st, v, st, out, st, RA_DTYPE_BF16, B, H, N, d, P, NULL, P, 0.0f, NULL, 0, NULL);
  if (s != RA_OK) {
    fprintf(stderr, "ra_ring_forward: status %d: %s\n", (int)s, ra_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(host, out, bytes, hipMemcpyDeviceToHost));
  FILE* f = fopen(op, "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", op);
    return 1;
  }
  fclose(f);
  HIP_OK(hipFree(q));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(out));
  free(host);
  printf("ring_forward_c: B=%lld H=%lld N=%lld d=%lld P=%d done\n", (long long)B, (long long)H, (long long)N,
         (long long)d, (int)P);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "check") == 0) return check();
  if (argc == 11 && strcmp(argv[1], "run") == 0)
    return run(atoll(argv[2]), atoll(argv[3]), atoll(argv[4]), atoll(argv[5]), (int32_t)atoi(argv[6]), argv[7],
               argv[8], argv[9], argv[10]);
  fprintf(stderr, "usage: %s check | run B H N d P q.bin k.bin v.bin out.bin\n", argv[0]);
  return 2;
}
