/*
 * Drives libstreamkl from plain C, with no Python and no torch: the HIP
 * runtime for device memory, the C ABI for everything else.  Reads a problem
 * from a file, runs the forward, the student and teacher backward calls (split
 * algorithm) and the joint backward call on the null stream, and writes every
 * output to a file for the caller to check.
 *
 *   skl_c_check <in> <out>
 *
 * <in>:  int64 B, H, N_Q, N_K, d1, d2, causal, dtype (0 bf16, 1 fp32), then
 *        float scale1, scale2, then Q1, K1, Q2, K2 as contiguous
 *        [B, H, N, d] arrays of that dtype (bf16 as uint16 bit patterns) and
 *        the upstream gradient dKL as fp32 [B, H, N_Q].
 * <out>: fp32 KL, LSE1, LSE2 [B, H, N_Q], then dQ2, dK2 (student call),
 *        dQ1, dK1 (teacher call), dQ1, dK1, dQ2, dK2 (joint call), each in the
 *        input dtype and layout.
 * Exit status 0 on success; a failing call prints its status and message.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "streamkl.h"

#define CHECK_HIP(x)                                                         \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 2;                                                              \
    }                                                                        \
  } while (0)

#define CHECK_SKL(x)                                                                      \
  do {                                                                                    \
    skl_status s_ = (x);                                                                  \
    if (s_ != SKL_OK) {                                                                   \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, skl_status_string(s_), skl_last_error()); \
      return 3;                                                                           \
    }                                                                                     \
  } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) { return fread(dst, 1, bytes, f) == bytes ? 0 : -1; }

/* A device copy of `bytes` bytes read from f. */
static void* upload(FILE* f, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  void* dev = NULL;
  if (!host || read_all(f, host, bytes) != 0 || hipMalloc(&dev, bytes ? bytes : 1) != hipSuccess ||
      hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    free(host);
    return NULL;
  }
  free(host);
  return dev;
}

/* Appends `bytes` bytes of device memory to f. */
static int download(FILE* f, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  int rc = -1;
  if (host && hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) == hipSuccess &&
      fwrite(host, 1, bytes, f) == bytes)
    rc = 0;
  free(host);
  return rc;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <in> <out>\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int64_t hdr[8];
  float scales[2];
  if (read_all(in, hdr, sizeof hdr) != 0 || read_all(in, scales, sizeof scales) != 0) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int64_t B = hdr[0], H = hdr[1], NQ = hdr[2], NK = hdr[3];
  const int d1 = (int)hdr[4], d2 = (int)hdr[5], causal = (int)hdr[6], dtype = (int)hdr[7];
  if (B < 0 || H < 0 || NQ < 0 || NK < 0 || B * H * (NQ + NK) > ((int64_t)1 << 28)) {
    fprintf(stderr, "problem size out of range for this check\n");
    return 1;
  }
  const size_t esz = dtype == SKL_BF16 ? 2 : 4;

  skl_shape s;
  memset(&s, 0, sizeof s);
  s.B = B;
  s.H = H;
  s.NQ = NQ;
  s.NK = NK;
  s.d1 = d1;
  s.d2 = d2;
  s.dtype = dtype;
  /* Contiguous [B, H, N, d]: strides of the b, h and n axes in elements. */
  const int64_t rows[4] = {NQ, NK, NQ, NK}, dims[4] = {d1, d1, d2, d2};
  int64_t* strides[4] = {s.sq1, s.sk1, s.sq2, s.sk2};
  size_t bytes[4];
  for (int t = 0; t < 4; ++t) {
    strides[t][0] = H * rows[t] * dims[t];
    strides[t][1] = rows[t] * dims[t];
    strides[t][2] = dims[t];
    bytes[t] = (size_t)(B * H * rows[t] * dims[t]) * esz;
  }
  const size_t vec = (size_t)(B * H * NQ) * sizeof(float);

  void* x[4];
  for (int t = 0; t < 4; ++t)
    if (!(x[t] = upload(in, bytes[t]))) {
      fprintf(stderr, "input %d: read or upload failed\n", t);
      return 2;
    }
  float* dkl = (float*)upload(in, vec);
  fclose(in);
  if (!dkl) {
    fprintf(stderr, "dKL: read or upload failed\n");
    return 2;
  }

  float *kl, *lse1, *lse2;
  CHECK_HIP(hipMalloc((void**)&kl, vec ? vec : 1));
  CHECK_HIP(hipMalloc((void**)&lse1, vec ? vec : 1));
  CHECK_HIP(hipMalloc((void**)&lse2, vec ? vec : 1));
  /* Gradients: student call, teacher call, joint call (dQ1, dK1, dQ2, dK2). */
  void* g[8];
  const int of[8] = {2, 3, 0, 1, 0, 1, 2, 3};
  for (int i = 0; i < 8; ++i) CHECK_HIP(hipMalloc(&g[i], bytes[of[i]] ? bytes[of[i]] : 1));

  CHECK_SKL(skl_forward(&s, x[0], x[1], x[2], x[3], scales[0], scales[1], causal, kl, lse1, lse2, NULL));
  CHECK_SKL(skl_backward_student(&s, x[0], x[1], x[2], x[3], scales[0], scales[1], causal, lse1, lse2, dkl, g[0],
                                 g[1], SKL_BWD_SPLIT, NULL, 0, NULL));
  CHECK_SKL(skl_backward_teacher(&s, x[0], x[1], x[2], x[3], scales[0], scales[1], causal, lse1, lse2, kl, dkl,
                                 g[2], g[3], SKL_BWD_SPLIT, NULL, 0, NULL));
  CHECK_SKL(skl_backward_joint(&s, x[0], x[1], x[2], x[3], scales[0], scales[1], causal, lse1, lse2, kl, dkl, g[4],
                               g[5], g[6], g[7], NULL, 0, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    perror(argv[2]);
    return 1;
  }
  int rc = download(out, kl, vec) | download(out, lse1, vec) | download(out, lse2, vec);
  for (int i = 0; i < 8; ++i) rc |= download(out, g[i], bytes[of[i]]);
  if (fclose(out) != 0 || rc != 0) {
    fprintf(stderr, "writing the outputs failed\n");
    return 2;
  }
  for (int t = 0; t < 4; ++t) hipFree(x[t]);
  for (int i = 0; i < 8; ++i) hipFree(g[i]);
  hipFree(dkl);
  hipFree(kl);
  hipFree(lse1);
  hipFree(lse2);
  printf("skl_c_check: libstreamkl %d, B=%lld H=%lld N_Q=%lld N_K=%lld d1=%d d2=%d causal=%d dtype=%d: ok\n",
         skl_version(), (long long)B, (long long)H, (long long)NQ, (long long)NK, d1, d2, causal, dtype);
  return 0;
}
