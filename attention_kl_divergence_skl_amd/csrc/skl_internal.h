// Internal interface between the C-ABI host code (api.cpp) and the kernel
// translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/streamkl.h"

namespace skl {

// Geometry fixed by the kernels.
constexpr int kFwdBQ = 128;  // queries per forward workgroup (4 waves x 32)
constexpr int kFwdBK = 64;   // keys per forward pipeline step
constexpr int kBwdBK = 128;  // keys per backward workgroup (4 waves x 32)
constexpr int kBwdBQ = 32;   // queries per backward step (fused and dK kernels)
constexpr int kDqBK = 64;    // keys per step of the dQ kernel
constexpr int kDkBQ = 64;    // queries per step of the dK kernel
constexpr int kThreads = 256;

struct Strides {
  int64_t b, h, n;
};

struct FwdParams {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  Strides sq1, sk1, sq2, sk2;
  int64_t NQ, NK;
  int32_t H;
  int32_t num_qtiles;   // ceil(NQ / kFwdBQ)
  int32_t splits;       // 1 for the plain forward
  int32_t split_len;    // keys per split (multiple of kFwdBK); unused when splits == 1
  float c1, c2;         // scale_k * log2(e)
  float* kl;            // plain forward outputs [B*H*NQ]
  float* lse1;
  float* lse2;
  float* part;          // split-K partials: [5][B*H][splits][NQ]
};

struct ReduceParams {
  const float* part;
  int64_t rows;         // B*H*NQ
  int64_t NQ;
  int32_t splits;
  float* kl;
  float* lse1;
  float* lse2;
};

struct BwdParams {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  Strides sq1, sk1, sq2, sk2;
  int64_t NQ, NK;
  int32_t H;
  int32_t num_ktiles;   // ceil(NK / kBwdBK)
  float c1, c2;         // scale_k * log2(e)
  float scale_g;        // scale of the optimised side
  const float* lse1;
  const float* lse2;
  const float* kl;      // teacher only
  const float* dkl;
  void* dk;             // gradient of the optimised side's keys (input strides)
  Strides sdk;
  void* dq;             // gradient of the optimised side's queries (split kernels)
  Strides sdq;
  float* ws;            // fp32 dQ accumulator [B*H][NQ][dg] (fused kernel)
  // Joint kernels (both settings at once): dk/dq/scale_g above are the
  // teacher's (Q1, K1) gradients, these the student's (Q2, K2).
  void* dk_s;
  Strides sdk_s;
  void* dq_s;
  Strides sdq_s;
  float scale_s;
  int32_t dq_splits;    // split kernels: key ranges of the dQ kernel (1: write dq directly)
  int32_t dq_split_len; // keys per range (multiple of kDqBK)
  float* dq_part;       // dq_splits > 1: unscaled fp32 partials [dq_splits][B*H][NQ][dg]
};

struct ConvertParams {
  const float* ws;      // [splits][rows][dg] fp32, summed over splits
  int32_t splits;
  int64_t split_stride; // elements between split planes (rows * dg)
  void* dq;
  Strides sdq;
  int64_t NQ;
  int32_t H;
  int32_t dg;
  int64_t rows;         // B*H*NQ
  float scale;
};

// Launchers: return the result of hipGetLastError() after the launch.
// Forward: the main pass, then the fixup pass that recomputes only the
// tiles the main pass marked.  `between` runs after the main pass's launch
// (profiling events).
hipError_t launch_forward(const FwdParams& p, int dtype, int d1, int d2, bool causal, bool split,
                          int64_t BH, hipStream_t s, void (*between)(hipStream_t));
hipError_t launch_reduce(const ReduceParams& p, hipStream_t s);
hipError_t launch_zero(float* ws, int64_t count, hipStream_t s);
// Fused backward: one kernel, dQ through fp32 atomics into p.ws.
hipError_t launch_backward_fused(const BwdParams& p, int dtype, int d1, int d2, bool causal, bool teacher,
                                 int64_t BH, hipStream_t s);
// Split backward: dK kernel then dQ kernel, plain stores, no workspace.
// `between` runs after the first launch (profiling events).
hipError_t launch_backward_split(const BwdParams& p, int dtype, int d1, int d2, bool causal, bool teacher,
                                 int64_t BH, hipStream_t s, void (*between)(hipStream_t));
// Both settings in one pass (joint dK kernel, then joint dQ kernel).
hipError_t launch_backward_joint(const BwdParams& p, int dtype, int d1, int d2, bool causal, int64_t BH,
                                 hipStream_t s, void (*between)(hipStream_t));
hipError_t launch_convert(const ConvertParams& p, int dtype, hipStream_t s);
// Zeros into a strided [B, H, N, d] tensor (16-byte aligned rows).
hipError_t launch_zero_rows(void* dst, const Strides& st, int64_t B, int64_t H, int64_t N, int d, int dtype,
                            hipStream_t s);

// Records a printf-style message as this thread's last error (skl_last_error)
// and returns `status` (api.cpp).
skl_status set_error(skl_status status, const char* fmt, ...);

}  // namespace skl
