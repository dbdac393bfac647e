// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// that api.cpp makes, so that the C-ABI host code can be built with g++ under
// AddressSanitizer / UndefinedBehaviorSanitizer and driven on a machine
// without a GPU.  Nothing here touches the pointers it is given: every
// launcher records its arguments for the harness and reports success.

#include <hip/hip_runtime_api.h>

#include "../../attention_kl_divergence_skl_amd/csrc/skl_internal.h"
#include "host_stubs.h"

namespace stub {
LaunchLog log;
int device_cus = 256;  // compute units hipDeviceGetAttribute reports (0: no device)
}  // namespace stub

extern "C" {
hipError_t hipGetDevice(int* dev) {
  if (stub::device_cus <= 0) return hipErrorNoDevice;
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *value = stub::device_cus;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  ++stub::log.events;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stubbed HIP error"; }
}

namespace skl {

hipError_t launch_forward(const FwdParams& p, int, int, int, bool, bool split, int64_t BH, hipStream_t s,
                          void (*between)(hipStream_t)) {
  ++stub::log.forward;
  stub::log.fwd = p;
  stub::log.fwd_split = split;
  stub::log.BH = BH;
  if (between) between(s);
  return hipSuccess;
}
hipError_t launch_reduce(const ReduceParams& p, hipStream_t) {
  ++stub::log.reduce;
  stub::log.red = p;
  return hipSuccess;
}
hipError_t launch_zero(float*, int64_t count, hipStream_t) {
  ++stub::log.zero;
  stub::log.zero_count = count;
  return hipSuccess;
}
hipError_t launch_backward_fused(const BwdParams& p, int, int, int, bool, bool teacher, int64_t BH, hipStream_t) {
  ++stub::log.fused;
  stub::log.bwd = p;
  stub::log.teacher = teacher;
  stub::log.BH = BH;
  return hipSuccess;
}
hipError_t launch_backward_split(const BwdParams& p, int, int, int, bool, bool teacher, int64_t BH, hipStream_t s,
                                 void (*between)(hipStream_t)) {
  ++stub::log.split;
  stub::log.bwd = p;
  stub::log.teacher = teacher;
  stub::log.BH = BH;
  if (between) between(s);
  return hipSuccess;
}
hipError_t launch_backward_joint(const BwdParams& p, int, int, int, bool, int64_t BH, hipStream_t s,
                                 void (*between)(hipStream_t)) {
  ++stub::log.joint;
  stub::log.bwd = p;
  stub::log.BH = BH;
  if (between) between(s);
  return hipSuccess;
}
hipError_t launch_zero_rows(void* dst, const Strides&, int64_t B, int64_t H, int64_t N, int d, int, hipStream_t) {
  ++stub::log.zero_rows;
  stub::log.zero_rows_dst = dst;
  stub::log.zero_rows_rows = B * H * N;
  stub::log.zero_rows_d = d;
  return hipSuccess;
}
hipError_t launch_convert(const ConvertParams& p, int, hipStream_t) {
  ++stub::log.convert;
  stub::log.conv = p;
  return hipSuccess;
}

}  // namespace skl
