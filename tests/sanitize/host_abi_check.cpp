// Drives every entry point of the C ABI through its host code (validation,
// workspace sizing, parameter setup and dispatch) with the launchers and the
// HIP runtime stubbed out (host_stubs.cpp).  Built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by the CPU test suite; a
// failed check, a memory error or undefined behaviour ends it with a
// non-zero status.  Device pointers are fake addresses the stubs never use.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/streamkl.h"
#include "host_stubs.h"

static int g_fail = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
                   skl_last_error());                                 \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }

static const uintptr_t A = 0x100000;
static void* const q1 = P(A);
static void* const k1 = P(A + 0x1000);
static void* const q2 = P(A + 0x2000);
static void* const k2 = P(A + 0x3000);
static float* const o1 = F(A + 0x4000);
static float* const o2 = F(A + 0x5000);
static float* const o3 = F(A + 0x6000);
static float* const o4 = F(A + 0x7000);
static void* const g1 = P(A + 0x8000);
static void* const g2 = P(A + 0x9000);
static void* const g3 = P(A + 0xa000);
static void* const g4 = P(A + 0xb000);
static void* const ws = P(A + 0x10000);

static skl_shape shape(int64_t B = 1, int64_t H = 2, int64_t NQ = 256, int64_t NK = 256, int d1 = 128, int d2 = 128,
                       int dtype = SKL_BF16) {
  skl_shape s;
  std::memset(&s, 0, sizeof s);
  s.B = B;
  s.H = H;
  s.NQ = NQ;
  s.NK = NK;
  s.d1 = d1;
  s.d2 = d2;
  s.dtype = dtype;
  const int64_t dims[4][2] = {{NQ, d1}, {NK, d1}, {NQ, d2}, {NK, d2}};
  int64_t* st[4] = {s.sq1, s.sk1, s.sq2, s.sk2};
  for (int t = 0; t < 4; ++t) {
    st[t][0] = H * dims[t][0] * dims[t][1];
    st[t][1] = dims[t][0] * dims[t][1];
    st[t][2] = dims[t][1];
  }
  return s;
}

static skl_status fwd(const skl_shape& s, float sc1 = 0.1f, float sc2 = 0.1f, int causal = 0) {
  return skl_forward(&s, q1, k1, q2, k2, sc1, sc2, causal, o1, o2, o3, nullptr);
}
static skl_status student(const skl_shape& s, int algo = SKL_BWD_SPLIT, void* w = nullptr, size_t wb = 0,
                          int causal = 0) {
  return skl_backward_student(&s, q1, k1, q2, k2, 0.1f, 0.1f, causal, o1, o2, o4, g1, g2, algo, w, wb, nullptr);
}
static skl_status teacher(const skl_shape& s, int algo = SKL_BWD_SPLIT, void* w = nullptr, size_t wb = 0) {
  return skl_backward_teacher(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, o1, o2, o3, o4, g1, g2, algo, w, wb, nullptr);
}
static skl_status joint(const skl_shape& s, void* w = nullptr, size_t wb = 0) {
  return skl_backward_joint(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, o1, o2, o3, o4, g1, g2, g3, g4, w, wb, nullptr);
}

static void forward_checks() {
  stub::log = {};
  skl_shape s = shape(2, 3, 300, 300, 128, 64);
  CHECK(fwd(s, 0.125f, 0.25f, 1) == SKL_OK);
  CHECK(stub::log.forward == 1 && !stub::log.fwd_split && stub::log.BH == 6);
  CHECK(stub::log.fwd.num_qtiles == 3 && stub::log.fwd.NQ == 300 && stub::log.fwd.H == 3);
  CHECK(std::fabs(stub::log.fwd.c1 - 0.125f * 1.4426950408889634f) < 1e-6f);
  CHECK(std::fabs(stub::log.fwd.c2 - 0.25f * 1.4426950408889634f) < 1e-6f);
  CHECK(stub::log.fwd.kl == o1 && stub::log.fwd.lse1 == o2 && stub::log.fwd.lse2 == o3);

  // Rejections: nothing is launched.
  stub::log = {};
  skl_shape b = shape();
  b.d1 = 96;
  CHECK(fwd(b) == SKL_ERR_UNSUPPORTED);
  b = shape();
  b.dtype = 9;
  CHECK(fwd(b) == SKL_ERR_UNSUPPORTED);
  b = shape();
  b.reserved = 1;
  CHECK(fwd(b) == SKL_ERR_INVALID_ARGUMENT);
  b = shape();
  b.NQ = -1;
  CHECK(fwd(b) == SKL_ERR_INVALID_ARGUMENT);
  b = shape();
  b.sk2[2] = 100;
  CHECK(fwd(b) == SKL_ERR_UNSUPPORTED);
  b = shape();
  b.sq1[1] = -8;
  CHECK(fwd(b) == SKL_ERR_INVALID_ARGUMENT);
  b = shape();
  b.sq2[2] = int64_t(1) << 24;
  CHECK(fwd(b) == SKL_ERR_UNSUPPORTED);
  b = shape(1, 2, int64_t(1) << 30, int64_t(1) << 30);
  CHECK(fwd(b) == SKL_ERR_UNSUPPORTED);
  CHECK(fwd(shape(), 0.f) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(fwd(shape(), std::numeric_limits<float>::quiet_NaN()) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(fwd(shape(), 0.1f, std::numeric_limits<float>::infinity()) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(fwd(shape(1, 2, 300, 200), 0.1f, 0.1f, 1) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(fwd(shape(1, 2, 4, 0)) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(skl_forward(nullptr, q1, k1, q2, k2, 0.1f, 0.1f, 0, o1, o2, o3, nullptr) == SKL_ERR_INVALID_ARGUMENT);
  skl_shape ok = shape();
  CHECK(skl_forward(&ok, P(A + 2), k1, q2, k2, 0.1f, 0.1f, 0, o1, o2, o3, nullptr) == SKL_ERR_UNSUPPORTED);
  CHECK(skl_forward(&ok, q1, nullptr, q2, k2, 0.1f, 0.1f, 0, o1, o2, o3, nullptr) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(skl_forward(&ok, q1, k1, q2, k2, 0.1f, 0.1f, 0, nullptr, o2, o3, nullptr) == SKL_ERR_INVALID_ARGUMENT);
  // 2^20 heads x 16 query tiles exceed the dispatch limit.
  CHECK(fwd(shape(1, int64_t(1) << 20, 2048, 2048)) == SKL_ERR_UNSUPPORTED);
  CHECK(std::strstr(skl_last_error(), "dispatch limit") != nullptr);
  CHECK(stub::log.forward == 0);

  // Empty problems enqueue nothing and need no pointers.
  skl_shape e = shape(0, 2);
  CHECK(skl_forward(&e, nullptr, nullptr, nullptr, nullptr, 0.1f, 0.1f, 0, nullptr, nullptr, nullptr, nullptr) ==
        SKL_OK);
  e = shape(1, 2, 0, 0);
  CHECK(skl_forward(&e, nullptr, nullptr, nullptr, nullptr, 0.1f, 0.1f, 0, nullptr, nullptr, nullptr, nullptr) ==
        SKL_OK);
  CHECK(stub::log.forward == 0);
  CHECK(std::strlen(skl_last_error()) == 0);
}

static void splitk_checks() {
  stub::log = {};
  skl_shape s = shape(1, 2, 256, 16384);
  const size_t need = skl_forward_splitk_workspace_size(&s, 4);
  CHECK(need == size_t(5) * 2 * 4 * 256 * 4);
  CHECK(skl_forward_splitk(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, 4, ws, need, nullptr) == SKL_OK);
  CHECK(stub::log.forward == 1 && stub::log.fwd_split && stub::log.fwd.splits == 4);
  CHECK(stub::log.fwd.split_len == 4096 && stub::log.fwd.part == ws);
  CHECK(skl_reduce(&s, 4, ws, need, o1, o2, o3, nullptr) == SKL_OK);
  CHECK(stub::log.reduce == 1 && stub::log.red.rows == 512 && stub::log.red.splits == 4);
  CHECK(skl_forward_splitk(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, 4, ws, need - 4, nullptr) ==
        SKL_ERR_WORKSPACE_TOO_SMALL);
  CHECK(skl_forward_splitk(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, 0, ws, need, nullptr) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(skl_forward_splitk(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, 70000, ws, ~size_t(0), nullptr) ==
        SKL_ERR_INVALID_ARGUMENT);
  CHECK(skl_reduce(&s, 4, ws, need - 1, o1, o2, o3, nullptr) == SKL_ERR_WORKSPACE_TOO_SMALL);
  CHECK(skl_reduce(&s, 4, nullptr, need, o1, o2, o3, nullptr) == SKL_ERR_INVALID_ARGUMENT);
  // 2^16 heads x 1 query tile x 256 splits exceed the dispatch limit.
  skl_shape big = shape(1, int64_t(1) << 16, 128, 65536);
  const size_t nb = skl_forward_splitk_workspace_size(&big, 256);
  CHECK(skl_forward_splitk(&big, q1, k1, q2, k2, 0.1f, 0.1f, 0, 256, ws, nb, nullptr) == SKL_ERR_UNSUPPORTED);
  CHECK(stub::log.forward == 1 && stub::log.reduce == 1);
  CHECK(skl_recommended_splits(&s, 0, 256) >= 2);
  skl_shape full = shape(1, 32, 65536, 65536);
  CHECK(skl_recommended_splits(&full, 1, 256) == 1);
  CHECK(skl_recommended_splits(nullptr, 1, 256) == 1);
}

static void backward_checks() {
  // Enough query tiles: split backward, no workspace, no convert.
  stub::device_cus = 256;
  stub::log = {};
  skl_shape s = shape(1, 32, 4096, 4096);
  CHECK(skl_backward_workspace_size(&s, 0, SKL_BWD_SPLIT) == 0);
  CHECK(student(s) == SKL_OK);
  CHECK(stub::log.split == 1 && !stub::log.teacher && stub::log.convert == 0 && stub::log.bwd.dq_splits == 1);
  CHECK(stub::log.bwd.dq == g1 && stub::log.bwd.dk == g2 && stub::log.bwd.num_ktiles == 32);
  CHECK(teacher(s) == SKL_OK);
  CHECK(stub::log.split == 2 && stub::log.teacher && stub::log.bwd.kl == o3);

  // Few query tiles: the dQ keys are split when the workspace is given.
  stub::log = {};
  skl_shape f = shape(1, 2, 256, 65536, 128, 64);
  const size_t wn = skl_backward_workspace_size(&f, 0, SKL_BWD_SPLIT);
  CHECK(wn > 0 && wn % (size_t(2) * 256 * 64 * 4) == 0);
  CHECK(student(f, SKL_BWD_SPLIT, ws, wn) == SKL_OK);
  CHECK(stub::log.split == 1 && stub::log.convert == 1 && stub::log.bwd.dq_splits > 1);
  CHECK(stub::log.conv.splits == stub::log.bwd.dq_splits && stub::log.conv.dg == 64);
  CHECK(student(f) == SKL_OK);  // no workspace: dQ over all keys
  CHECK(stub::log.split == 2 && stub::log.convert == 1 && stub::log.bwd.dq_splits == 1);
  CHECK(student(f, SKL_BWD_SPLIT, P(A + 0x10008), wn) == SKL_ERR_UNSUPPORTED);  // misaligned ws

  // No device: no key ranges.
  stub::device_cus = 0;
  CHECK(skl_backward_workspace_size(&f, 0, SKL_BWD_SPLIT) == 0);
  stub::device_cus = 256;

  // Fused algorithm: clear, kernel, convert.
  stub::log = {};
  const size_t wf = skl_backward_workspace_size(&s, 1, SKL_BWD_FUSED_ATOMIC);
  CHECK(wf == size_t(32) * 4096 * 128 * 4);
  CHECK(teacher(s, SKL_BWD_FUSED_ATOMIC, ws, wf) == SKL_OK);
  CHECK(stub::log.zero == 1 && stub::log.fused == 1 && stub::log.convert == 1);
  CHECK(stub::log.zero_count == int64_t(32) * 4096 * 128);
  CHECK(teacher(s, SKL_BWD_FUSED_ATOMIC, ws, wf - 16) == SKL_ERR_WORKSPACE_TOO_SMALL);
  CHECK(teacher(s, SKL_BWD_FUSED_ATOMIC, nullptr, wf) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(student(s, 7) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(skl_backward_teacher(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, o1, o2, nullptr, o4, g1, g2, 0, nullptr, 0,
                             nullptr) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(skl_backward_student(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, o1, o2, o4, P(A + 0x8008), g2, 0, nullptr, 0,
                             nullptr) == SKL_ERR_UNSUPPORTED);

  // Gradient layouts that repeat elements.
  skl_shape bc = shape(2);
  bc.sk2[1] = 0;  // K2 broadcast over heads
  CHECK(student(bc) == SKL_ERR_UNSUPPORTED);
  CHECK(joint(bc) == SKL_ERR_UNSUPPORTED);
  skl_shape ov = shape();
  ov.sq1[2] = 64;  // Q1 rows overlap (head dim 128)
  CHECK(teacher(ov) == SKL_ERR_UNSUPPORTED);
  skl_shape bnhd = shape(2, 4, 256, 256);
  for (int64_t* st : {bnhd.sq1, bnhd.sk1, bnhd.sq2, bnhd.sk2}) {
    st[0] = 256 * 4 * 128;
    st[1] = 128;
    st[2] = 4 * 128;
  }
  CHECK(student(bnhd) == SKL_OK);
  CHECK(teacher(bnhd) == SKL_OK);
  skl_shape one = shape(1, 1, 256, 256);
  one.sk2[0] = 0;
  one.sk2[1] = 0;  // size-1 axes: any stride
  CHECK(student(one) == SKL_OK);

  // Dispatch limit (key tiles / query tiles).
  CHECK(student(shape(1, int64_t(1) << 20, 2048, 2048)) == SKL_ERR_UNSUPPORTED);
  CHECK(joint(shape(1, int64_t(1) << 20, 2048, 2048)) == SKL_ERR_UNSUPPORTED);

  // Joint: one pass, or the two split settings when the workspace is given
  // and the query tiles are few.
  stub::log = {};
  CHECK(joint(s) == SKL_OK);
  CHECK(stub::log.joint == 1 && stub::log.bwd.dk == g2 && stub::log.bwd.dk_s == g4);
  const size_t wj = skl_backward_joint_workspace_size(&f);
  CHECK(wj == skl_backward_workspace_size(&f, 0, 0) + skl_backward_workspace_size(&f, 1, 0));
  CHECK(joint(f, ws, wj) == SKL_OK);
  CHECK(stub::log.joint == 1 && stub::log.split == 2 && stub::log.convert == 2);
  CHECK(skl_backward_joint(&s, q1, k1, q2, k2, 0.1f, 0.1f, 0, o1, o2, nullptr, o4, g1, g2, g3, g4, nullptr, 0,
                           nullptr) == SKL_ERR_INVALID_ARGUMENT);

  // No query rows but keys: every backward call writes zeros into its key
  // gradients (and needs them), nothing else; no rows at all: nothing.
  const skl_shape nq = shape(2, 3, 0, 77, 128, 64);
  stub::log = {};
  CHECK(student(nq) == SKL_OK);
  CHECK(stub::log.zero_rows == 1 && stub::log.zero_rows_dst == g2 && stub::log.zero_rows_rows == 2 * 3 * 77 &&
        stub::log.zero_rows_d == 64 && stub::log.split == 0);
  CHECK(teacher(nq, SKL_BWD_FUSED_ATOMIC) == SKL_OK);
  CHECK(stub::log.zero_rows == 2 && stub::log.zero_rows_dst == g2 && stub::log.zero_rows_d == 128 &&
        stub::log.fused == 0 && stub::log.zero == 0);
  CHECK(joint(nq) == SKL_OK);
  CHECK(stub::log.zero_rows == 4 && stub::log.zero_rows_dst == g4 && stub::log.joint == 0);
  CHECK(skl_backward_student(&nq, nullptr, nullptr, nullptr, nullptr, 0.1f, 0.1f, 0, nullptr, nullptr, nullptr,
                             nullptr, nullptr, SKL_BWD_SPLIT, nullptr, 0, nullptr) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(student(nq, 7) == SKL_ERR_INVALID_ARGUMENT);  // unknown algorithm, also for an empty problem
  stub::log = {};
  CHECK(student(shape(0, 3, 0, 77)) == SKL_OK && joint(shape(2, 3, 0, 0)) == SKL_OK);
  CHECK(stub::log.zero_rows == 0);
}

static void misc_checks() {
  hipEvent_t ev[4] = {reinterpret_cast<hipEvent_t>(A), reinterpret_cast<hipEvent_t>(A + 1),
                      reinterpret_cast<hipEvent_t>(A + 2), reinterpret_cast<hipEvent_t>(A + 3)};
  CHECK(skl_set_kernel_events(ev, 5) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(skl_set_kernel_events(nullptr, 2) == SKL_ERR_INVALID_ARGUMENT);
  CHECK(skl_set_kernel_events(ev, 4) == SKL_OK);
  stub::log = {};
  skl_shape s = shape(1, 32, 4096, 4096);
  CHECK(fwd(s) == SKL_OK);
  CHECK(stub::log.events == 2);
  CHECK(student(s) == SKL_OK);
  CHECK(stub::log.events == 5);
  CHECK(skl_set_kernel_events(nullptr, 0) == SKL_OK);
  CHECK(fwd(s) == SKL_OK);
  CHECK(stub::log.events == 5);
  CHECK(std::strcmp(skl_status_string(SKL_ERR_HIP), "SKL_ERR_HIP") == 0);
  CHECK(std::strcmp(skl_status_string(static_cast<skl_status>(42)), "SKL_UNKNOWN_STATUS") == 0);
  CHECK(skl_version() >= 100);
  CHECK(skl_forward_splitk_workspace_size(nullptr, 2) == 0);
  CHECK(skl_backward_workspace_size(nullptr, 0, 0) == 0);
}

int main() {
  forward_checks();
  splitk_checks();
  backward_checks();
  misc_checks();
  if (g_fail) {
    std::fprintf(stderr, "%d host ABI check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
