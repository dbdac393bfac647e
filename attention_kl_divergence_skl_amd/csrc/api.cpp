// C-ABI entry points of libstreamkl: argument validation, workspace sizing and
// kernel dispatch.  Every check runs on the host before anything is enqueued.

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/streamkl.h"
#include "skl_internal.h"

namespace {

thread_local std::string g_last_error;
// Profiling events (skl_set_kernel_events): slot 0 before the first main
// kernel of a call, slot k after its k-th main kernel.
constexpr int kMaxEvents = 4;
thread_local hipEvent_t g_ev[kMaxEvents] = {};
thread_local int g_nev = 0;

hipError_t mark(int k, hipStream_t s) {
  if (k < g_nev && g_ev[k]) return hipEventRecord(g_ev[k], s);
  return hipSuccess;
}
void mark1(hipStream_t s) { (void)mark(1, s); }

// Run one main kernel launch between event slots 0 and 1.
template <typename F>
hipError_t timed(hipStream_t stream, F&& launch) {
  hipError_t e = mark(0, stream);
  if (e != hipSuccess) return e;
  e = launch();
  if (e == hipSuccess) e = mark(1, stream);
  return e;
}

skl_status fail(skl_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

skl_status ok() {
  g_last_error.clear();
  return SKL_OK;
}

skl_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SKL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t esize(int dtype) { return dtype == SKL_BF16 ? 2 : 4; }

// Shape checks shared by every call.  `need_nk` is false for skl_reduce.
skl_status check_shape(const skl_shape* s, bool need_nk) {
  if (!s) return fail(SKL_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->B < 0 || s->H < 0 || s->NQ < 0 || s->NK < 0)
    return fail(SKL_ERR_INVALID_ARGUMENT, "negative size (B=%lld H=%lld NQ=%lld NK=%lld)", (long long)s->B,
                (long long)s->H, (long long)s->NQ, (long long)s->NK);
  if (s->reserved != 0) return fail(SKL_ERR_INVALID_ARGUMENT, "skl_shape.reserved must be 0");
  if (s->dtype != SKL_BF16 && s->dtype != SKL_F32) return fail(SKL_ERR_UNSUPPORTED, "dtype %d", s->dtype);
  if (!need_nk) return ok();
  if ((s->d1 != 64 && s->d1 != 128) || (s->d2 != 64 && s->d2 != 128))
    return fail(SKL_ERR_UNSUPPORTED, "head dims d1=%d d2=%d (supported: 64, 128)", s->d1, s->d2);
  if (s->NK == 0 && s->NQ > 0 && s->B > 0 && s->H > 0)
    return fail(SKL_ERR_INVALID_ARGUMENT, "N_K = 0 with N_Q > 0: empty softmax");
  // Index arithmetic inside the kernels: grid sizes fit in 32 bits, and row
  // indices (plus a tile) in 31.
  if (s->NQ >= (int64_t(1) << 30) || s->NK >= (int64_t(1) << 30) || s->B * s->H > (int64_t(1) << 31))
    return fail(SKL_ERR_UNSUPPORTED, "sizes too large");
  const int64_t mult = s->dtype == SKL_BF16 ? 8 : 4;
  const int64_t* all[4] = {s->sq1, s->sk1, s->sq2, s->sk2};
  for (int t = 0; t < 4; ++t)
    for (int a = 0; a < 3; ++a) {
      if (all[t][a] < 0) return fail(SKL_ERR_INVALID_ARGUMENT, "negative stride");
      if (all[t][a] % mult != 0)
        return fail(SKL_ERR_UNSUPPORTED, "stride %lld not a multiple of %lld elements", (long long)all[t][a],
                    (long long)mult);
    }
  // Tile loads address a 64-row span with 32-bit offsets.
  const int64_t esz = s->dtype == SKL_BF16 ? 2 : 4;
  for (int t = 0; t < 4; ++t)
    if (all[t][2] * esz * 64 >= (int64_t(1) << 31))
      return fail(SKL_ERR_UNSUPPORTED, "row stride %lld elements too large", (long long)all[t][2]);
  return ok();
}

bool empty(const skl_shape* s) { return s->B == 0 || s->H == 0 || s->NQ == 0; }

// An empty problem whose key gradients still have rows: no query sees any
// key, so a backward call writes zeros into dK.
bool keys_without_queries(const skl_shape* s) { return s->B > 0 && s->H > 0 && s->NQ == 0 && s->NK > 0; }

skl_status check_ptr(const void* p, const char* name, bool align16 = true) {
  if (!p) return fail(SKL_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (align16 && (reinterpret_cast<uintptr_t>(p) & 15u) != 0)
    return fail(SKL_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
  return ok();
}

// A 1-D dispatch holds at most 2^32 - 1 work-items, i.e. this many
// 256-thread workgroups.  Every launch with one workgroup per tile checks its
// grid against it on the host (the fill, convert and reduce kernels loop over
// their elements and cap their grids).
constexpr int64_t kMaxWorkgroups = ((int64_t(1) << 32) - 1) / skl::kThreads;

skl_status check_grid(int64_t groups, const char* what) {
  if (groups > kMaxWorkgroups)
    return fail(SKL_ERR_UNSUPPORTED, "%s: %lld workgroups exceed the dispatch limit of %lld", what,
                (long long)groups, (long long)kMaxWorkgroups);
  return ok();
}

// True when the [B, H, N, d] view with (b, h, n) element strides `st` and a
// contiguous d axis gives every element its own address: taking the axes of
// size > 1 in order of increasing stride, each stride reaches past everything
// the axes inside it span.  (Sufficient, not necessary: exotic interleaved
// layouts that happen to be one-to-one are rejected too.)
bool disjoint_layout(const int64_t st[3], int64_t B, int64_t H, int64_t N, int64_t d) {
  int64_t size[3] = {B, H, N}, stride[3] = {st[0], st[1], st[2]};
  int idx[3] = {0, 1, 2};
  std::sort(idx, idx + 3, [&](int a, int b) { return stride[a] < stride[b]; });
  int64_t span = d;  // offsets [0, span) are covered by the axes inside
  for (int k = 0; k < 3; ++k) {
    const int a = idx[k];
    if (size[a] <= 1) continue;
    if (stride[a] < span) return false;
    span += stride[a] * (size[a] - 1);
  }
  return true;
}

// Gradients are written with the strides of the corresponding input, so an
// input whose layout repeats elements (a stride of 0, e.g. one K broadcast
// over heads, or overlapping rows) cannot receive its gradient in place.
skl_status check_grad_layout(const int64_t st[3], int64_t B, int64_t H, int64_t N, int64_t d, const char* name) {
  if (!disjoint_layout(st, B, H, N, d))
    return fail(SKL_ERR_UNSUPPORTED,
                "%s: the gradient takes this input's strides, which map several elements to one address "
                "(a zero or overlapping stride); pass a copy with a one-to-one layout",
                name);
  return ok();
}

skl_status check_scales(float s1, float s2, int causal, const skl_shape* s) {
  if (!std::isfinite(s1) || !std::isfinite(s2) || !(s1 > 0.f) || !(s2 > 0.f))
    return fail(SKL_ERR_INVALID_ARGUMENT, "scales must be finite and > 0 (got %g, %g)", (double)s1, (double)s2);
  if (causal && s->NQ > s->NK)
    return fail(SKL_ERR_INVALID_ARGUMENT, "causal needs N_Q <= N_K (got %lld > %lld)", (long long)s->NQ,
                (long long)s->NK);
  return ok();
}

#define SKL_TRY(expr)                 \
  do {                                \
    skl_status st_ = (expr);          \
    if (st_ != SKL_OK) return st_;    \
  } while (0)

skl_status check_inputs(const skl_shape* s, const void* q1, const void* k1, const void* q2, const void* k2,
                        float scale1, float scale2, int causal) {
  SKL_TRY(check_shape(s, true));
  SKL_TRY(check_scales(scale1, scale2, causal, s));
  if (empty(s)) return ok();
  SKL_TRY(check_ptr(q1, "q1"));
  SKL_TRY(check_ptr(k1, "k1"));
  SKL_TRY(check_ptr(q2, "q2"));
  SKL_TRY(check_ptr(k2, "k2"));
  return ok();
}

skl::Strides strides(const int64_t* a) { return skl::Strides{a[0], a[1], a[2]}; }

skl::FwdParams fwd_params(const skl_shape* s, const void* q1, const void* k1, const void* q2, const void* k2,
                          float scale1, float scale2) {
  skl::FwdParams p{};
  p.q1 = q1;
  p.k1 = k1;
  p.q2 = q2;
  p.k2 = k2;
  p.sq1 = strides(s->sq1);
  p.sk1 = strides(s->sk1);
  p.sq2 = strides(s->sq2);
  p.sk2 = strides(s->sk2);
  p.NQ = s->NQ;
  p.NK = s->NK;
  p.H = (int32_t)s->H;
  p.num_qtiles = (int32_t)cdiv(s->NQ, skl::kFwdBQ);
  p.splits = 1;
  p.split_len = 0;
  p.c1 = (float)(scale1 * 1.4426950408889634);
  p.c2 = (float)(scale2 * 1.4426950408889634);
  return p;
}

int64_t split_len_for(int64_t nk, int splits) {
  return cdiv(cdiv(nk, splits), skl::kFwdBK) * skl::kFwdBK;
}

}  // namespace

namespace skl {

skl_status set_error(skl_status status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

}  // namespace skl

extern "C" {

int skl_version(void) { return 100; }

skl_status skl_set_kernel_events(hipEvent_t* events, int count) {
  if (count < 0 || count > kMaxEvents || (count > 0 && !events))
    return fail(SKL_ERR_INVALID_ARGUMENT, "events: count must be 0..%d with a non-NULL array", kMaxEvents);
  for (int i = 0; i < kMaxEvents; ++i) g_ev[i] = i < count ? events[i] : nullptr;
  g_nev = count;
  return ok();
}

const char* skl_last_error(void) { return g_last_error.c_str(); }

const char* skl_status_string(skl_status st) {
  switch (st) {
    case SKL_OK: return "SKL_OK";
    case SKL_ERR_INVALID_ARGUMENT: return "SKL_ERR_INVALID_ARGUMENT";
    case SKL_ERR_UNSUPPORTED: return "SKL_ERR_UNSUPPORTED";
    case SKL_ERR_WORKSPACE_TOO_SMALL: return "SKL_ERR_WORKSPACE_TOO_SMALL";
    case SKL_ERR_HIP: return "SKL_ERR_HIP";
  }
  return "SKL_UNKNOWN_STATUS";
}

skl_status skl_forward(const skl_shape* s, const void* q1, const void* k1, const void* q2, const void* k2,
                       float scale1, float scale2, int causal, float* kl, float* lse1, float* lse2,
                       hipStream_t stream) {
  SKL_TRY(check_inputs(s, q1, k1, q2, k2, scale1, scale2, causal));
  if (empty(s)) return ok();
  SKL_TRY(check_ptr(kl, "kl", false));
  SKL_TRY(check_ptr(lse1, "lse1", false));
  SKL_TRY(check_ptr(lse2, "lse2", false));
  SKL_TRY(check_grid(s->B * s->H * cdiv(s->NQ, skl::kFwdBQ), "skl_forward"));
  skl::FwdParams p = fwd_params(s, q1, k1, q2, k2, scale1, scale2);
  p.kl = kl;
  p.lse1 = lse1;
  p.lse2 = lse2;
  hipError_t e = mark(0, stream);
  if (e == hipSuccess)
    e = skl::launch_forward(p, s->dtype, s->d1, s->d2, causal != 0, false, s->B * s->H, stream, mark1);
  return from_hip(e, "skl_forward launch");
}

size_t skl_forward_splitk_workspace_size(const skl_shape* s, int num_splits) {
  if (!s || num_splits < 1 || s->B < 0 || s->H < 0 || s->NQ < 0) return 0;
  return (size_t)5 * (size_t)s->B * (size_t)s->H * (size_t)num_splits * (size_t)s->NQ * sizeof(float);
}

skl_status skl_forward_splitk(const skl_shape* s, const void* q1, const void* k1, const void* q2, const void* k2,
                              float scale1, float scale2, int causal, int num_splits, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  SKL_TRY(check_inputs(s, q1, k1, q2, k2, scale1, scale2, causal));
  if (num_splits < 1 || num_splits > 65536) return fail(SKL_ERR_INVALID_ARGUMENT, "num_splits=%d", num_splits);
  if (empty(s)) return ok();
  SKL_TRY(check_ptr(ws, "ws"));
  const size_t need = skl_forward_splitk_workspace_size(s, num_splits);
  if (ws_bytes < need)
    return fail(SKL_ERR_WORKSPACE_TOO_SMALL, "split-K workspace %zu < %zu bytes", ws_bytes, need);
  SKL_TRY(check_grid(s->B * s->H * cdiv(s->NQ, skl::kFwdBQ) * num_splits, "skl_forward_splitk"));
  skl::FwdParams p = fwd_params(s, q1, k1, q2, k2, scale1, scale2);
  p.splits = num_splits;
  p.split_len = (int32_t)split_len_for(s->NK, num_splits);
  p.part = static_cast<float*>(ws);
  hipError_t e = mark(0, stream);
  if (e == hipSuccess)
    e = skl::launch_forward(p, s->dtype, s->d1, s->d2, causal != 0, true, s->B * s->H, stream, mark1);
  return from_hip(e, "skl_forward_splitk launch");
}

skl_status skl_reduce(const skl_shape* s, int num_splits, const void* ws, size_t ws_bytes, float* kl, float* lse1,
                      float* lse2, hipStream_t stream) {
  SKL_TRY(check_shape(s, false));
  if (num_splits < 1 || num_splits > 65536) return fail(SKL_ERR_INVALID_ARGUMENT, "num_splits=%d", num_splits);
  if (empty(s)) return ok();
  SKL_TRY(check_ptr(ws, "ws"));
  SKL_TRY(check_ptr(kl, "kl", false));
  SKL_TRY(check_ptr(lse1, "lse1", false));
  SKL_TRY(check_ptr(lse2, "lse2", false));
  const size_t need = skl_forward_splitk_workspace_size(s, num_splits);
  if (ws_bytes < need)
    return fail(SKL_ERR_WORKSPACE_TOO_SMALL, "split-K workspace %zu < %zu bytes", ws_bytes, need);
  skl::ReduceParams p{};
  p.part = static_cast<const float*>(ws);
  p.rows = s->B * s->H * s->NQ;
  p.NQ = s->NQ;
  p.splits = num_splits;
  p.kl = kl;
  p.lse1 = lse1;
  p.lse2 = lse2;
  return from_hip(skl::launch_reduce(p, stream), "skl_reduce launch");
}

}  // extern "C"

namespace {

// Compute units of the current device (cached per device id).
int current_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Key ranges of the split backward's dQ kernel.  Its workgroups own 128
// queries each; when those alone cannot fill the device (two resident
// workgroups per CU) the keys are cut into ranges of at least 8 tiles.
int64_t dq_splits_for(const skl_shape* s) {
  const int cus = current_cus();
  if (cus <= 0) return 1;
  const int64_t target = 2 * (int64_t)cus;
  const int64_t tiles = s->B * s->H * cdiv(s->NQ, 128);
  if (tiles <= 0 || tiles >= target) return 1;
  int64_t splits = cdiv(target, tiles);
  splits = std::min<int64_t>(splits, cdiv(s->NK, 8 * skl::kDqBK));
  splits = std::min<int64_t>(splits, 64);
  return std::max<int64_t>(splits, 1);
}

int64_t dq_split_len(const skl_shape* s, int64_t splits) {
  return cdiv(cdiv(s->NK, splits), skl::kDqBK) * skl::kDqBK;
}

}  // namespace

extern "C" {

size_t skl_backward_workspace_size(const skl_shape* s, int teacher, int algo) {
  if (!s || s->B <= 0 || s->H <= 0 || s->NQ <= 0 || s->NK <= 0) return 0;
  const int d = teacher ? s->d1 : s->d2;
  if (d <= 0) return 0;
  const size_t plane = (size_t)s->B * (size_t)s->H * (size_t)s->NQ * (size_t)d * sizeof(float);
  if (algo == SKL_BWD_FUSED_ATOMIC) return plane;
  if (algo != SKL_BWD_SPLIT) return 0;
  const int64_t splits = dq_splits_for(s);
  return splits > 1 ? (size_t)splits * plane : 0;
}

static skl_status backward_common(const skl_shape* s, const void* q1, const void* k1, const void* q2,
                                  const void* k2, float scale1, float scale2, int causal, const float* lse1,
                                  const float* lse2, const float* kl, const float* dkl, void* dq, void* dk,
                                  int algo, void* ws, size_t ws_bytes, bool teacher, hipStream_t stream) {
  SKL_TRY(check_inputs(s, q1, k1, q2, k2, scale1, scale2, causal));
  if (algo != SKL_BWD_SPLIT && algo != SKL_BWD_FUSED_ATOMIC)
    return fail(SKL_ERR_INVALID_ARGUMENT, "unknown backward algorithm %d", algo);
  const int64_t* sqg = teacher ? s->sq1 : s->sq2;
  const int64_t* skg = teacher ? s->sk1 : s->sk2;
  const int64_t dgd = teacher ? s->d1 : s->d2;
  if (empty(s)) {
    if (!keys_without_queries(s)) return ok();
    SKL_TRY(check_ptr(dk, teacher ? "dk1" : "dk2"));
    SKL_TRY(check_grad_layout(skg, s->B, s->H, s->NK, dgd, teacher ? "k1" : "k2"));
    return from_hip(skl::launch_zero_rows(dk, strides(skg), s->B, s->H, s->NK, (int)dgd, s->dtype, stream),
                    "dK zero launch");
  }
  SKL_TRY(check_ptr(lse1, "lse1", false));
  SKL_TRY(check_ptr(lse2, "lse2", false));
  if (teacher) SKL_TRY(check_ptr(kl, "kl", false));
  SKL_TRY(check_ptr(dkl, "dkl", false));
  SKL_TRY(check_ptr(dq, teacher ? "dq1" : "dq2"));
  SKL_TRY(check_ptr(dk, teacher ? "dk1" : "dk2"));
  const bool fused = algo == SKL_BWD_FUSED_ATOMIC;
  SKL_TRY(check_grad_layout(sqg, s->B, s->H, s->NQ, dgd, teacher ? "q1" : "q2"));
  SKL_TRY(check_grad_layout(skg, s->B, s->H, s->NK, dgd, teacher ? "k1" : "k2"));
  SKL_TRY(check_grid(s->B * s->H * cdiv(s->NK, skl::kBwdBK), "backward (key tiles)"));
  if (fused) {
    SKL_TRY(check_ptr(ws, "ws"));
    const size_t need = skl_backward_workspace_size(s, teacher ? 1 : 0, algo);
    if (ws_bytes < need)
      return fail(SKL_ERR_WORKSPACE_TOO_SMALL, "backward workspace %zu < %zu bytes", ws_bytes, need);
  }
  const int64_t BH = s->B * s->H;
  const int dg = teacher ? s->d1 : s->d2;
  const float scale_g = teacher ? scale1 : scale2;

  skl::BwdParams p{};
  p.q1 = q1;
  p.k1 = k1;
  p.q2 = q2;
  p.k2 = k2;
  p.sq1 = strides(s->sq1);
  p.sk1 = strides(s->sk1);
  p.sq2 = strides(s->sq2);
  p.sk2 = strides(s->sk2);
  p.NQ = s->NQ;
  p.NK = s->NK;
  p.H = (int32_t)s->H;
  p.num_ktiles = (int32_t)cdiv(s->NK, skl::kBwdBK);
  p.c1 = (float)(scale1 * 1.4426950408889634);
  p.c2 = (float)(scale2 * 1.4426950408889634);
  p.scale_g = scale_g;
  p.lse1 = lse1;
  p.lse2 = lse2;
  p.kl = kl;
  p.dkl = dkl;
  p.dk = dk;
  p.sdk = teacher ? p.sk1 : p.sk2;
  p.dq = dq;
  p.sdq = teacher ? p.sq1 : p.sq2;
  p.ws = static_cast<float*>(ws);

  skl::ConvertParams c{};
  c.dq = dq;
  c.sdq = teacher ? p.sq1 : p.sq2;
  c.NQ = s->NQ;
  c.H = (int32_t)s->H;
  c.dg = dg;
  c.rows = BH * s->NQ;
  c.scale = scale_g;
  c.splits = 1;
  c.split_stride = c.rows * dg;

  if (!fused) {
    // With the workspace skl_backward_workspace_size() asks for, the dQ kernel
    // splits its keys into ranges whose fp32 partials convert_kernel sums;
    // without it (or when the query tiles fill the device) dQ is written
    // directly.
    const int64_t splits = dq_splits_for(s);
    const size_t need = skl_backward_workspace_size(s, teacher ? 1 : 0, algo);
    const bool split_dq = splits > 1 && ws != nullptr && ws_bytes >= need;
    SKL_TRY(check_grid(BH * cdiv(s->NQ, 128) * (split_dq ? splits : 1), "backward (query tiles)"));
    if (split_dq) {
      if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return fail(SKL_ERR_UNSUPPORTED, "ws must be 16-byte aligned");
      p.dq_splits = (int32_t)splits;
      p.dq_split_len = (int32_t)dq_split_len(s, splits);
      p.dq_part = static_cast<float*>(ws);
    } else {
      p.dq_splits = 1;
    }
    hipError_t e = mark(0, stream);
    if (e == hipSuccess)
      e = skl::launch_backward_split(p, s->dtype, s->d1, s->d2, causal != 0, teacher, BH, stream, mark1);
    if (e == hipSuccess) e = mark(2, stream);
    if (e == hipSuccess && split_dq) {
      c.ws = p.dq_part;
      c.splits = (int32_t)splits;
      e = skl::launch_convert(c, s->dtype, stream);
      if (e == hipSuccess) e = mark(3, stream);
    }
    return from_hip(e, "backward launch");
  }

  hipError_t e = skl::launch_zero(static_cast<float*>(ws), BH * s->NQ * dg, stream);
  if (e != hipSuccess) return from_hip(e, "workspace clear launch");
  e = timed(stream, [&] {
    return skl::launch_backward_fused(p, s->dtype, s->d1, s->d2, causal != 0, teacher, BH, stream);
  });
  if (e != hipSuccess) return from_hip(e, "backward launch");

  c.ws = static_cast<const float*>(ws);
  return from_hip(skl::launch_convert(c, s->dtype, stream), "dq convert launch");
}

skl_status skl_backward_student(const skl_shape* s, const void* q1, const void* k1, const void* q2, const void* k2,
                                float scale1, float scale2, int causal, const float* lse1, const float* lse2,
                                const float* dkl, void* dq2, void* dk2, int algo, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return backward_common(s, q1, k1, q2, k2, scale1, scale2, causal, lse1, lse2, nullptr, dkl, dq2, dk2, algo, ws,
                         ws_bytes, false, stream);
}

skl_status skl_backward_teacher(const skl_shape* s, const void* q1, const void* k1, const void* q2, const void* k2,
                                float scale1, float scale2, int causal, const float* lse1, const float* lse2,
                                const float* kl, const float* dkl, void* dq1, void* dk1, int algo, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  return backward_common(s, q1, k1, q2, k2, scale1, scale2, causal, lse1, lse2, kl, dkl, dq1, dk1, algo, ws,
                         ws_bytes, true, stream);
}

size_t skl_backward_joint_workspace_size(const skl_shape* s) {
  return skl_backward_workspace_size(s, 0, SKL_BWD_SPLIT) + skl_backward_workspace_size(s, 1, SKL_BWD_SPLIT);
}

skl_status skl_backward_joint(const skl_shape* s, const void* q1, const void* k1, const void* q2, const void* k2,
                              float scale1, float scale2, int causal, const float* lse1, const float* lse2,
                              const float* kl, const float* dkl, void* dq1, void* dk1, void* dq2, void* dk2,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  SKL_TRY(check_inputs(s, q1, k1, q2, k2, scale1, scale2, causal));
  if (empty(s)) {
    if (!keys_without_queries(s)) return ok();
    SKL_TRY(check_ptr(dk1, "dk1"));
    SKL_TRY(check_ptr(dk2, "dk2"));
    SKL_TRY(check_grad_layout(s->sk1, s->B, s->H, s->NK, s->d1, "k1"));
    SKL_TRY(check_grad_layout(s->sk2, s->B, s->H, s->NK, s->d2, "k2"));
    hipError_t e = skl::launch_zero_rows(dk1, strides(s->sk1), s->B, s->H, s->NK, s->d1, s->dtype, stream);
    if (e == hipSuccess) e = skl::launch_zero_rows(dk2, strides(s->sk2), s->B, s->H, s->NK, s->d2, s->dtype, stream);
    return from_hip(e, "dK zero launch");
  }
  SKL_TRY(check_ptr(lse1, "lse1", false));
  SKL_TRY(check_ptr(lse2, "lse2", false));
  SKL_TRY(check_ptr(kl, "kl", false));
  SKL_TRY(check_ptr(dkl, "dkl", false));
  SKL_TRY(check_ptr(dq1, "dq1"));
  SKL_TRY(check_ptr(dk1, "dk1"));
  SKL_TRY(check_ptr(dq2, "dq2"));
  SKL_TRY(check_ptr(dk2, "dk2"));
  SKL_TRY(check_grad_layout(s->sq1, s->B, s->H, s->NQ, s->d1, "q1"));
  SKL_TRY(check_grad_layout(s->sk1, s->B, s->H, s->NK, s->d1, "k1"));
  SKL_TRY(check_grad_layout(s->sq2, s->B, s->H, s->NQ, s->d2, "q2"));
  SKL_TRY(check_grad_layout(s->sk2, s->B, s->H, s->NK, s->d2, "k2"));

  const size_t need_s = skl_backward_workspace_size(s, 0, SKL_BWD_SPLIT);
  const size_t need_t = skl_backward_workspace_size(s, 1, SKL_BWD_SPLIT);
  if (need_s + need_t > 0 && ws != nullptr && ws_bytes >= need_s + need_t) {
    // Few query tiles and the workspace to split the keys of dQ: the two
    // settings one after the other, each with its dQ over key ranges.
    skl_status st = backward_common(s, q1, k1, q2, k2, scale1, scale2, causal, lse1, lse2, nullptr, dkl, dq2, dk2,
                                    SKL_BWD_SPLIT, ws, need_s, false, stream);
    if (st != SKL_OK) return st;
    return backward_common(s, q1, k1, q2, k2, scale1, scale2, causal, lse1, lse2, kl, dkl, dq1, dk1, SKL_BWD_SPLIT,
                           static_cast<char*>(ws) + need_s, need_t, true, stream);
  }

  const int64_t BH = s->B * s->H;
  SKL_TRY(check_grid(BH * cdiv(s->NK, skl::kBwdBK), "joint backward (key tiles)"));
  SKL_TRY(check_grid(BH * cdiv(s->NQ, 128), "joint backward (query tiles)"));
  skl::BwdParams p{};
  p.q1 = q1;
  p.k1 = k1;
  p.q2 = q2;
  p.k2 = k2;
  p.sq1 = strides(s->sq1);
  p.sk1 = strides(s->sk1);
  p.sq2 = strides(s->sq2);
  p.sk2 = strides(s->sk2);
  p.NQ = s->NQ;
  p.NK = s->NK;
  p.H = (int32_t)s->H;
  p.num_ktiles = (int32_t)cdiv(s->NK, skl::kBwdBK);
  p.c1 = (float)(scale1 * 1.4426950408889634);
  p.c2 = (float)(scale2 * 1.4426950408889634);
  p.lse1 = lse1;
  p.lse2 = lse2;
  p.kl = kl;
  p.dkl = dkl;
  p.dk = dk1;
  p.sdk = p.sk1;
  p.dq = dq1;
  p.sdq = p.sq1;
  p.scale_g = scale1;
  p.dk_s = dk2;
  p.sdk_s = p.sk2;
  p.dq_s = dq2;
  p.sdq_s = p.sq2;
  p.scale_s = scale2;
  p.dq_splits = 1;
  hipError_t e = mark(0, stream);
  if (e == hipSuccess) e = skl::launch_backward_joint(p, s->dtype, s->d1, s->d2, causal != 0, BH, stream, mark1);
  if (e == hipSuccess) e = mark(2, stream);
  return from_hip(e, "joint backward launch");
}

int skl_recommended_splits(const skl_shape* s, int causal, int num_cus) {
  if (!s || s->B <= 0 || s->H <= 0 || s->NQ <= 0 || s->NK <= 0 || num_cus <= 0) return 1;
  // Two resident forward workgroups per CU; aim for at least two waves of them.
  const int64_t target = 4 * (int64_t)num_cus;
  const int64_t tiles = s->B * s->H * cdiv(s->NQ, skl::kFwdBQ);
  if (tiles >= target) return 1;
  // Each split keeps at least 4 key tiles of work (for causal, of the longest rows).
  const int64_t max_by_keys = cdiv(s->NK, 4 * skl::kFwdBK);
  int64_t splits = cdiv(target, tiles);
  if (splits > max_by_keys) splits = max_by_keys;
  if (splits > 64) splits = 64;
  (void)causal;
  return (int)(splits < 1 ? 1 : splits);
}

}  // extern "C"
