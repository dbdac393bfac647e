// Launch log shared by the host stubs and the sanitizer harness.
#pragma once

#include "../../attention_kl_divergence_skl_amd/csrc/skl_internal.h"

namespace stub {

struct LaunchLog {
  int forward = 0, reduce = 0, zero = 0, fused = 0, split = 0, joint = 0, convert = 0, events = 0, zero_rows = 0;
  void* zero_rows_dst = nullptr;  // last zero_rows launch: tensor, rows, head dim
  int64_t zero_rows_rows = 0;
  int zero_rows_d = 0;
  skl::FwdParams fwd{};
  bool fwd_split = false;
  skl::ReduceParams red{};
  skl::BwdParams bwd{};
  bool teacher = false;
  skl::ConvertParams conv{};
  int64_t BH = 0;
  int64_t zero_count = 0;
};

extern LaunchLog log;
extern int device_cus;

}  // namespace stub
