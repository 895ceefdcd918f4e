// mqa_attend.h -- launch parameters of attention over a fixed memory
// (non-causal, optional additive mask).
#pragma once

#include "mqa_internal.h"

namespace mqa {

struct AttendParams {
  PrefillParams base;  // Q, K, V, O, b, n (queries), h, G, dh, dtype, scale; no cache
  int m;               // memory positions
  const float* mask;   // nullable: mask[b*msb + head*msh + t*msn + j], j contiguous
  int64_t msb, msh, msn;
};

hipError_t launch_attend(const AttendParams& p, hipStream_t s);

}  // namespace mqa
