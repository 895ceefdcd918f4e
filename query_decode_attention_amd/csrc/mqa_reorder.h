// mqa_reorder.h -- launch parameters of the in-place beam reorder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

constexpr int kMaxBeam = 16;

struct ReorderParams {
  char* k;
  char* v;
  int32_t* lens;           // read; permuted in place when lens_out is null
  int32_t* lens_out;       // nullable: the permuted lengths go here instead
  const int32_t* parent;  // beam-local parent of every hypothesis
  int32_t* err_flag;      // nullable
  int b, m_cap, beam;
  int row_bytes;          // G * d_h * element size
};

hipError_t launch_kv_reorder(const ReorderParams& p, hipStream_t s);

}  // namespace mqa
