// mqa_probe.hip -- measurement aid, not part of the attention path: a plain
// streaming read of a device buffer, the practical HBM read rate against
// which the decode's bandwidth is judged (the vendor's 8 TB/s is a peak no
// kernel reaches).  Every 16-byte word is read once with coalesced vector
// loads, four in flight per thread, one 512-thread workgroup per CU (the
// fastest of 1/2/4 workgroups per CU x 4/8/16 loads in flight measured on
// MI355X: 6.3-6.5 TB/s over 128 MiB-2 GiB); the XOR of everything read is stored to
// *sink only when it equals a value no all-zero or all-one buffer produces,
// so the loads cannot be removed and nothing is written in practice.
#include "mqa_device.h"
#include "mqa_internal.h"

namespace mqa {

__global__ __launch_bounds__(512) void read_probe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                         uint32_t* sink) {
  constexpr int kUnroll = 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x5a5aa5a5u) *sink = 1u;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  int dev = 0;
  const int cus = current_device_cus(&dev);
  if (cus <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)cus), dim3(512), 0, s,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace mqa
