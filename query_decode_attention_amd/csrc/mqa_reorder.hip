// mqa_reorder.hip -- in-place beam reorder of the K/V cache.
//
// Beam decoding (the study notes' section 6.2 beam-4 measurements) keeps
// `beam` hypotheses per source sequence as `beam` consecutive cache rows.
// Before a step every hypothesis i continues hypothesis src(i) = group base +
// parent[i] of its own group and takes over its cached positions
// [0, L(src(i))) and its length; positions past that keep their contents.
//
// The permutation only mixes rows at one position across the beams of one
// group.  So one thread owns one (group, position, 16-byte chunk) for ALL the
// beam rows of its group: it loads every source chunk that some moved row
// needs, then stores the moved rows.  No other thread touches those bytes,
// which makes the update in place safe with no LDS and no barrier, and no
// second cache is needed.  A row whose parent is itself is neither read nor
// written, so a step where most beams keep their parent moves little.
// Consecutive lanes take consecutive chunks of consecutive positions: every
// load and store instruction of a wave covers whole rows.
//
// In place, lens is rewritten by a second, one-workgroup kernel afterwards
// (every block of the first kernel reads the old lengths).  With a separate
// output array the first block of each group writes the group's permuted
// lengths there, and there is no second launch.
#include "mqa_device.h"
#include "mqa_reorder.h"

namespace mqa {

__device__ __forceinline__ int clamp_len(int raw, int m_cap) {
  return raw < 0 ? 0 : (raw > m_cap ? m_cap : raw);
}

// blockIdx.y (+ gridDim.y * k): group; blockIdx.x: block of positions.
// MB >= beam bounds the per-thread register arrays.
template <int MB>
__global__ __launch_bounds__(256) void reorder_rows_kernel(ReorderParams p) {
  const int cpr = p.row_bytes >> 4;  // 16-byte chunks per position row
  const int groups = p.b / p.beam;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int pos = (int)(e / cpr), c = (int)(e % cpr);
  const size_t seq = (size_t)p.m_cap * p.row_bytes;
  const size_t off = (size_t)pos * p.row_bytes + (size_t)c * 16;
  for (int grp = blockIdx.y; grp < groups; grp += gridDim.y) {
    const int base = grp * p.beam;
    // The group's parents and lengths, loaded together (one round trip
    // before the copy's loads, not a parent load and then a length load).
    int par[MB], lg[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      par[i] = i < p.beam ? p.parent[base + i] : i;
      lg[i] = i < p.beam ? p.lens[base + i] : 0;
    }
    // Which rows move, where from, and how many positions (uniform).
    int src[MB], len[MB];
    int span = 0;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      src[i] = i;
      len[i] = 0;
      if (i < p.beam) {
        if (par[i] >= 0 && par[i] < p.beam) {
          src[i] = par[i];
          int L = lg[0];
#pragma unroll
          for (int k = 1; k < MB; ++k)
            if (par[i] == k) L = lg[k];  // par[i] is uniform: a scalar choice
          if (par[i] != i) len[i] = clamp_len(L, p.m_cap);
        } else if (blockIdx.x == 0 && threadIdx.x == 0 && p.err_flag) {
          *p.err_flag = 1;
        }
      }
      src[i] = __builtin_amdgcn_readfirstlane(src[i]);
      len[i] = __builtin_amdgcn_readfirstlane(len[i]);
      span = len[i] > span ? len[i] : span;
    }
    if (p.lens_out && blockIdx.x == 0 && (int)threadIdx.x < p.beam) {
      const int i = base + (int)threadIdx.x;
      const int pr = p.parent[i];
      p.lens_out[i] = (pr >= 0 && pr < p.beam) ? p.lens[base + pr] : p.lens[i];
    }
    if (pos >= span) continue;
    // Every source chunk, K and V, is loaded before any moved row is stored:
    // in place is safe, and the K and V loads are in flight together.
    char* at[2] = {p.k + (size_t)base * seq + off, p.v + (size_t)base * seq + off};
    u32x4 x[2][MB];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int s = 0; s < MB; ++s) {
        bool need = false;
#pragma unroll
        for (int i = 0; i < MB; ++i) need |= (src[i] == s && src[i] != i && pos < len[i]);
        x[half][s] = need ? *reinterpret_cast<const u32x4*>(at[half] + (size_t)s * seq)
                          : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (src[i] == i || pos >= len[i]) continue;
        u32x4 v = x[half][0];
#pragma unroll
        for (int s = 1; s < MB; ++s)
          if (src[i] == s) v = x[half][s];  // src[i] is uniform: a scalar choice
        *reinterpret_cast<u32x4*>(at[half] + (size_t)i * seq) = v;
      }
  }
}

// lens[i] = lens[src(i)] for every hypothesis with a valid parent.  One
// workgroup; hypotheses go in chunks of whole groups, each chunk read
// completely before any of it is written.
__global__ __launch_bounds__(256) void reorder_lens_kernel(ReorderParams p) {
  const int chunk = (256 / p.beam) * p.beam;
  for (int c0 = 0; c0 < p.b; c0 += chunk) {
    const int i = c0 + (int)threadIdx.x;
    int v = 0;
    bool write = false;
    if ((int)threadIdx.x < chunk && i < p.b) {
      const int par = p.parent[i];
      if (par >= 0 && par < p.beam) {
        v = p.lens[(i / p.beam) * p.beam + par];
        write = true;
      }
    }
    __syncthreads();
    if (write) p.lens[i] = v;
    __syncthreads();
  }
}

hipError_t launch_kv_reorder(const ReorderParams& p, hipStream_t s) {
  const int groups = p.b / p.beam;
  const int64_t chunks = (int64_t)p.m_cap * (p.row_bytes >> 4);
  const unsigned gx = (unsigned)((chunks + 255) / 256);
  const unsigned gy = (unsigned)(groups < 65535 ? groups : 65535);
  if (p.beam <= 4)
    hipLaunchKernelGGL(reorder_rows_kernel<4>, dim3(gx, gy), dim3(256), 0, s, p);
  else if (p.beam <= 8)
    hipLaunchKernelGGL(reorder_rows_kernel<8>, dim3(gx, gy), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(reorder_rows_kernel<kMaxBeam>, dim3(gx, gy), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.lens_out) return e;
  hipLaunchKernelGGL(reorder_lens_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mqa
