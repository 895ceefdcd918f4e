// mqa_prefill.hip -- gfx950 batched attention of n queries per sequence:
//   causal prefill:  O[b,t,i,:] = softmax_{j<=t}(scale * Q[b,t,i,:] . K[b,j,g(i),:]) V[b,j,g(i),:]
//   (study notes section 1: O = softmax(QK^T/sqrt(d_h) + M) V, M = -inf above
//   the diagonal), and
//   attention over a fixed memory of m positions with an optional additive
//   mask, no causal structure (encoder-decoder attention; paper review
//   section 2.3 batched form, weights = softmax(logits + mask)):
//                    O[b,t,i,:] = softmax_{j<m}(scale * Q[b,t,i,:] . K[b,j,g(i),:] + mask[b,i,t,j]) V[b,j,g(i),:]
//
// Columns.  A wave owns 32 query columns = rpw consecutive rows x hgp head
// slots of one group (hgp = h/G rounded up to a power of two), so with MQA
// (h/G = 32) one wave is one row with all its heads, and every column of a
// row shares the causal limit.  Each column keeps its own online softmax; the
// causal mask is a per-column limit on the key position.
//
// Workgroup.  NW waves cover NW*rpw consecutive rows of one (sequence, group)
// and walk the key tiles [0, last row] once.  Per tile, the K rows and the V
// rows (already transposed into the PV operand layout by an exact selection
// MFMA) are staged in LDS once and read by all NW waves; LDS is double
// buffered so the next tile's global loads overlap this tile's MFMAs.  Row
// blocks are launched last-row-first so the longest causal rows start early.
#include "mqa_device.h"
#include "mqa_internal.h"
#include "mqa_attend.h"

namespace mqa {

struct PrefillArgs {
  const char* Q;
  const char* K;
  const char* V;
  char* O;
  const float* mask;        // non-causal only; nullable
  int64_t msb, msh, msn;    // mask element strides over (b, head, query row)
  int b, n, m, h, G, hg, hgp, rpw, nrb;  // m: key/value positions (= n when causal)
  float scale_log2;
};

// FOLD: the softmax takes its max over the raw scores and folds the scale
// into one FMA per score (only for scale > 0 and no mask; chosen at launch).
// MASK (non-causal only): kMaskNone, kMaskKeys (one value per key: the
// head and query strides are 0, as for key padding) or kMaskFull.
constexpr int kMaskNone = 0, kMaskKeys = 1, kMaskFull = 2;
template <typename T, int DH, int NW, bool CAUSAL, bool FOLD, int MASK>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillArgs a) {
  using S = TileShape<T, DH>;
  constexpr int NQ = S::NQ, ND = S::ND, VTC = S::VTC;
  static_assert(NW >= ND, "a wave per d block transposes V");
  constexpr int KPW = (NQ + NW - 1) / NW;     // K chunks per wave
  constexpr int VPW = NQ / ND;                // V chunks per d block
  __shared__ u32x4 s_k[2][NQ][64];
  __shared__ u32x4 s_vt[2][ND][VTC][64];
  __shared__ f32x4 s_kb[2][kTileRows / 4];  // per-key mask of the tile (key padding)

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;

  const int rb = a.nrb - 1 - (int)(blockIdx.x % a.nrb);
  const int bg = blockIdx.x / a.nrb;
  const int bi = bg / a.G, g = bg % a.G;
  const int rows_per_block = NW * a.rpw;
  const int r_begin = rb * rows_per_block;
  if (r_begin >= a.n) return;
  const int r_end = min(a.n, r_begin + rows_per_block);
  const int ntiles = CAUSAL ? (r_end - 1) / kTileRows + 1 : (a.m + kTileRows - 1) / kTileRows;

  const int w_row0 = r_begin + wave * a.rpw;
  const int w_last = min(a.n - 1, w_row0 + a.rpw - 1);
  const int w_tiles = (w_row0 < a.n) ? (CAUSAL ? w_last / kTileRows + 1 : ntiles) : 0;
  const int crow = w_row0 + col / a.hgp;
  const int chead = col % a.hgp;
  const bool col_ok = crow < a.n && chead < a.hg;

  u32x4 qr[NQ];
  if (col_ok) {
    const char* qp = a.Q + (((size_t)bi * a.n + crow) * a.h + (size_t)g * a.hg + chead) * DH * sizeof(T);
#pragma unroll
    for (int c = 0; c < NQ; ++c) qr[c] = *reinterpret_cast<const u32x4*>(qp + (2 * c + half) * 16);
  } else {
#pragma unroll
    for (int c = 0; c < NQ; ++c) qr[c] = u32x4{0u, 0u, 0u, 0u};
  }

  SelOps<T> sel;
  sel.init(col, half);
  const size_t rs = (size_t)a.G * DH * sizeof(T);
  const size_t seq_off = ((size_t)bi * a.m * a.G + (size_t)g) * DH * sizeof(T);
  const char* kseq = a.K + seq_off;
  const char* vseq = a.V + seq_off;

  // Every wave stages K chunks wave, wave + NW, ...; waves below ND also
  // transpose d block `wave` of V into the PV operand layout.
  const bool v_wave = wave < ND;
  // A key-padding mask (one value per key) travels with the tile: the last
  // wave loads the tile's 32 values with its chunks and stages them in LDS.
  const bool kb_wave = MASK == kMaskKeys && wave == NW - 1;
  const float* kb_row = kb_wave ? a.mask + (int64_t)bi * a.msb : nullptr;
  struct Chunks {
    u32x4 k[KPW];
    u32x4 v[VPW];
    float kb;
  };
  auto issue = [&](int tile, Chunks& ld) {
    const int pos = tile * kTileRows + col;
    const bool valid = pos < a.m;
    const char* kp = kseq + (size_t)pos * rs;
    const char* vp = vseq + (size_t)pos * rs;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int c = wave + i * NW;
      ld.k[i] = u32x4{0u, 0u, 0u, 0u};
      if (c < NQ && valid) ld.k[i] = *reinterpret_cast<const u32x4*>(kp + (2 * c + half) * 16);
    }
    if (v_wave) {
#pragma unroll
      for (int i = 0; i < VPW; ++i) {
        const int c = wave * VPW + i;
        ld.v[i] = u32x4{0u, 0u, 0u, 0u};
        if (valid) ld.v[i] = *reinterpret_cast<const u32x4*>(vp + (2 * c + half) * 16);
      }
    }
    if (kb_wave) ld.kb = valid ? kb_row[pos] * 1.4426950408889634f : 0.f;  // log2 units
  };
  auto commit = [&](int buf, const Chunks& ld) {
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int c = wave + i * NW;
      if (c < NQ) s_k[buf][c][lane] = ld.k[i];
    }
    if (v_wave) {
      u32x4 ops[VTC];
      transpose_block<T, VPW>(ld.v, 0, sel, ops);
#pragma unroll
      for (int k = 0; k < VTC; ++k) s_vt[buf][wave][k][lane] = ops[k];
    }
    if (kb_wave && half == 0) reinterpret_cast<float*>(s_kb[buf])[col] = ld.kb;
  };

  // additive mask row of this lane's column (non-causal only)
  const float* mrow = nullptr;
  if (MASK == kMaskFull && col_ok)
    mrow = a.mask + (int64_t)bi * a.msb + (int64_t)(g * a.hg + chead) * a.msh + (int64_t)crow * a.msn;
  constexpr float kLog2e = 1.4426950408889634f;

  WaveState<ND> st;
  st.reset();
  auto compute = [&](int it, int buf) {
    // a general mask's values are fetched before the score product so that
    // its latency overlaps the MFMAs
    float mk[16];
    if constexpr (MASK == kMaskFull) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = it * kTileRows + d_row(r, half);
        mk[r] = (mrow && j < a.m) ? mrow[j] : 0.f;
      }
    }
    u32x4 kr[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) kr[c] = s_k[buf][c][lane];
    const f32x16 s = tile_scores<T, NQ>(kr, qr);
    const int pos0 = it * kTileRows;
    ProbTile<T> p;
    if constexpr (CAUSAL) {
      if (pos0 + kTileRows - 1 <= w_row0)
        softmax_tile<T, ND, true, false, FOLD, true>(st, s, a.scale_log2, pos0, crow, half, p);
      else
        softmax_tile<T, ND, false, false, FOLD, true>(st, s, a.scale_log2, pos0, crow, half, p);
    } else if constexpr (MASK != kMaskNone) {
      float bias[16];
      if constexpr (MASK == kMaskKeys) {
        // keys 8k + 4*half .. +3 of the tile for registers 4k .. 4k+3
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4 kb = s_kb[buf][2 * k + half];
#pragma unroll
          for (int e = 0; e < 4; ++e) bias[4 * k + e] = kb[e];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) bias[r] = mk[r] * kLog2e;
      }
      softmax_tile<T, ND, false, true, false, true>(st, s, a.scale_log2, pos0, a.m - 1, half, p, bias);
    } else {
      if (pos0 + kTileRows <= a.m)
        softmax_tile<T, ND, true, false, FOLD, true>(st, s, a.scale_log2, pos0, a.m - 1, half, p);
      else
        softmax_tile<T, ND, false, false, FOLD, true>(st, s, a.scale_log2, pos0, a.m - 1, half, p);
    }
    PvOps<T> pv;
    pv.set(p);
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      u32x4 ops[VTC];
#pragma unroll
      for (int k = 0; k < VTC; ++k) ops[k] = s_vt[buf][d][k][lane];
      st.o[d] = pv.apply(ops, st.o[d]);
    }
  };

  // Tile it is committed to LDS buffer it & 1 from the chunk set it was
  // loaded into two steps earlier; right after the barrier that set is
  // refilled with tile it + 2, so loads have two tiles of compute to land.
  Chunks la, lb;
  issue(0, la);
  if (ntiles > 1) issue(1, lb);
  auto step = [&](int it, Chunks& ld) {
    const int buf = it & 1;
    commit(buf, ld);
    __syncthreads();
    if (it + 2 < ntiles) issue(it + 2, ld);
    if (it < w_tiles) compute(it, buf);
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, la);
    if (it + 1 < ntiles) step(it + 1, lb);
  }

  const float l_tot = sum_halves(st.l);
  if (col_ok) {
    // a row whose every key is masked out gets zeros (as an empty decode row)
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    T* op = reinterpret_cast<T*>(a.O) + (((size_t)bi * a.n + crow) * a.h + (size_t)g * a.hg + chead) * DH;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4(op + 32 * d + 8 * r4 + 4 * half, st.o[d][4 * r4] * inv, st.o[d][4 * r4 + 1] * inv,
               st.o[d][4 * r4 + 2] * inv, st.o[d][4 * r4 + 3] * inv);
  }
}

// Copies the prompt's K/V rows into positions [0, n) of every sequence of the
// cache and sets lens[b] = n.
__global__ void prefill_cache_copy_kernel(const char* K, const char* V, char* ck, char* cv,
                                          int32_t* lens, int b_copy, int b_lens, int n, int m_cap,
                                          int row_bytes) {
  const size_t per_seq = (size_t)n * row_bytes / 16;
  const size_t total = (size_t)b_copy * per_seq;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const size_t bi = idx / per_seq, r = idx % per_seq;
    const size_t src = bi * per_seq * 16 + r * 16;
    const size_t dst = bi * (size_t)m_cap * row_bytes + r * 16;
    *reinterpret_cast<u32x4*>(ck + dst) = *reinterpret_cast<const u32x4*>(K + src);
    *reinterpret_cast<u32x4*>(cv + dst) = *reinterpret_cast<const u32x4*>(V + src);
  }
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < (size_t)b_lens; i += stride)
    lens[i] = n;
}

namespace {
constexpr int kPrefillWaves = 8;

// Row blocks of NW * rpw query rows per (sequence, group).
PrefillArgs row_blocks(const PrefillParams& p, int m) {
  PrefillArgs a;
  a.Q = (const char*)p.Q;
  a.K = (const char*)p.K;
  a.V = (const char*)p.V;
  a.O = (char*)p.O;
  a.mask = nullptr;
  a.msb = a.msh = a.msn = 0;
  a.b = p.b;
  a.n = p.n;
  a.m = m;
  a.h = p.h;
  a.G = p.G;
  a.hg = p.h / p.G;
  int hgp = 1;
  while (hgp < a.hg) hgp *= 2;
  a.hgp = hgp;
  a.rpw = 32 / hgp;
  const int rows_per_block = kPrefillWaves * a.rpw;
  a.nrb = (p.n + rows_per_block - 1) / rows_per_block;
  a.scale_log2 = (float)((double)p.scale * 1.4426950408889634);
  return a;
}

template <typename T, int DH>
hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
  const int row_bytes = p.G * p.dh * (int)sizeof(T);
  if (p.cache_k || p.lens) {
    const size_t chunks = (size_t)p.b * p.n * row_bytes / 16;
    size_t blocks = (chunks + 255) / 256;
    if (blocks < (size_t)(p.b + 255) / 256) blocks = (p.b + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(prefill_cache_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const char*)p.K, (const char*)p.V, (char*)p.cache_k, (char*)p.cache_v,
                       p.lens, p.cache_k ? p.b : 0, p.lens ? p.b : 0, p.n, p.m_cap, row_bytes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const PrefillArgs a = row_blocks(p, p.n);
  const size_t blocks = (size_t)p.b * p.G * a.nrb;
  if (a.scale_log2 > 0.f)
    hipLaunchKernelGGL((prefill_kernel<T, DH, kPrefillWaves, true, true, kMaskNone>),
                       dim3((unsigned)blocks), dim3(kPrefillWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, DH, kPrefillWaves, true, false, kMaskNone>),
                       dim3((unsigned)blocks), dim3(kPrefillWaves * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t launch_attend_t(const AttendParams& q, hipStream_t s) {
  PrefillArgs a = row_blocks(q.base, q.m);
  a.mask = q.mask;
  a.msb = q.msb;
  a.msh = q.msh;
  a.msn = q.msn;
  const size_t blocks = (size_t)q.base.b * q.base.G * a.nrb;
  const dim3 grid((unsigned)blocks), block(kPrefillWaves * 64);
  if (q.mask && q.msh == 0 && q.msn == 0)
    hipLaunchKernelGGL((prefill_kernel<T, DH, kPrefillWaves, false, false, kMaskKeys>), grid,
                       block, 0, s, a);
  else if (q.mask)
    hipLaunchKernelGGL((prefill_kernel<T, DH, kPrefillWaves, false, false, kMaskFull>), grid,
                       block, 0, s, a);
  else if (a.scale_log2 > 0.f)
    hipLaunchKernelGGL((prefill_kernel<T, DH, kPrefillWaves, false, true, kMaskNone>), grid,
                       block, 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, DH, kPrefillWaves, false, false, kMaskNone>), grid,
                       block, 0, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  if (p.dtype == 1) {
    if (p.dh == 128) return launch_prefill_t<__bf16, 128>(p, s);
    return launch_prefill_t<__bf16, 64>(p, s);
  }
  if (p.dh == 128) return launch_prefill_t<float, 128>(p, s);
  return launch_prefill_t<float, 64>(p, s);
}

hipError_t launch_attend(const AttendParams& p, hipStream_t s) {
  if (p.base.dtype == 1) {
    if (p.base.dh == 128) return launch_attend_t<__bf16, 128>(p, s);
    return launch_attend_t<__bf16, 64>(p, s);
  }
  if (p.base.dh == 128) return launch_attend_t<float, 128>(p, s);
  return launch_attend_t<float, 64>(p, s);
}

}  // namespace mqa
