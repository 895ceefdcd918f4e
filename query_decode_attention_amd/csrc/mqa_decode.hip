// mqa_decode.hip -- gfx950 kernels of one MQA/GQA decode step:
//   kv_append_kernel      : concat of one new K/V row per sequence
//                           (paper review, section 3 incremental pseudocode)
//   decode_split_kernel   : scores, online softmax and weighted V over a
//                           balanced share of all cached positions
//                           (study notes section 4: o_i = softmax(q_i K^T s) V)
//   decode_combine_kernel : exact merge of the split-K partial softmaxes
//
// Work decomposition.  The visible positions of every (sequence b, group g)
// are cut into tiles of 32.  All tiles of all segments form one flat list of
// T tiles; workgroup w of a grid of W takes tiles [T*w/W, T*(w+1)/W), so
// every workgroup streams the same number of bytes whatever the length mix.
// Inside a workgroup, wave k takes every NW-th tile of a segment; waves merge
// their (max, sum, accumulator) through LDS; a segment that one workgroup
// covers completely is normalised and written directly, the (at most two)
// segments it shares with neighbours become fp32 partial records that the
// combine kernel merges.  The flat tile list is derived on the device from
// lens, so no host synchronisation is needed.
//
// One wave, one 32-position tile, all h/G <= 32 heads of the group:
//   S^T[32 pos][32 heads] = K_tile . Q^T        (MFMA; K rows are the A operand
//                                                loaded straight from HBM)
//   online softmax per head column (log2 domain, scale*log2(e) folded in)
//   V_tile^T via an exact 0/1-selection MFMA    (turns position-major rows into
//                                                the d-major A operand of PV)
//   O^T[d][heads] += V^T . P^T                   (MFMA; P stays in registers)
// Each K/V byte is read from HBM once and used by every head of its group.
#include "mqa_device.h"
#include "mqa_internal.h"

namespace mqa {

// ----------------------------------------------------------------- append ----

__global__ void kv_append_kernel(AppendParams p) {
  const int bi = blockIdx.x;
  const int pos = p.lens[bi];
  if (pos < 0 || pos >= p.m_cap) {
    if (threadIdx.x == 0 && p.err_flag) *p.err_flag = 1;
    return;
  }
  const int chunks = p.row_bytes >> 4;
  const size_t dst = ((size_t)bi * p.m_cap + pos) * (size_t)p.row_bytes;
  const size_t src = (size_t)bi * p.row_bytes;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>((const char*)p.k_new + src + 16 * c);
    const u32x4 vv = *reinterpret_cast<const u32x4*>((const char*)p.v_new + src + 16 * c);
    *reinterpret_cast<u32x4*>((char*)p.k + dst + 16 * c) = kv;
    *reinterpret_cast<u32x4*>((char*)p.v + dst + 16 * c) = vv;
  }
  __syncthreads();  // every thread has read lens[bi] before it changes
  if (threadIdx.x == 0) p.lens[bi] = pos + 1;
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(p.b), dim3(64), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------- decode: shared ----

struct SplitArgs {
  const char* q;
  const char* k;
  const char* v;
  const int32_t* lens;
  char* o;
  int32_t* prefix;  // [b + 1] exclusive prefix of tiles per sequence (written by block 0)
  float* records;   // [2 * grid][rec_floats]
  int b, h, G, hg, m_cap, window;
  int rec_floats;
  float scale_log2;
};

__device__ __forceinline__ void visible_range(const int32_t* lens, int bi, int m_cap, int window,
                                              int& j0, int& L) {
  int l = lens[bi];
  l = l < 0 ? 0 : (l > m_cap ? m_cap : l);
  j0 = (window > 0 && l > window) ? l - window : 0;
  L = l;
}

__device__ __forceinline__ int tiles_of(int j0, int L) { return (L - j0 + kTileRows - 1) / kTileRows; }

// First flat tile of workgroup w out of W over T tiles.
__device__ __forceinline__ int64_t wg_start(int64_t T, int w, int W) { return T * w / W; }
// Workgroup whose range contains flat tile t (T > 0).
__device__ __forceinline__ int wg_of(int64_t t, int64_t T, int W) {
  return (int)(((t + 1) * W + T - 1) / T) - 1;
}

// Exclusive block-wide prefix sum of v; `total` receives the block sum.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = s_tmp[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// ------------------------------------------------------ decode: split kernel ----

template <int NQ, bool FULL>
__device__ __forceinline__ void load_kv(const char* kp, const char* vp, bool valid, int half,
                                        u32x4 (&kr)[NQ], u32x4 (&vr)[NQ]) {
  if (FULL || valid) {
#pragma unroll
    for (int c = 0; c < NQ; ++c)
      kr[c] = *reinterpret_cast<const u32x4*>(kp + (2 * c + half) * 16);
#pragma unroll
    for (int c = 0; c < NQ; ++c)
      vr[c] = *reinterpret_cast<const u32x4*>(vp + (2 * c + half) * 16);
  } else {
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      kr[c] = u32x4{0u, 0u, 0u, 0u};
      vr[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// One decode tile: scores, online softmax with the tail masked at L, and P.V
// with the V rows transposed in registers.
template <typename T, int DH, bool FULL>
__device__ __forceinline__ void tile_update(WaveState<TileShape<T, DH>::ND>& st,
                                            const u32x4 (&kr)[TileShape<T, DH>::NQ],
                                            const u32x4 (&vr)[TileShape<T, DH>::NQ],
                                            const u32x4 (&qr)[TileShape<T, DH>::NQ],
                                            const SelOps<T>& sel, float scale_log2,
                                            int pos0, int L, int half) {
  constexpr int NQ = TileShape<T, DH>::NQ;
  constexpr int ND = TileShape<T, DH>::ND;
  constexpr int VTC = TileShape<T, DH>::VTC;
  const f32x16 s = tile_scores<T, NQ>(kr, qr);
  float p[16];
  softmax_tile<T, ND, FULL>(st, s, scale_log2, pos0, L - 1, half, p);
  PvOps<T> pv;
  pv.set(p);
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    u32x4 ops[VTC];
    transpose_block<T, NQ>(vr, d, sel, ops);
    st.o[d] = pv.apply(ops, st.o[d]);
  }
}

template <int ND>
struct MergeSlot {
  f32x4 o[ND][4][64];
  float m[64];
  float l[64];
};

// Fold `other` (m_o, l_o, o_o) into `st` (exact softmax re-association).
template <int ND>
__device__ __forceinline__ void merge_into(WaveState<ND>& st, const MergeSlot<ND>& sl, int lane) {
  const float m_o = sl.m[lane], l_o = sl.l[lane];
  const float M = fmaxf(st.m, m_o);
  const float Ms = (M == kNegInf) ? 0.f : M;  // both empty: keep zeros, avoid inf - inf
  const float fa = fast_exp2(st.m - Ms), fb = fast_exp2(m_o - Ms);
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 x = sl.o[d][r4][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[d][4 * r4 + i] = st.o[d][4 * r4 + i] * fa + x[i] * fb;
    }
  st.l = st.l * fa + l_o * fb;
  st.m = M;
}

template <int ND>
__device__ __forceinline__ void store_slot(const WaveState<ND>& st, MergeSlot<ND>& sl, int lane) {
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      sl.o[d][r4][lane] = f32x4{st.o[d][4 * r4], st.o[d][4 * r4 + 1], st.o[d][4 * r4 + 2],
                                st.o[d][4 * r4 + 3]};
  sl.m[lane] = st.m;
  sl.l[lane] = st.l;
}

template <typename T, int DH, int NW, bool PREFETCH>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(SplitArgs a) {
  using S = TileShape<T, DH>;
  constexpr int NQ = S::NQ, ND = S::ND;
  static_assert(NW == 1 || NW == 2 || NW == 4 || NW == 8, "tree merge assumes NW a power of two <= 8");
  __shared__ int s_scan[NW];
  __shared__ int s_found[2];
  __shared__ MergeSlot<ND> s_slot[NW > 1 ? NW / 2 : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 31, half = lane >> 5;

  // ---- schedule: tiles per sequence, total, and this workgroup's range ----
  int total = 0;
  for (int c = 0; c < a.b; c += NW * 64) {
    const int bi = c + (int)threadIdx.x;
    int v = 0;
    if (bi < a.b) {
      int j0, L;
      visible_range(a.lens, bi, a.m_cap, a.window, j0, L);
      v = tiles_of(j0, L);
    }
    int tot;
    const int ex = block_excl_scan<NW>(v, s_scan, tot);
    if (blockIdx.x == 0 && bi < a.b) a.prefix[bi] = total + ex;
    total += tot;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) a.prefix[a.b] = total;
  const int64_t Tt = (int64_t)total * a.G;
  const int W = gridDim.x;
  const int64_t t0 = wg_start(Tt, blockIdx.x, W), t1 = wg_start(Tt, blockIdx.x + 1, W);
  if (t0 >= t1) return;

  // locate the sequence holding flat tile t0
  if (threadIdx.x == 0) s_found[0] = -1;
  __syncthreads();
  int run = 0;
  for (int c = 0; c < a.b; c += NW * 64) {
    const int bi = c + (int)threadIdx.x;
    int v = 0;
    if (bi < a.b) {
      int j0, L;
      visible_range(a.lens, bi, a.m_cap, a.window, j0, L);
      v = tiles_of(j0, L);
    }
    int tot;
    const int ex = block_excl_scan<NW>(v, s_scan, tot);
    const int64_t lo = (int64_t)(run + ex) * a.G, hi = (int64_t)(run + ex + v) * a.G;
    if (bi < a.b && v > 0 && lo <= t0 && t0 < hi) {
      s_found[0] = bi;
      s_found[1] = run + ex;
    }
    run += tot;
    __syncthreads();
    if (s_found[0] >= 0) break;
  }
  int b_cur = __builtin_amdgcn_readfirstlane(s_found[0]);
  int64_t seg_base = (int64_t)__builtin_amdgcn_readfirstlane(s_found[1]) * a.G;

  SelOps<T> sel;
  sel.init(row, half);

  const size_t row_stride = (size_t)a.G * DH * sizeof(T);
  int64_t t = t0;
  bool first = true;
  while (t < t1 && b_cur < a.b) {
    int j0, L;
    visible_range(a.lens, b_cur, a.m_cap, a.window, j0, L);
    j0 = __builtin_amdgcn_readfirstlane(j0);
    L = __builtin_amdgcn_readfirstlane(L);
    const int nb = tiles_of(j0, L);
    if (nb == 0) {
      ++b_cur;
      continue;
    }
    const int g = (int)((t - seg_base) / nb);
    const int64_t seg0 = seg_base + (int64_t)g * nb;
    const int ta = (int)(t - seg0);
    const int te = (int)((t1 < seg0 + nb ? t1 : seg0 + nb) - seg0);
    const bool complete = (ta == 0 && te == nb);

    // ---- per-wave pass over tiles ta + wave, ta + wave + NW, ... < te ----
    WaveState<ND> st;
    st.reset();
    const int head = row;
    u32x4 qr[NQ];
    if (head < a.hg) {
      const char* qp = a.q + ((size_t)b_cur * a.h + (size_t)g * a.hg + head) * DH * sizeof(T);
#pragma unroll
      for (int c = 0; c < NQ; ++c) qr[c] = *reinterpret_cast<const u32x4*>(qp + (2 * c + half) * 16);
    } else {
#pragma unroll
      for (int c = 0; c < NQ; ++c) qr[c] = u32x4{0u, 0u, 0u, 0u};
    }
    const size_t seq_off = ((size_t)b_cur * a.m_cap * a.G + (size_t)g) * DH * sizeof(T);
    const char* kseq = a.k + seq_off;
    const char* vseq = a.v + seq_off;

    auto tile_ptrs = [&](int tile, const char*& kp, const char*& vp, int& pos0) {
      pos0 = j0 + tile * kTileRows;
      const size_t off = (size_t)(pos0 + row) * row_stride;
      kp = kseq + off;
      vp = vseq + off;
    };
    auto run_tile = [&](int tile, const u32x4 (&kr)[NQ], const u32x4 (&vr)[NQ]) {
      const int pos0 = j0 + tile * kTileRows;
      if (pos0 + kTileRows <= L)
        tile_update<T, DH, true>(st, kr, vr, qr, sel, a.scale_log2, pos0, L, half);
      else
        tile_update<T, DH, false>(st, kr, vr, qr, sel, a.scale_log2, pos0, L, half);
    };
    auto load_tile = [&](int tile, u32x4 (&kr)[NQ], u32x4 (&vr)[NQ]) {
      const char *kp, *vp;
      int pos0;
      tile_ptrs(tile, kp, vp, pos0);
      if (pos0 + kTileRows <= L)
        load_kv<NQ, true>(kp, vp, true, half, kr, vr);
      else
        load_kv<NQ, false>(kp, vp, pos0 + row < L, half, kr, vr);
    };

    int tile = ta + wave;
    if constexpr (PREFETCH) {
      u32x4 kA[NQ], vA[NQ], kB[NQ], vB[NQ];
      if (tile < te) load_tile(tile, kA, vA);
      while (tile < te) {
        if (tile + NW < te) load_tile(tile + NW, kB, vB);
        run_tile(tile, kA, vA);
        tile += NW;
        if (tile >= te) break;
        if (tile + NW < te) load_tile(tile + NW, kA, vA);
        run_tile(tile, kB, vB);
        tile += NW;
      }
    } else {
      u32x4 kA[NQ], vA[NQ];
      for (; tile < te; tile += NW) {
        load_tile(tile, kA, vA);
        run_tile(tile, kA, vA);
      }
    }

    // ---- merge the waves (tree through LDS) ----
#pragma unroll
    for (int s = NW / 2; s >= 1; s /= 2) {
      if (wave >= s && wave < 2 * s) store_slot<ND>(st, s_slot[wave - s], lane);
      __syncthreads();
      if (wave < s) merge_into<ND>(st, s_slot[wave], lane);
      __syncthreads();
    }

    // ---- wave 0 writes the segment result ----
    const float l_tot = st.l + xor32(st.l);
    if (wave == 0 && head < a.hg) {
      if (complete) {
        const float inv = 1.0f / l_tot;
        T* op = reinterpret_cast<T*>(a.o) + ((size_t)b_cur * a.h + (size_t)g * a.hg + head) * DH;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            store4(op + 32 * d + 8 * r4 + 4 * half, st.o[d][4 * r4] * inv,
                   st.o[d][4 * r4 + 1] * inv, st.o[d][4 * r4 + 2] * inv,
                   st.o[d][4 * r4 + 3] * inv);
      } else {
        float* rec = a.records + ((size_t)blockIdx.x * 2 + (first ? 0 : 1)) * a.rec_floats;
        float* ro = rec + (size_t)head * DH;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            store4(ro + 32 * d + 8 * r4 + 4 * half, st.o[d][4 * r4], st.o[d][4 * r4 + 1],
                   st.o[d][4 * r4 + 2], st.o[d][4 * r4 + 3]);
        if (half == 0) {
          rec[(size_t)a.hg * DH + head] = st.m;
          rec[(size_t)a.hg * DH + a.hg + head] = l_tot;
        }
      }
    }

    first = false;
    t = seg0 + te;
    if (g == a.G - 1 && te == nb) {
      seg_base += (int64_t)a.G * nb;
      ++b_cur;
    }
  }
}

// --------------------------------------------------- decode: combine kernel ----

struct CombineArgs {
  const int32_t* lens;
  const int32_t* prefix;
  const float* records;
  char* o;
  int b, h, G, hg, m_cap, window, rec_floats, grid;
};

template <typename T, int DH>
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineArgs a) {
  const int seg = blockIdx.x;
  const int bi = seg / a.G, g = seg % a.G;
  const int idx = blockIdx.y * 256 + threadIdx.x;
  if (idx >= a.hg * (DH / 4)) return;
  const int head = idx / (DH / 4), d4 = idx % (DH / 4);
  T* out = reinterpret_cast<T*>(a.o) + ((size_t)bi * a.h + (size_t)g * a.hg + head) * DH + 4 * d4;
  int j0, L;
  visible_range(a.lens, bi, a.m_cap, a.window, j0, L);
  const int nb = tiles_of(j0, L);
  if (nb == 0) {  // empty row: zeros by convention
    store4(out, 0.f, 0.f, 0.f, 0.f);
    return;
  }
  const int64_t Tt = (int64_t)a.prefix[a.b] * a.G;
  const int64_t S = (int64_t)a.prefix[bi] * a.G + (int64_t)g * nb;
  const int wf = wg_of(S, Tt, a.grid), wl = wg_of(S + nb - 1, Tt, a.grid);
  if (wf == wl) return;  // one workgroup covered the segment and wrote it
  // Workgroups between wf and wl whose range is empty (grid > tiles) wrote
  // nothing and are skipped.
  float M = kNegInf;
  for (int w = wf; w <= wl; ++w) {
    if (wg_start(Tt, w, a.grid) == wg_start(Tt, w + 1, a.grid)) continue;
    const int slot = (w == wf && wg_start(Tt, w, a.grid) < S) ? 1 : 0;
    const float* rec = a.records + ((size_t)w * 2 + slot) * a.rec_floats;
    M = fmaxf(M, rec[(size_t)a.hg * DH + head]);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  for (int w = wf; w <= wl; ++w) {
    if (wg_start(Tt, w, a.grid) == wg_start(Tt, w + 1, a.grid)) continue;
    const int slot = (w == wf && wg_start(Tt, w, a.grid) < S) ? 1 : 0;
    const float* rec = a.records + ((size_t)w * 2 + slot) * a.rec_floats;
    const float f = fast_exp2(rec[(size_t)a.hg * DH + head] - M);
    lsum += f * rec[(size_t)a.hg * DH + a.hg + head];
    const f32x4 x = *reinterpret_cast<const f32x4*>(rec + (size_t)head * DH + 4 * d4);
    acc += x * f;
  }
  const float inv = 1.0f / lsum;
  store4(out, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
}

// ------------------------------------------------------------------- host ----

size_t decode_record_bytes(int hg, int dh) {
  size_t f = (size_t)hg * dh + 2 * (size_t)hg;
  f = (f + 3) & ~(size_t)3;  // 16-byte multiple
  return f * sizeof(float);
}

size_t decode_records_offset(int b) {
  return (((size_t)b + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
}

int decode_grid_cap(int b, int G, int m_cap) {
  const int64_t max_tiles = (int64_t)b * G * ((m_cap + kTileRows - 1) / kTileRows);
  return (int)(max_tiles < kMaxDecodeGrid ? max_tiles : kMaxDecodeGrid);
}

size_t decode_workspace_bytes(int b, int h, int G, int dh, int m_cap) {
  return decode_records_offset(b) +
         2 * (size_t)decode_grid_cap(b, G, m_cap) * decode_record_bytes(h / G, dh);
}

namespace {
constexpr int kDecodeWaves = 8;

template <typename T, int DH>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  constexpr bool kPrefetch = false;
  auto split = decode_split_kernel<T, DH, kDecodeWaves, kPrefetch>;
  int dev = 0;
  const int cus = current_device_cus(&dev);
  if (cus <= 0) return hipErrorInvalidDevice;
  // Occupancy of the split kernel, cached per device.
  static int occ_cache[64];
  int occ = (dev >= 0 && dev < 64) ? occ_cache[dev] : 0;
  if (occ <= 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, split, kDecodeWaves * 64, 0);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    if (dev >= 0 && dev < 64) occ_cache[dev] = occ;
  }
  int grid = cus * occ;
  const int cap = decode_grid_cap(p.b, p.G, p.m_cap);
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;

  SplitArgs sa;
  sa.q = (const char*)p.q;
  sa.k = (const char*)p.k;
  sa.v = (const char*)p.v;
  sa.lens = p.lens;
  sa.o = (char*)p.o;
  sa.prefix = (int32_t*)p.ws;
  sa.records = (float*)((char*)p.ws + decode_records_offset(p.b));
  sa.b = p.b;
  sa.h = p.h;
  sa.G = p.G;
  sa.hg = p.h / p.G;
  sa.m_cap = p.m_cap;
  sa.window = p.window;
  sa.rec_floats = (int)(decode_record_bytes(sa.hg, DH) / sizeof(float));
  sa.scale_log2 = (float)((double)p.scale * 1.4426950408889634);
  hipError_t e;
  if (p.ev_begin && (e = hipEventRecord(p.ev_begin, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(split, dim3(grid), dim3(kDecodeWaves * 64), 0, s, sa);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_end && (e = hipEventRecord(p.ev_end, s)) != hipSuccess) return e;

  CombineArgs ca;
  ca.lens = p.lens;
  ca.prefix = sa.prefix;
  ca.records = sa.records;
  ca.o = (char*)p.o;
  ca.b = p.b;
  ca.h = p.h;
  ca.G = p.G;
  ca.hg = sa.hg;
  ca.m_cap = p.m_cap;
  ca.window = p.window;
  ca.rec_floats = sa.rec_floats;
  ca.grid = grid;
  const int per_seg = sa.hg * (DH / 4);
  dim3 cgrid((unsigned)(p.b * p.G), (unsigned)((per_seg + 255) / 256));
  hipLaunchKernelGGL((decode_combine_kernel<T, DH>), cgrid, dim3(256), 0, s, ca);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (p.dtype == 1) {
    if (p.dh == 128) return launch_decode_t<__bf16, 128>(p, s);
    return launch_decode_t<__bf16, 64>(p, s);
  }
  if (p.dh == 128) return launch_decode_t<float, 128>(p, s);
  return launch_decode_t<float, 64>(p, s);
}

}  // namespace mqa
