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
// rows are staged in LDS once and read by all NW waves, in several buffers so
// that later tiles' global loads overlap this tile's MFMAs.  The fp32 kernel
// stages V transposed into the PV operand layout (an exact selection MFMA);
// the bf16 kernel stages V rows as they are and reads the operand with the
// LDS transposing read.  Row blocks are launched last-row-first so the
// longest causal rows start early.
#include <type_traits>

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
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) float lds_float;
// LDS bytes prefill_rows uses (double-buffered K chunks, transposed V
// chunks and the per-key mask of a tile).
template <typename T, int DH>
struct RowsLds {
  using S = TileShape<T, DH>;
  static constexpr size_t kBytesK = 2 * S::NQ * 64 * sizeof(u32x4);               // s_k[2][NQ][64]
  static constexpr size_t kBytesVt = 2 * S::ND * S::VTC * 64 * sizeof(u32x4);    // s_vt[2][ND][VTC][64]
  static constexpr size_t kBytesKb = 2 * (kTileRows / 4) * sizeof(f32x4);        // s_kb[2][8]
};

// The rescaling body: the workgroup's rows with a running softmax maximum
// (the fp32 kernel, and the bf16 kernel's rescue).  Not inlined: the bf16
// kernel calls it only to recompute a workgroup whose logits outgrew their
// fixed softmax reference, and inlining it there would add its registers to
// the bf16 kernel's hot loops.  Its LDS comes from the caller: the fp32
// kernel's own arrays, or, in the bf16 kernel's rescue, the bf16 loops' tile
// buffers (free by then).
template <typename T, int DH, int NW, bool CAUSAL, bool FOLD, int MASK>
__device__ __attribute__((noinline)) void prefill_rows(const PrefillArgs a, lds_u32x4* k_mem,
                                                       lds_u32x4* vt_mem, lds_f32x4* kb_mem) {
  using S = TileShape<T, DH>;
  constexpr int NQ = S::NQ, ND = S::ND, VTC = S::VTC;
  static_assert(NW >= ND, "a wave per d block transposes V");
  constexpr int KPW = (NQ + NW - 1) / NW;     // K chunks per wave
  constexpr int VPW = NQ / ND;                // V chunks per d block
  lds_u32x4 (*const s_k)[NQ][64] = reinterpret_cast<lds_u32x4 (*)[NQ][64]>(k_mem);
  lds_u32x4 (*const s_vt)[ND][VTC][64] = reinterpret_cast<lds_u32x4 (*)[ND][VTC][64]>(vt_mem);
  // per-key mask of the tile (key padding)
  lds_f32x4 (*const s_kb)[kTileRows / 4] = reinterpret_cast<lds_f32x4 (*)[kTileRows / 4]>(kb_mem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;

  // Causal: row blocks in order of decreasing length (the latest rows see
  // the most keys) with the (sequence, group) pairs interleaved, so that no
  // long block is left for the end and a pair's workgroups share an XCD's L2
  // when the pair count divides the XCD count.  Otherwise pair-major: every
  // XCD takes its share of every pair (pairs may differ in length when a
  // key-padding mask cuts them short).
  const int nbg = a.b * a.G;
  const int rb = a.nrb - 1 - (int)(CAUSAL ? blockIdx.x / nbg : blockIdx.x % a.nrb);
  const int bg = CAUSAL ? (int)(blockIdx.x % nbg) : (int)(blockIdx.x / a.nrb);
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
    if (kb_wave && half == 0) reinterpret_cast<lds_float*>(s_kb[buf])[col] = ld.kb;
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

template <typename T, int DH, int NW, bool CAUSAL, bool FOLD, int MASK>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillArgs a) {
  using L = RowsLds<T, DH>;
  __shared__ u32x4 s_k[L::kBytesK / sizeof(u32x4)];
  __shared__ u32x4 s_vt[L::kBytesVt / sizeof(u32x4)];
  __shared__ f32x4 s_kb[L::kBytesKb / sizeof(f32x4)];
  prefill_rows<T, DH, NW, CAUSAL, FOLD, MASK>(a, (lds_u32x4*)s_k, (lds_u32x4*)s_vt, (lds_f32x4*)s_kb);
}

// ------------------------------------------------------------ bf16 kernel
//
// The bf16 path runs the same computation with the tiles of a wave software
// pipelined, so that matrix-core and vector work overlap inside each wave:
// iteration j of a wave issues
//     PV(j-1):  O^T += V_{j-1}^T . P_{j-1}^T     (MFMA)
//     softmax(j): S_j -> P_j                      (VALU: max, exp2, bf16 pack)
//     S(j+1) = K_{j+1} . Q^T                      (MFMA)
// and neither product depends on the softmax between them, so the scheduler
// is asked to interleave them.  K and V rows go straight into four LDS tile
// buffers, three tiles ahead (see the staging below), and the PV operand is
// read transposed from the V rows.  Tiles that every wave of the workgroup
// sees in full run in a loop without any masking; the diagonal and the tiles
// after it run in a second loop whose softmax masks by position.
//
// The softmax packs its probabilities two at a time (v_cvt_pk_bf16_f32) and
// sums the packed, rounded values with v_dot2_f32_bf16 against (1, 1), so the
// normaliser l sums exactly the weights the PV product uses.
//
// A column's softmax reference m is fixed at the first tile where it sees a
// finite logit and is never raised inside the loops: rescaling O under a
// branch makes the compiler copy the 64 accumulator registers around it,
// which costs more than the whole softmax.  While no later logit exceeds m
// by more than kFixedSlack (log2 units), every probability is below
// 2^kFixedSlack, so l <= n * 2^64 and O stay far inside fp32 and bf16 range.
// A workgroup in which some column's logit does exceed its reference by more
// than that recomputes its rows with the rescaling kernel body instead.
//
// Once every column of a wave holds its reference, its tiles skip the tile
// maximum altogether: a probability above 2^kFixedSlack then shows in the
// lane's sum of the tile's rounded probabilities, which is at least as large
// (all terms are non-negative, and bf16 rounding to nearest keeps a value
// above 2^64 at or above 2^64).  The sum test also fires for sums of many
// smaller terms that reach 2^64; those workgroups take the exact rescue too.
// Every flag is set branch-free, so a tile's products and softmax stay one
// basic block the scheduler can interleave.

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Workgroup barrier for LDS data only: this wave's LDS writes complete, then
// s_barrier.  __syncthreads() would also wait for every outstanding memory
// load, including direct-to-LDS loads of tiles that are not needed yet;
// those are waited for by the wave that issued them (s_waitcnt vmcnt)
// before the barrier that publishes them.  The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Largest index p < m with mask[p] != -inf (the last key a key-padding mask
// leaves visible), or -1; the same in every lane of the wave.
__device__ __forceinline__ int last_visible_key(const float* mask, int m, int lane) {
  int last = -1;
  int p = lane;
  for (; p + 7 * 64 < m; p += 8 * 64) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = mask[p + u * 64];
#pragma unroll
    for (int u = 0; u < 8; ++u) last = v[u] != kNegInf ? p + u * 64 : last;
  }
  for (; p < m; p += 64) last = mask[p] != kNegInf ? p : last;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  return last;
}

constexpr float kFixedSlack = 64.0f;
constexpr float kOverSum = 0x1p64f;  // 2^kFixedSlack

// Softmax of one tile against the column's fixed reference; `over` is set in
// a lane whose tile exceeds the reference by more than the slack.  REF: every
// column of the wave already holds a finite reference (no tile maximum).
template <int ND, bool FULL, bool BIAS, bool FOLD, bool REF>
__device__ __forceinline__ void softmax_fixed(WaveState<ND>& st, const f32x16& s, float scale_log2,
                                              int pos0, int lim, int half, bf16x8 (&pb)[2],
                                              const float* bias, bool& over) {
  static_assert(!(FOLD && BIAS), "the folded form has no bias");
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    x[r] = FOLD ? s[r] : s[r] * scale_log2;
    if constexpr (BIAS) x[r] += bias[r];
    if (!FULL && pos0 + d_row(r, half) > lim) x[r] = kNegInf;
  }
  float ref = st.m;
  if constexpr (!REF) {
    // max over the lane's 16 values in a tree of three-input maxima
    float m3[6];
#pragma unroll
    for (int k = 0; k < 5; ++k) m3[k] = fmaxf(fmaxf(x[3 * k], x[3 * k + 1]), x[3 * k + 2]);
    m3[5] = x[15];
    float mt = fmaxf(fmaxf(m3[0], m3[1]), m3[2]);
    mt = fmaxf(fmaxf(mt, m3[3]), fmaxf(m3[4], m3[5]));
    mt = max_halves(mt);
    if constexpr (FOLD) mt *= scale_log2;  // -inf stays -inf (scale_log2 > 0)
    const bool had = st.m != kNegInf;
    over = over | (had & (mt > st.m + kFixedSlack));
    st.m = had ? st.m : mt;
    ref = (st.m == kNegInf) ? 0.f : st.m;
  }
  bf16x2 p2[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float e0 = fast_exp2(FOLD ? __builtin_fmaf(x[2 * k], scale_log2, -ref) : x[2 * k] - ref);
    const float e1 =
        fast_exp2(FOLD ? __builtin_fmaf(x[2 * k + 1], scale_log2, -ref) : x[2 * k + 1] - ref);
    p2[k] = __builtin_convertvector(f32x2{e0, e1}, bf16x2);
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float sa = 0.f, sb = 0.f;  // two chains of dependent sums
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    sa = __builtin_amdgcn_fdot2_f32_bf16(p2[k], ones, sa, false);
    sb = __builtin_amdgcn_fdot2_f32_bf16(p2[k + 1], ones, sb, false);
  }
  const float tile_sum = sa + sb;
  if constexpr (REF) over = over | (tile_sum >= kOverSum);
  st.l += tile_sum;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pb[h] = bf16x8{p2[4 * h][0], p2[4 * h][1], p2[4 * h + 1][0], p2[4 * h + 1][1],
                   p2[4 * h + 2][0], p2[4 * h + 2][1], p2[4 * h + 3][0], p2[4 * h + 3][1]};
  }
}

// (at least two waves per SIMD: with four-wave workgroups, two share a CU)
template <int DH, int NW, bool CAUSAL, bool FOLD, int MASK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_bf16_kernel(
    PrefillArgs a) {
  using T = __bf16;
  using S = TileShape<T, DH>;
  constexpr int NQ = S::NQ, ND = S::ND;
  constexpr int NB = 4;                       // LDS tile buffers (a power of two)
  constexpr int CPW = 2 * NQ / NW;            // K and V chunks staged per wave and tile
  static_assert(2 * NQ % NW == 0, "K and V chunks shared out evenly");
  constexpr bool BIAS = MASK != kMaskNone;
  // K chunk c: entry `lane` holds the score product's operand fragment (key
  // lane % 32, d 16c + 8 (lane / 32) ..).  V chunk c: entry 2 key + e holds
  // d 16c + 8e .. of the key, so the chunk is the 32 keys' d range as 32-byte
  // rows, which the PV operand reads transposed (read_vt below).
  __shared__ u32x4 s_k[NB][NQ][64];
  // (V chunks 1152 bytes apart: the two chunks of a 32-wide d block, read
  // by lanes 0-15 and 16-31 of one transposing read, then fall in different
  // LDS banks)
  __shared__ u32x4 s_v[NB][NQ][72];
  __shared__ float s_kbw[NB][NW][64];  // per-key mask of the tile (key padding), a copy per wave
  __shared__ int s_over;                     // some column exceeded its reference

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;

  // Causal: row blocks in order of decreasing length (the latest rows see
  // the most keys) with the (sequence, group) pairs interleaved, so that no
  // long block is left for the end and a pair's workgroups share an XCD's L2
  // when the pair count divides the XCD count.  Otherwise pair-major: every
  // XCD takes its share of every pair (pairs may differ in length when a
  // key-padding mask cuts them short).
  const int nbg = a.b * a.G;
  const int rb = a.nrb - 1 - (int)(CAUSAL ? blockIdx.x / nbg : blockIdx.x % a.nrb);
  const int bg = CAUSAL ? (int)(blockIdx.x % nbg) : (int)(blockIdx.x / a.nrb);
  const int bi = bg / a.G, g = bg % a.G;
  const int rows_per_block = NW * a.rpw;
  const int r_begin = rb * rows_per_block;
  if (r_begin >= a.n) return;
  const int r_end = min(a.n, r_begin + rows_per_block);
  int ntiles = CAUSAL ? (r_end - 1) / kTileRows + 1 : (a.m + kTileRows - 1) / kTileRows;
  if constexpr (MASK == kMaskKeys) {
    // tiles past the last key the mask leaves visible add exactly nothing:
    // skip them (tile 0 always runs, so a fully hidden row still ends at 0)
    const int last = last_visible_key(a.mask + (int64_t)bi * a.msb, a.m, lane);
    ntiles = min(ntiles, max(1, last / kTileRows + 1));
  }
  // tiles [0, j_full) are visible in full to every column of the workgroup
  const int j_full = min(ntiles, CAUSAL ? (r_begin + 1) / kTileRows : a.m / kTileRows);

  const int w_row0 = r_begin + wave * a.rpw;
  const int w_last = min(a.n - 1, w_row0 + a.rpw - 1);
  const int w_tiles = (w_row0 < a.n) ? (CAUSAL ? w_last / kTileRows + 1 : ntiles) : 0;
  const int crow = w_row0 + col / a.hgp;
  const int chead = col % a.hgp;
  const bool col_ok = crow < a.n && chead < a.hg;
  const int lim = CAUSAL ? crow : a.m - 1;
  if (threadIdx.x == 0) s_over = 0;  // ordered before its readers by the loops' barriers

  u32x4 qr[NQ];
  {
    // columns past n or past h/G read a real row (finite values, never stored)
    const int qrow = crow < a.n ? crow : a.n - 1;
    const int qhead = chead < a.hg ? chead : 0;
    const char* qp =
        a.Q + (((size_t)bi * a.n + qrow) * a.h + (size_t)g * a.hg + qhead) * DH * sizeof(T);
#pragma unroll
    for (int c = 0; c < NQ; ++c) qr[c] = *reinterpret_cast<const u32x4*>(qp + (2 * c + half) * 16);
  }

  const size_t rs = (size_t)a.G * DH * sizeof(T);
  const size_t seq_off = ((size_t)bi * a.m * a.G + (size_t)g) * DH * sizeof(T);
  const char* kseq = a.K + seq_off;
  const char* vseq = a.V + seq_off;

  // Staging, straight into LDS (global_load_lds) three tiles ahead: the
  // 2*NQ chunks of a tile's K and V rows (1 KB each) are shared out evenly,
  // wave w taking chunks w, w + NW, ... (K chunks first).  A K chunk is
  // loaded in its operand layout (lane: key lane % 32, d half lane / 32), a
  // V chunk as 32-byte rows (lane: key lane / 2, d half lane % 2), so both
  // land lane by lane, contiguously.  Positions past m read row m - 1
  // (finite; masked).  With a key-padding mask every wave also fetches the
  // tile's mask values into a slot of its own.  Tile t + 3 is issued after
  // iteration t's barrier, by which every wave is done with the buffer it
  // refills (that of tile t - 1, whose last reader is PV(t - 1) before the
  // barrier).
  const uint32_t rs32 = (uint32_t)rs;
  // byte offsets of this lane's K and V rows of a tile (positions clamped;
  // one 32 x 32 -> 64-bit multiply each)
  auto row_offsets = [&](int tile, uint32_t& pos_k, uint64_t& off_k, uint64_t& off_v) {
    const int pk = tile * kTileRows + col, pv_ = tile * kTileRows + (lane >> 1);
    pos_k = (uint32_t)(pk < a.m ? pk : a.m - 1);
    off_k = (uint64_t)pos_k * rs32;
    off_v = (uint64_t)(uint32_t)(pv_ < a.m ? pv_ : a.m - 1) * rs32;
  };
  const float* kbw_row = MASK == kMaskKeys ? a.mask + (int64_t)bi * a.msb : nullptr;
  constexpr int kPerTile = CPW + (MASK == kMaskKeys ? 1 : 0);  // loads per wave and tile
  static_assert(2 * kPerTile <= 15, "vmcnt immediate");
  auto issue_dma = [&](int tile) {
    uint32_t pos;
    uint64_t off_k, off_v;
    row_offsets(tile, pos, off_k, off_v);
    const int buf = tile & (NB - 1);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = wave + i * NW;  // wave-uniform
      if (c < NQ)
        load_to_lds(kseq + off_k + (2 * c + half) * 16, &s_k[buf][c][0]);
      else
        load_to_lds(vseq + off_v + (2 * (c - NQ) + (lane & 1)) * 16, &s_v[buf][c - NQ][0]);
    }
    // lanes 32..63 repeat lanes 0..31 into the slot's second half
    if constexpr (MASK == kMaskKeys)
      __builtin_amdgcn_global_load_lds((const void*)(kbw_row + pos),
                                       (__attribute__((address_space(3))) void*)&s_kbw[buf][wave][0],
                                       4, 0, 0);
  };

  // additive mask row of this lane's column (general mask only)
  const float* mrow = nullptr;
  if (MASK == kMaskFull && col_ok)
    mrow = a.mask + (int64_t)bi * a.msb + (int64_t)(g * a.hg + chead) * a.msh + (int64_t)crow * a.msn;
  constexpr float kLog2e = 1.4426950408889634f;

  WaveState<ND> st;
  st.reset();
  f32x16 s_cur = {};   // S_j
  bf16x8 p_prev[2];    // P_{j-1}
  p_prev[0] = p_prev[1] = bf16x8{};
  bool over = false;

  auto read_k = [&](int buf, u32x4 (&kr)[NQ]) {
#pragma unroll
    for (int c = 0; c < NQ; ++c) kr[c] = s_k[buf][c][lane];
  };
  auto scores_of = [&](const u32x4 (&kr)[NQ], const f32x16& init) {
    f32x16 s = init;
#pragma unroll
    for (int c = 0; c < NQ; ++c) s = mfma_bf16(as_bf16x8(kr[c]), as_bf16x8(qr[c]), s);
    return s;
  };
  // The PV operand V^T (row d, 8 keys per lane) of d block db and keys
  // 16k .. 16k + 15, read transposed from the V rows in LDS: within each
  // group of 16 lanes, a transposing read hands lane 4u + e element e of the
  // 8-byte rows addressed by lanes u, u + 4, u + 8, u + 12.  Lane l addresses
  // key 4 (l / 32) + (l % 16) / 4 (+ 8 for the second read), d 16 ((l / 16)
  // % 2) + 4 (l % 4) of the block, so it receives d = l % 32 and keys
  // 4 (l / 32) + 0..3 and 8 + 4 (l / 32) + 0..3: the key order of the
  // probability operand (registers d_row(r, l / 32)).
  constexpr int kVChunk = sizeof(s_v[0][0]);  // bytes between V chunks
  const int vt_lane = ((lane >> 4) & 1) * kVChunk + (4 * (lane >> 5) + ((lane & 15) >> 2)) * 32 +
                      8 * (lane & 3);
  auto read_vt = [&](int buf, int db, int k) {
    using lds_bf16x4 = __attribute__((address_space(3))) bf16x4;
    auto base = (__attribute__((address_space(3))) char*)&s_v[buf][0][0] + vt_lane +
                db * 2 * kVChunk + k * 512;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)base);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 256));
    return bf16x8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_v = [&](int buf, bf16x8 (&vt)[ND][2]) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int k = 0; k < 2; ++k) vt[d][k] = read_vt(buf, d, k);
  };
  auto pv_of = [&](const bf16x8 (&vt)[ND][2]) {
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      st.o[d] = mfma_bf16(vt[d][0], p_prev[0], st.o[d]);
      st.o[d] = mfma_bf16(vt[d][1], p_prev[1], st.o[d]);
    }
  };
  // Mask values of tile j, register r holding key d_row(r, half), in log2
  // units times `post` (masked kinds only).
  auto load_bias = [&](int j, float (&bias)[16], float post) {
    if constexpr (MASK == kMaskKeys) {
      // keys 8k + 4*half .. +3 of the tile for registers 4k .. 4k+3
      // (read with a wait of its own: behind the next tile's direct-to-LDS
      // loads, the compiler would make the reads wait for those loads)
      f32x4 kb[4];
      const uint32_t addr = (uint32_t)(uintptr_t)(
          (__attribute__((address_space(3))) char*)&s_kbw[j & (NB - 1)][wave][0] + 16 * half);
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %4 offset:32\n\t"
          "ds_read_b128 %2, %4 offset:64\n\t"
          "ds_read_b128 %3, %4 offset:96\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kb[0]), "=&v"(kb[1]), "=&v"(kb[2]), "=&v"(kb[3])
          : "v"(addr)
          : "memory");
      const float mult = kLog2e * post;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[4 * k + e] = kb[k][e] * mult;
    } else if constexpr (MASK == kMaskFull) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jj = j * kTileRows + d_row(r, half);
        bias[r] = (mrow && jj < a.m) ? mrow[jj] * (kLog2e * post) : 0.f;
      }
    }
  };
  // The initial accumulator of tile j's score product.  With a positive
  // scale c (log2 units) the mask enters here as mask / c, so that the
  // folded softmax's c * (s + mask / c) is the masked logit; otherwise the
  // product starts from zero and the softmax adds the mask.
  const float inv_c = FOLD ? 1.0f / a.scale_log2 : 0.f;
  auto score_init = [&](int j) {
    f32x16 init = {};
    if constexpr (FOLD && BIAS) {
      float b[16];
      load_bias(j, b, inv_c);
#pragma unroll
      for (int r = 0; r < 16; ++r) init[r] = b[r];
    }
    return init;
  };
  constexpr bool SM_BIAS = BIAS && !FOLD;  // the softmax adds the mask itself

  // One iteration.  Every iteration runs both products and the softmax (a
  // product under a branch makes the compiler copy the accumulators): a tile
  // past the wave's last goes through the masked softmax with every key
  // hidden, which leaves (m, l, O) unchanged and yields P = 0, so the next PV
  // adds exactly zero; the score product of a tile no one will read is
  // discarded the same way.
  //
  // The iteration's barrier publishes tile j + 1.  The V^T operand of PV of
  // tile j - 1 (tile 0's buffer when j = 0: finite, and P = 0), published by
  // an earlier barrier, is read before it, the K operand of the scores of
  // tile j + 1 after it; the products and the softmax go where the compiler
  // schedules them (keeping PV and the softmax ahead of the barrier measured
  // slower).  Tile j + 3's loads are issued after the iteration's last LDS
  // operand read (the compiler would make any LDS read behind them wait for
  // them).
  auto iter = [&](int j, auto full_tile, auto ref_known) {
    constexpr bool FULL = decltype(full_tile)::value;
    constexpr bool REF = decltype(ref_known)::value;
    // this wave's part of tile j + 1 (issued in iteration j - 2) landed;
    // tile j + 2 may stay in flight
    if (j + 2 < ntiles)
      __builtin_amdgcn_s_waitcnt(0x0F70 | kPerTile);
    else if (j + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(0x0F70);
    bf16x8 vt[ND][2];
    read_v(j == 0 ? 0 : (j - 1) & (NB - 1), vt);
    float bias[16];
    if constexpr (SM_BIAS) load_bias(j, bias, 1.0f);
    pv_of(vt);
    bf16x8 p_cur[2];
    softmax_fixed<ND, FULL, SM_BIAS, FOLD, REF>(st, s_cur, a.scale_log2, j * kTileRows,
                                           j < w_tiles ? lim : -1, half, p_cur, bias, over);
    p_prev[0] = p_cur[0];
    p_prev[1] = p_cur[1];
    if constexpr (FULL) {
      // the LDS operands first, then the MFMAs spread over the vector work
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * ND, 0);
#pragma unroll
      for (int i = 0; i < 2 * ND; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
      }
    }
    lds_barrier();
    u32x4 kr[NQ];
    read_k((j + 1) & (NB - 1), kr);
    // a general mask comes from global memory: loaded before the next tile's
    // loads, since loads complete in order
    f32x16 init;
    if constexpr (MASK == kMaskFull) init = score_init(j + 1);
    if (j + 3 < ntiles) issue_dma(j + 3);
    if constexpr (MASK != kMaskFull) init = score_init(j + 1);
    s_cur = scores_of(kr, init);
    if constexpr (FULL) {
      __builtin_amdgcn_sched_group_barrier(0x100, NQ, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NQ, 0);
    }
  };

  // prologue: tiles 0, 1 and 2 in flight, 0 landed and published, its
  // scores computed
  issue_dma(0);
  if (ntiles > 1) issue_dma(1);
  if (ntiles > 2) issue_dma(2);
  if (ntiles > 2)
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kPerTile));
  else if (ntiles > 1)
    __builtin_amdgcn_s_waitcnt(0x0F70 | kPerTile);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
  lds_barrier();
  {
    u32x4 kr[NQ];
    read_k(0, kr);
    s_cur = scores_of(kr, score_init(0));
  }
  // Tile 0 sets the references.  A wave with a column still without one (a
  // mask hides its first keys) keeps taking tile maxima to the end; the
  // others run the tiles without a maximum.
  iter(0, std::false_type{}, std::false_type{});
  int j = 1;
  if (__builtin_amdgcn_ballot_w64(st.m == kNegInf) != 0)
    for (; j <= ntiles; ++j) iter(j, std::false_type{}, std::false_type{});
  for (; j < j_full; ++j) iter(j, std::true_type{}, std::true_type{});
  for (; j <= ntiles; ++j) iter(j, std::false_type{}, std::true_type{});

  if (__any(over) && lane == 0) s_over = 1;
  __syncthreads();
  if (s_over) {
    // some logit exceeded its column's fixed reference by more than the
    // slack: recompute the workgroup's rows with the rescaling kernel body
    // (its LDS: the K tile buffers for its K and V^T tiles, a V tile buffer
    // for its mask values; every wave is past the loops)
    using RL = RowsLds<T, DH>;
    static_assert(RL::kBytesK + RL::kBytesVt <= sizeof(s_k) && RL::kBytesKb <= sizeof(s_v),
                  "the rescue fits the tile buffers");
    lds_u32x4* const kmem = (lds_u32x4*)&s_k[0][0][0];
    prefill_rows<T, DH, NW, CAUSAL, false, MASK>(a, kmem, kmem + RL::kBytesK / sizeof(u32x4),
                                                 (lds_f32x4*)&s_v[0][0][0]);
    return;
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
constexpr int kPrefillWaves = 8;      // fp32 workgroups
constexpr int kPrefillWavesBf16 = 8;  // bf16 workgroups
template <typename T>
constexpr int prefill_waves() { return sizeof(T) == 2 ? kPrefillWavesBf16 : kPrefillWaves; }

// Row blocks of NW * rpw query rows per (sequence, group).
PrefillArgs row_blocks(const PrefillParams& p, int m, int nw) {
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
  const int rows_per_block = nw * a.rpw;
  a.nrb = (p.n + rows_per_block - 1) / rows_per_block;
  a.scale_log2 = (float)((double)p.scale * 1.4426950408889634);
  return a;
}

// The kernel for element type T: the pipelined one for bf16, the plain one
// (fp32 operands twice as wide) otherwise.
template <typename T, int DH, bool CAUSAL, bool FOLD, int MASK>
void launch_rows(const PrefillArgs& a, dim3 grid, hipStream_t s) {
  constexpr int NW = prefill_waves<T>();
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((prefill_bf16_kernel<DH, NW, CAUSAL, FOLD, MASK>), grid, dim3(NW * 64), 0, s,
                       a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, DH, NW, CAUSAL, FOLD, MASK>), grid, dim3(NW * 64), 0, s,
                       a);
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
  const PrefillArgs a = row_blocks(p, p.n, prefill_waves<T>());
  const dim3 grid((unsigned)((size_t)p.b * p.G * a.nrb));
  if (a.scale_log2 > 0.f)
    launch_rows<T, DH, true, true, kMaskNone>(a, grid, s);
  else
    launch_rows<T, DH, true, false, kMaskNone>(a, grid, s);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t launch_attend_t(const AttendParams& q, hipStream_t s) {
  PrefillArgs a = row_blocks(q.base, q.m, prefill_waves<T>());
  a.mask = q.mask;
  a.msb = q.msb;
  a.msh = q.msh;
  a.msn = q.msn;
  const dim3 grid((unsigned)((size_t)q.base.b * q.base.G * a.nrb));
  const bool fold = a.scale_log2 > 0.f;
  const int kind = !q.mask ? kMaskNone : (q.msh == 0 && q.msn == 0) ? kMaskKeys : kMaskFull;
  if (kind == kMaskNone) {
    if (fold) launch_rows<T, DH, false, true, kMaskNone>(a, grid, s);
    else launch_rows<T, DH, false, false, kMaskNone>(a, grid, s);
  } else if constexpr (sizeof(T) == 2) {
    // bf16: a positive scale folds the mask into the score product too
    if (kind == kMaskKeys) {
      if (fold) launch_rows<T, DH, false, true, kMaskKeys>(a, grid, s);
      else launch_rows<T, DH, false, false, kMaskKeys>(a, grid, s);
    } else {
      if (fold) launch_rows<T, DH, false, true, kMaskFull>(a, grid, s);
      else launch_rows<T, DH, false, false, kMaskFull>(a, grid, s);
    }
  } else {
    if (kind == kMaskKeys) launch_rows<T, DH, false, false, kMaskKeys>(a, grid, s);
    else launch_rows<T, DH, false, false, kMaskFull>(a, grid, s);
  }
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
