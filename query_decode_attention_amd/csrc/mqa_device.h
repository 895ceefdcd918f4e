// mqa_device.h -- device-side building blocks shared by the gfx950 kernels of
// libmqa: vector types, the CDNA4 matrix-core (MFMA) operations used by the
// decode and prefill kernels, and small wavefront utilities.
//
// MFMA operand layouts relied upon (32x32 output family, wave64):
//   * A operand (M x K): lane l supplies row m = l % 32 and a group of
//     consecutive-in-register K elements selected by the lane half l / 32.
//   * B operand (K x N): lane l supplies column n = l % 32, K elements selected
//     by l / 32 exactly as for A.  Because A and B share that (half, element)
//     -> k pairing, any consistent assignment of the contraction index to
//     (half, element) gives the same product; the kernels use this freedom to
//     feed rows read straight from memory.
//   * D (32 x 32 fp32, 16 values per lane): lane l holds column n = l % 32 and
//     rows 8*(r/4) + 4*(l/32) + (r%4) for register r = 0..15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

// Row index (within a 32-row MFMA tile) held by D register r of lane half hf.
__device__ __forceinline__ constexpr int d_row(int r, int hf) {
  return 8 * (r >> 2) + 4 * hf + (r & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// 16 bytes per lane from `src` straight into LDS word `lane` of `dst` (the
// direct-to-LDS load path; the LDS base must be the same for the whole wave).
// Completion is counted by vmcnt.
__device__ __forceinline__ void load_to_lds(const char* src, u32x4* dst) {
  __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst,
                                   16, 0, 0);
}

// Combine a value with the one held by lane ^ 32, through one cross-half
// swap (v_permlane32_swap: each lane receives the values of lanes l % 32 and
// l % 32 + 32, in that order, so both halves compute the same result).
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- bf16 <-> u32x4 bit casts -------------------------------------------------
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round 8 fp32 values to bf16 (round-to-nearest-even) and pack them.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// ---- MFMA wrappers -------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---- element traits ------------------------------------------------------------
template <typename T> struct Elt;
template <> struct Elt<__bf16> {
  static constexpr int kPer16B = 8;
};
template <> struct Elt<float> {
  static constexpr int kPer16B = 4;
};

// Store 4 consecutive output elements converted from fp32.
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

// ---- one 32-row tile of attention, shared by decode and prefill ---------------
//
// A wave holds 32 "columns" (query vectors: the h/G heads of a group for
// decode; (row, head) pairs for prefill) and consumes key/value positions
// 32 at a time.

template <typename T, int DH>
struct TileShape {
  static constexpr int kChunks = DH * (int)sizeof(T) / 16;  // 16-byte chunks per row
  static constexpr int NQ = kChunks / 2;                    // chunks held per lane
  static constexpr int ND = DH / 32;                        // 32-wide column blocks of d
  static constexpr int VTC = sizeof(T) == 2 ? 2 : 4;        // u32x4 per lane per PV A block
};

// Per-wave running softmax state.
template <int ND>
struct WaveState {
  f32x16 o[ND];  // O^T: lane (column n, half j), reg r -> d = 32*blk + d_row(r, j)
  float m;       // running max of scaled logits (log2 domain), equal in both halves
  float l;       // running sum of exp2(logit - m) over this lane half's rows
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x16{};
    m = kNegInf;
    l = 0.f;
  }
};

// S^T[32 positions][32 columns] = rows . cols^T, both operands given as this
// lane's 16-byte chunks (2c + half) of its row / column vector.
template <typename T, int NQ>
__device__ __forceinline__ f32x16 tile_scores(const u32x4 (&kr)[NQ], const u32x4 (&qr)[NQ]) {
  f32x16 s = {};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < NQ; ++c) s = mfma_bf16(as_bf16x8(kr[c]), as_bf16x8(qr[c]), s);
  } else {
#pragma unroll
    for (int c = 0; c < NQ; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = mfma_f32(__uint_as_float(kr[c][e]), __uint_as_float(qr[c][e]), s);
  }
  return s;
}

// 0/1 selection operands that move a position-major V block into the
// d-major layout PV needs: D = V_block . Sel has D[pos][n] = V[pos][32*blk + n].
// The products are x*1 and x*0 summed in fp32, so the result is exact.
template <typename T> struct SelOps;
template <> struct SelOps<__bf16> {
  bf16x8 s[2];
  __device__ __forceinline__ void init(int n, int half) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[a][e] = (__bf16)((n == 16 * a + 8 * half + e) ? 1.0f : 0.0f);
  }
  // Keeps the set-up where it is written, after the memory requests before
  // it (the compiler would otherwise sink it to the first use).
  __device__ __forceinline__ void pin() { asm volatile("" : "+v"(s[0]), "+v"(s[1]) : : "memory"); }
};
template <> struct SelOps<float> {
  float s[4][4];
  __device__ __forceinline__ void init(int n, int half) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[a][e] = (n == 8 * a + 4 * half + e) ? 1.0f : 0.0f;
  }
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(s[a][e]) : : "memory");
  }
};

// Transpose 32-wide d block `blk` of this lane's V chunks into PV A operands.
template <typename T, int NQ>
__device__ __forceinline__ void transpose_block(const u32x4 (&vr)[NQ], int blk,
                                                const SelOps<T>& sel,
                                                u32x4 (&ops)[sizeof(T) == 2 ? 2 : 4]) {
  f32x16 vt = {};
  if constexpr (sizeof(T) == 2) {
    vt = mfma_bf16(as_bf16x8(vr[2 * blk]), sel.s[0], vt);
    vt = mfma_bf16(as_bf16x8(vr[2 * blk + 1]), sel.s[1], vt);
    ops[0] = __builtin_bit_cast(u32x4, pack_bf16x8(vt[0], vt[1], vt[2], vt[3], vt[4], vt[5],
                                                   vt[6], vt[7]));
    ops[1] = __builtin_bit_cast(u32x4, pack_bf16x8(vt[8], vt[9], vt[10], vt[11], vt[12], vt[13],
                                                   vt[14], vt[15]));
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) vt = mfma_f32(__uint_as_float(vr[4 * blk + a][e]), sel.s[a][e], vt);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      ops[k] = u32x4{__float_as_uint(vt[4 * k]), __float_as_uint(vt[4 * k + 1]),
                     __float_as_uint(vt[4 * k + 2]), __float_as_uint(vt[4 * k + 3])};
  }
}

// The P^T operand of one tile: the unnormalised probabilities of this lane's
// 16 positions (rows d_row(r, half) of the tile), bf16-packed for bf16 inputs.
template <typename T>
struct ProbTile;
template <> struct ProbTile<__bf16> {
  bf16x8 pb[2];
};
template <> struct ProbTile<float> {
  float pf[16];
};

// Weighted-V products of one d block: o += V_block^T . P^T.
template <typename T>
struct PvOps;
template <> struct PvOps<__bf16> {
  bf16x8 pb[2];
  __device__ __forceinline__ void set(const ProbTile<__bf16>& pt) {
    pb[0] = pt.pb[0];
    pb[1] = pt.pb[1];
  }
  __device__ __forceinline__ f32x16 apply(const u32x4 (&ops)[2], f32x16 o) const {
    o = mfma_bf16(as_bf16x8(ops[0]), pb[0], o);
    return mfma_bf16(as_bf16x8(ops[1]), pb[1], o);
  }
};
template <> struct PvOps<float> {
  float pf[16];
  __device__ __forceinline__ void set(const ProbTile<float>& pt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r] = pt.pf[r];
  }
  __device__ __forceinline__ f32x16 apply(const u32x4 (&ops)[4], f32x16 o) const {
#pragma unroll
    for (int u = 0; u < 16; ++u) o = mfma_f32(__uint_as_float(ops[u >> 2][u & 3]), pf[u], o);
    return o;
  }
};

// Online-softmax step: scale the raw scores, add the additive mask `bias`
// (already in log2 units) when BIAS, mask positions beyond this lane's limit
// (pos > lim) unless FULL, update (m, l), rescale o when needed, and return
// the unnormalised probabilities p = exp2(logit - m) as the PV operand.  For
// bf16 the probabilities are rounded to bf16 and the normaliser l sums
// exactly the rounded values the PV product uses.
//
// FOLD (requires scale_log2 > 0 and no bias): the max is taken over the raw
// scores and scaled once, and each probability is exp2(fma(s, scale, -m)).
//
// The reference m may lag the true running max: it is raised (and o, l
// rescaled) only when some column's tile max exceeds it by more than
// kRescaleSlack, so after the first tile the rescale is rare.  p is then at
// most 2^kRescaleSlack, far inside fp32 range, and o and l always share the
// same reference, so o / l is unchanged.
constexpr float kRescaleSlack = 8.0f;

// SWAP: the cross-half max uses v_permlane32_swap instead of an LDS
// permute (faster in the compute-bound prefill; the memory-bound decode
// measured slower with it at long context, so it keeps the permute).
template <typename T, int ND, bool FULL, bool BIAS = false, bool FOLD = false, bool SWAP = false>
__device__ __forceinline__ void softmax_tile(WaveState<ND>& st, const f32x16& s, float scale_log2,
                                             int pos0, int lim, int half, ProbTile<T>& pt,
                                             const float* bias = nullptr) {
  static_assert(!(FOLD && BIAS), "the folded form has no bias");
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    x[r] = FOLD ? s[r] : s[r] * scale_log2;
    if constexpr (BIAS) x[r] += bias[r];
    if (!FULL && pos0 + d_row(r, half) > lim) x[r] = kNegInf;
  }
  float mt = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
  mt = SWAP ? max_halves(mt) : fmaxf(mt, xor32(mt));
  if constexpr (FOLD) mt *= scale_log2;  // -inf stays -inf (scale_log2 > 0)
  // st.m == -inf (nothing visible yet) compares as -inf + slack = -inf, so
  // the first visible position always raises it.
  if (__any(mt > st.m + kRescaleSlack)) {
    const float m_new = fmaxf(st.m, mt);
    // A column with no visible position yet keeps m = -inf; use 0 as the
    // reference so exp2 sees -inf - 0 (= 0) and never -inf - (-inf).
    const float alpha = fast_exp2(st.m - (m_new == kNegInf ? 0.f : m_new));
#pragma unroll
    for (int d = 0; d < ND; ++d) st.o[d] *= alpha;
    st.l *= alpha;
    st.m = m_new;
  }
  const float ref = (st.m == kNegInf) ? 0.f : st.m;
  float e[16];
#pragma unroll
  for (int r = 0; r < 16; ++r)
    e[r] = fast_exp2(FOLD ? __builtin_fmaf(x[r], scale_log2, -ref) : x[r] - ref);
  float psum = 0.f;
  if constexpr (sizeof(T) == 2) {
    pt.pb[0] = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    pt.pb[1] = pack_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
    // the rounded values, widened back exactly (bf16 is the top half of fp32)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32x4 w = __builtin_bit_cast(u32x4, pt.pb[k]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        psum += __uint_as_float(w[i] << 16) + __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pt.pf[r] = e[r];
      psum += e[r];
    }
  }
  st.l += psum;
}

}  // namespace mqa
