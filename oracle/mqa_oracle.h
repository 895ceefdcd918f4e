/*
 * mqa_oracle.h -- plain, slow, fp64 CPU oracle for Multi-Query / Grouped-Query
 * attention decoding.  TEST INFRASTRUCTURE ONLY: nothing on the product path
 * may include, link or call this file.  It shares no code with the HIP library.
 *
 * What it computes (sources: the Shazeer 2019 study notes, section 1 causal
 * attention formula and section 4 per-head MQA formula; the paper review's
 * section 3 incremental multi-query pseudocode and section 2.3 batched
 * pseudocode with an additive mask; the GQA essay's section 3 grouping):
 *
 *   decode : o[b,i,:] = sum_j softmax_j(scale * q[b,i,:].K[b,j,g(i),:]) V[b,j,g(i),:]
 *            over the cached positions j < L_b, with g(i) = i / (h/G)
 *   prefill: O[b,t,i,:] = softmax over all j of (scale * Q[b,t,i,:].K[b,j,g(i),:] + M_tj)
 *            applied to V, with M_tj = 0 for j <= t and -inf for j > t
 *   append : the concatenation of one new K/V row per sequence onto the cache
 *
 * Element storage: dtype 0 = IEEE fp32, dtype 1 = bfloat16 held as raw 16-bit
 * patterns.  Every input element is widened exactly to double; every sum is a
 * plain fp64 sum in index order.
 *
 * Layouts (row-major, innermost last):
 *   q, o          [b][h][dh]
 *   K, V cache    [b][m_cap][G][dh]
 *   k_new, v_new  [b][G][dh]
 *   lens          int32 [b]
 *   Q, O prefill  [b][n][h][dh];  K, V prefill [b][n][G][dh]
 *   attend: Q, O [b][n][h][dh]; K, V memory [b][m][G][dh]
 */
#ifndef MQA_ORACLE_H
#define MQA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* Concatenate one row per sequence onto the cache (the incremental concat of
 * the paper review, section 3).  Sequences whose cache is already full
 * (lens[b] >= m_cap) are left untouched and counted in *overflow. */
int oracle_kv_append(int dtype, int b, int G, int dh, int m_cap,
                     const void* k_new, const void* v_new, void* K, void* V,
                     int32_t* lens, int32_t* overflow);

/* Beam reorder of the cache.  Beam search over the incremental decoder (the
 * study notes' section 6.2 beam-4 measurements) keeps `beam` hypotheses per
 * source; before a step every hypothesis continues one hypothesis of its own
 * source and inherits its cache.  The pages do not spell the mechanics out;
 * the reading taken: the b cache rows form b / beam groups of `beam`
 * consecutive hypotheses and, with src(i) = (i / beam) * beam + parent[i],
 *   K'[i, j] = K[src(i), j] and V'[i, j] = V[src(i), j] for j < L(src(i)),
 *   lens'[i] = lens[src(i)],
 * all read from the cache as it was before the call (L = lens clamped to
 * [0, m_cap]).  Positions j >= L(src(i)) of row i keep their contents.  A
 * parent outside [0, beam) leaves row i and lens[i] as they were and is
 * counted in *bad. */
int oracle_kv_reorder(int dtype, int b, int G, int dh, int m_cap, int beam,
                      const int32_t* parent, void* K, void* V, int32_t* lens,
                      int32_t* bad);

/* One decode step over the cache.  L_b = clamp(lens[b], 0, m_cap).  window > 0
 * restricts the visible positions to the last `window` ones (local attention,
 * study notes section 6.4); window <= 0 means all of them.  An empty row
 * (L_b == 0) yields zeros.  o is fp64 [b][h][dh]. */
int oracle_decode(int dtype, int b, int h, int G, int dh, int m_cap,
                  const void* q, const void* K, const void* V,
                  const int32_t* lens, double scale, int window,
                  double* o, int nthreads);

/* The softmax weights of one decode row (b, i): w[j] for j < L_b (window
 * applied).  Returns the number of weights written, or ORACLE_EINVAL. */
int oracle_decode_weights(int dtype, int b, int h, int G, int dh, int m_cap,
                          const void* q, const void* K, const void* V,
                          const int32_t* lens, double scale, int window,
                          int bi, int i, double* w);

/* Causal prefill through the full masked row.  rows lists flattened (b, t)
 * indices r = b*n + t to evaluate (NULL: all b*n rows, in order); O receives
 * [nrows][h][dh] in fp64. */
int oracle_prefill(int dtype, int b, int n, int h, int G, int dh,
                   const void* Q, const void* K, const void* V, double scale,
                   const int64_t* rows, int64_t nrows, double* O, int nthreads);

/* Attention of n queries per sequence over a fixed memory of m positions,
 * with no causal structure and an optional additive mask (the paper review's
 * section 2.3 batched pseudocode: softmax(logits + mask) over the memory
 * axis; the study notes' section 6.1: multi-query attention also serves
 * encoder-decoder attention):
 *   x_j = scale * Q[b,t,i,:].K[b,j,g(i),:] + mask[b*sb + i*sh + t*sn + j],  j < m
 *   O[b,t,i,:] = sum_j softmax(x)_j V[b,j,g(i),:]
 * Q [b][n][h][dh]; K, V [b][m][G][dh]; mask fp32 (NULL: none); a row whose
 * every x_j is -inf yields zeros.  rows / nrows / O as in oracle_prefill. */
int oracle_attend(int dtype, int b, int n, int m, int h, int G, int dh,
                  const void* Q, const void* K, const void* V, double scale,
                  const float* mask, int64_t sb, int64_t sh, int64_t sn,
                  const int64_t* rows, int64_t nrows, double* O, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
