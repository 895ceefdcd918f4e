/*
 * mqa_oracle.c -- fp64 reference for MQA/GQA decoding.  TEST INFRASTRUCTURE
 * ONLY (see mqa_oracle.h); the product library never links it.
 *
 * Each function is the plain definition written out, one query row at a time,
 * with no blocking, fusion or reordering:
 *   - scores   S_j = scale * sum_r q_r K_jr    (study notes section 2, score
 *              definition; section 4 per-head MQA formula)
 *   - softmax  w_j = exp(S_j - max S) / sum exp(S - max S)
 *              (study notes section 2, A = softmax(S))
 *   - output   o_r = sum_j w_j V_jr           (study notes section 2, O = AV)
 * Head i reads K/V group g(i) = i / (h/G): one group of query heads shares one
 * K/V head (study notes section 9 table; GQA essay section 3, G=1 is MQA and
 * G=h is MHA).
 */
#include "mqa_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* Widen one stored element to double.  bf16 is the upper half of an IEEE
 * binary32, so the widening is exact. */
static double elem(int dtype, const void* base, int64_t idx) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int elem_size(int dtype) { return dtype == 0 ? 4 : 2; }

static int check_common(int dtype, int b, int h, int G, int dh) {
  if (dtype != 0 && dtype != 1) return ORACLE_EINVAL;
  if (b < 0 || h <= 0 || G <= 0 || dh <= 0) return ORACLE_EINVAL;
  if (h % G != 0) return ORACLE_EINVAL;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ append */

int oracle_kv_append(int dtype, int b, int G, int dh, int m_cap,
                     const void* k_new, const void* v_new, void* K, void* V,
                     int32_t* lens, int32_t* overflow) {
  if (check_common(dtype, b, G, G, dh) != ORACLE_OK || m_cap <= 0) return ORACLE_EINVAL;
  const size_t row = (size_t)G * dh * elem_size(dtype);      /* one position, all groups */
  int32_t over = 0;
  for (int bi = 0; bi < b; ++bi) {
    int32_t p = lens[bi];
    if (p < 0 || p >= m_cap) { ++over; continue; }
    size_t dst = ((size_t)bi * m_cap + (size_t)p) * row;
    memcpy((char*)K + dst, (const char*)k_new + (size_t)bi * row, row);
    memcpy((char*)V + dst, (const char*)v_new + (size_t)bi * row, row);
    lens[bi] = p + 1;
  }
  if (overflow) *overflow = over;
  return ORACLE_OK;
}

/* ----------------------------------------------------------------- reorder */

int oracle_kv_reorder(int dtype, int b, int G, int dh, int m_cap, int beam,
                      const int32_t* parent, void* K, void* V, int32_t* lens,
                      int32_t* bad) {
  if (check_common(dtype, b, G, G, dh) != ORACLE_OK || m_cap <= 0 || beam <= 0 || b % beam != 0)
    return ORACLE_EINVAL;
  const size_t row = (size_t)G * dh * elem_size(dtype);      /* one position, all groups */
  const size_t seq = row * (size_t)m_cap;                     /* one hypothesis */
  /* the cache as it was: every copy reads from here */
  char* K0 = (char*)malloc(seq * (size_t)b);
  char* V0 = (char*)malloc(seq * (size_t)b);
  int32_t* lens0 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(b > 0 ? b : 1));
  if (!K0 || !V0 || !lens0) {
    free(K0);
    free(V0);
    free(lens0);
    return ORACLE_EINVAL;
  }
  memcpy(K0, K, seq * (size_t)b);
  memcpy(V0, V, seq * (size_t)b);
  memcpy(lens0, lens, sizeof(int32_t) * (size_t)b);
  int32_t nbad = 0;
  for (int i = 0; i < b; ++i) {
    const int32_t p = parent[i];
    if (p < 0 || p >= beam) { ++nbad; continue; }
    const int src = (i / beam) * beam + p;
    int32_t L = lens0[src];
    if (L < 0) L = 0;
    if (L > m_cap) L = m_cap;
    memcpy((char*)K + (size_t)i * seq, K0 + (size_t)src * seq, (size_t)L * row);
    memcpy((char*)V + (size_t)i * seq, V0 + (size_t)src * seq, (size_t)L * row);
    lens[i] = lens0[src];
  }
  free(K0);
  free(V0);
  free(lens0);
  if (bad) *bad = nbad;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ decode */

typedef struct {
  int dtype, b, h, G, dh, m_cap, window;
  const void *q, *K, *V;
  const int32_t* lens;
  double scale;
  double* o;
  int64_t row_begin, row_end;  /* flattened (b, i) rows */
} decode_job;

/* Visible range [j0, L) of sequence bi. */
static void visible(const decode_job* J, int bi, int* j0, int* L) {
  int32_t l = J->lens[bi];
  if (l < 0) l = 0;
  if (l > J->m_cap) l = J->m_cap;
  int start = 0;
  if (J->window > 0 && l > J->window) start = l - J->window;
  *j0 = start;
  *L = l;
}

/* Softmax weights of row (bi, i) into w[0 .. L-j0).  Returns the count. */
static int row_weights(const decode_job* J, int bi, int i, double* w) {
  int j0, L;
  visible(J, bi, &j0, &L);
  const int g = i / (J->h / J->G);
  const int64_t qoff = ((int64_t)bi * J->h + i) * J->dh;
  double mx = -INFINITY;
  for (int j = j0; j < L; ++j) {
    const int64_t koff = (((int64_t)bi * J->m_cap + j) * J->G + g) * J->dh;
    double s = 0.0;
    for (int r = 0; r < J->dh; ++r)
      s += elem(J->dtype, J->q, qoff + r) * elem(J->dtype, J->K, koff + r);
    s *= J->scale;
    w[j - j0] = s;
    if (s > mx) mx = s;
  }
  double z = 0.0;
  for (int j = j0; j < L; ++j) {
    w[j - j0] = exp(w[j - j0] - mx);
    z += w[j - j0];
  }
  for (int j = j0; j < L; ++j) w[j - j0] /= z;
  return L - j0;
}

static void* decode_worker(void* arg) {
  decode_job* J = (decode_job*)arg;
  double* w = (double*)malloc(sizeof(double) * (size_t)(J->m_cap > 0 ? J->m_cap : 1));
  for (int64_t r = J->row_begin; r < J->row_end; ++r) {
    const int bi = (int)(r / J->h), i = (int)(r % J->h);
    const int g = i / (J->h / J->G);
    double* out = J->o + r * J->dh;
    for (int d = 0; d < J->dh; ++d) out[d] = 0.0;
    int j0, L;
    visible(J, bi, &j0, &L);
    if (L - j0 <= 0) continue;               /* empty row: zeros by convention */
    row_weights(J, bi, i, w);
    for (int d = 0; d < J->dh; ++d) {
      double acc = 0.0;
      for (int j = j0; j < L; ++j) {
        const int64_t voff = (((int64_t)bi * J->m_cap + j) * J->G + g) * J->dh;
        acc += w[j - j0] * elem(J->dtype, J->V, voff + d);
      }
      out[d] = acc;
    }
  }
  free(w);
  return NULL;
}

static void run_jobs(void* (*fn)(void*), void* jobs, size_t job_size, int nthreads) {
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  char* ok = (char*)calloc((size_t)nthreads, 1);
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, fn, (char*)jobs + (size_t)t * job_size) == 0) ok[t] = 1;
    else fn((char*)jobs + (size_t)t * job_size);   /* no thread: run inline */
  }
  fn(jobs);
  for (int t = 1; t < nthreads; ++t)
    if (ok[t]) pthread_join(th[t], NULL);
  free(ok);
  free(th);
}

int oracle_decode(int dtype, int b, int h, int G, int dh, int m_cap,
                  const void* q, const void* K, const void* V,
                  const int32_t* lens, double scale, int window,
                  double* o, int nthreads) {
  if (check_common(dtype, b, h, G, dh) != ORACLE_OK || m_cap < 0) return ORACLE_EINVAL;
  const int64_t rows = (int64_t)b * h;
  if (rows == 0) return ORACLE_OK;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = (int)rows;
  decode_job* jobs = (decode_job*)calloc((size_t)nthreads, sizeof(decode_job));
  for (int t = 0; t < nthreads; ++t) {
    decode_job* J = &jobs[t];
    J->dtype = dtype; J->b = b; J->h = h; J->G = G; J->dh = dh; J->m_cap = m_cap;
    J->window = window; J->q = q; J->K = K; J->V = V; J->lens = lens;
    J->scale = scale; J->o = o;
    J->row_begin = rows * t / nthreads;
    J->row_end = rows * (t + 1) / nthreads;
  }
  run_jobs(decode_worker, jobs, sizeof(decode_job), nthreads);
  free(jobs);
  return ORACLE_OK;
}

int oracle_decode_weights(int dtype, int b, int h, int G, int dh, int m_cap,
                          const void* q, const void* K, const void* V,
                          const int32_t* lens, double scale, int window,
                          int bi, int i, double* w) {
  if (check_common(dtype, b, h, G, dh) != ORACLE_OK) return ORACLE_EINVAL;
  if (bi < 0 || bi >= b || i < 0 || i >= h) return ORACLE_EINVAL;
  decode_job J;
  memset(&J, 0, sizeof J);
  J.dtype = dtype; J.b = b; J.h = h; J.G = G; J.dh = dh; J.m_cap = m_cap;
  J.window = window; J.q = q; J.K = K; J.V = V; J.lens = lens; J.scale = scale;
  int j0, L;
  visible(&J, bi, &j0, &L);
  if (L - j0 <= 0) return 0;
  return row_weights(&J, bi, i, w);
}

/* ----------------------------------------------------------------- prefill */

typedef struct {
  int dtype, b, n, h, G, dh;
  const void *Q, *K, *V;
  double scale;
  const int64_t* rows;
  int64_t r_begin, r_end;
  double* O;
} prefill_job;

static void* prefill_worker(void* arg) {
  prefill_job* J = (prefill_job*)arg;
  double* x = (double*)malloc(sizeof(double) * (size_t)J->n);
  for (int64_t k = J->r_begin; k < J->r_end; ++k) {
    const int64_t r = J->rows ? J->rows[k] : k;
    const int bi = (int)(r / J->n), t = (int)(r % J->n);
    for (int i = 0; i < J->h; ++i) {
      const int g = i / (J->h / J->G);
      const int64_t qoff = (((int64_t)bi * J->n + t) * J->h + i) * J->dh;
      /* logits + additive causal mask over the FULL row of n keys */
      double mx = -INFINITY;
      for (int j = 0; j < J->n; ++j) {
        const int64_t koff = (((int64_t)bi * J->n + j) * J->G + g) * J->dh;
        double s = 0.0;
        for (int r2 = 0; r2 < J->dh; ++r2)
          s += elem(J->dtype, J->Q, qoff + r2) * elem(J->dtype, J->K, koff + r2);
        s *= J->scale;
        const double mask = (j > t) ? -INFINITY : 0.0;
        x[j] = s + mask;
        if (x[j] > mx) mx = x[j];
      }
      double z = 0.0;
      for (int j = 0; j < J->n; ++j) {
        x[j] = exp(x[j] - mx);                 /* exp(-inf) = 0 */
        z += x[j];
      }
      double* out = J->O + (k * J->h + i) * J->dh;
      for (int d = 0; d < J->dh; ++d) {
        double acc = 0.0;
        for (int j = 0; j < J->n; ++j) {
          const int64_t voff = (((int64_t)bi * J->n + j) * J->G + g) * J->dh;
          acc += (x[j] / z) * elem(J->dtype, J->V, voff + d);
        }
        out[d] = acc;
      }
    }
  }
  free(x);
  return NULL;
}

int oracle_prefill(int dtype, int b, int n, int h, int G, int dh,
                   const void* Q, const void* K, const void* V, double scale,
                   const int64_t* rows, int64_t nrows, double* O, int nthreads) {
  if (check_common(dtype, b, h, G, dh) != ORACLE_OK || n <= 0) return ORACLE_EINVAL;
  const int64_t total = rows ? nrows : (int64_t)b * n;
  if (rows)
    for (int64_t k = 0; k < nrows; ++k)
      if (rows[k] < 0 || rows[k] >= (int64_t)b * n) return ORACLE_EINVAL;
  if (total == 0) return ORACLE_OK;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > total) nthreads = (int)total;
  prefill_job* jobs = (prefill_job*)calloc((size_t)nthreads, sizeof(prefill_job));
  for (int t = 0; t < nthreads; ++t) {
    prefill_job* J = &jobs[t];
    J->dtype = dtype; J->b = b; J->n = n; J->h = h; J->G = G; J->dh = dh;
    J->Q = Q; J->K = K; J->V = V; J->scale = scale; J->rows = rows; J->O = O;
    J->r_begin = total * t / nthreads;
    J->r_end = total * (t + 1) / nthreads;
  }
  run_jobs(prefill_worker, jobs, sizeof(prefill_job), nthreads);
  free(jobs);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ attend */

typedef struct {
  int dtype, b, n, m, h, G, dh;
  const void *Q, *K, *V;
  const float* mask;
  int64_t sb, sh, sn;
  double scale;
  const int64_t* rows;
  int64_t r_begin, r_end;
  double* O;
} attend_job;

static void* attend_worker(void* arg) {
  attend_job* J = (attend_job*)arg;
  double* x = (double*)malloc(sizeof(double) * (size_t)J->m);
  for (int64_t k = J->r_begin; k < J->r_end; ++k) {
    const int64_t r = J->rows ? J->rows[k] : k;
    const int bi = (int)(r / J->n), t = (int)(r % J->n);
    for (int i = 0; i < J->h; ++i) {
      const int g = i / (J->h / J->G);
      const int64_t qoff = (((int64_t)bi * J->n + t) * J->h + i) * J->dh;
      /* logits + additive mask over the whole memory */
      double mx = -INFINITY;
      for (int j = 0; j < J->m; ++j) {
        const int64_t koff = (((int64_t)bi * J->m + j) * J->G + g) * J->dh;
        double s = 0.0;
        for (int r2 = 0; r2 < J->dh; ++r2)
          s += elem(J->dtype, J->Q, qoff + r2) * elem(J->dtype, J->K, koff + r2);
        s *= J->scale;
        if (J->mask) s += (double)J->mask[bi * J->sb + i * J->sh + t * J->sn + j];
        x[j] = s;
        if (x[j] > mx) mx = x[j];
      }
      double* out = J->O + (k * J->h + i) * J->dh;
      if (mx == -INFINITY) {                   /* every key hidden: zeros */
        for (int d = 0; d < J->dh; ++d) out[d] = 0.0;
        continue;
      }
      double z = 0.0;
      for (int j = 0; j < J->m; ++j) {
        x[j] = exp(x[j] - mx);                 /* exp(-inf) = 0 */
        z += x[j];
      }
      for (int d = 0; d < J->dh; ++d) {
        double acc = 0.0;
        for (int j = 0; j < J->m; ++j) {
          const int64_t voff = (((int64_t)bi * J->m + j) * J->G + g) * J->dh;
          acc += (x[j] / z) * elem(J->dtype, J->V, voff + d);
        }
        out[d] = acc;
      }
    }
  }
  free(x);
  return NULL;
}

int oracle_attend(int dtype, int b, int n, int m, int h, int G, int dh,
                  const void* Q, const void* K, const void* V, double scale,
                  const float* mask, int64_t sb, int64_t sh, int64_t sn,
                  const int64_t* rows, int64_t nrows, double* O, int nthreads) {
  if (check_common(dtype, b, h, G, dh) != ORACLE_OK || n <= 0 || m <= 0) return ORACLE_EINVAL;
  if (mask && (sb < 0 || sh < 0 || sn < 0)) return ORACLE_EINVAL;
  const int64_t total = rows ? nrows : (int64_t)b * n;
  if (rows)
    for (int64_t k = 0; k < nrows; ++k)
      if (rows[k] < 0 || rows[k] >= (int64_t)b * n) return ORACLE_EINVAL;
  if (total == 0) return ORACLE_OK;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > total) nthreads = (int)total;
  attend_job* jobs = (attend_job*)calloc((size_t)nthreads, sizeof(attend_job));
  for (int t = 0; t < nthreads; ++t) {
    attend_job* J = &jobs[t];
    J->dtype = dtype; J->b = b; J->n = n; J->m = m; J->h = h; J->G = G; J->dh = dh;
    J->Q = Q; J->K = K; J->V = V; J->scale = scale; J->rows = rows; J->O = O;
    J->mask = mask; J->sb = sb; J->sh = sh; J->sn = sn;
    J->r_begin = total * t / nthreads;
    J->r_end = total * (t + 1) / nthreads;
  }
  run_jobs(attend_worker, jobs, sizeof(attend_job), nthreads);
  free(jobs);
  return ORACLE_OK;
}
