/*
 * mqa.h -- C ABI of libmqa.so: Multi-Query / Grouped-Query attention
 * incremental decoding on AMD Instinct MI355X (gfx950).
 *
 * The operation (Shazeer 2019, "Fast Transformer Decoding: One Write-Head is
 * All You Need"; the study notes' section 4 formula and the paper review's
 * section 3 multi-query incremental pseudocode): every query head i of a
 * sequence attends, with its own query vector, over ONE key/value head shared
 * by all heads -- or, in the grouped generalisation (GQA essay, section 3),
 * over the K/V head of its group g(i) = i / (h/G); G = 1 is MQA, G = h is
 * MHA.  Each decode step appends one new K/V row per sequence to a growing
 * cache and re-reads the whole cache once.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller.  The library allocates nothing and keeps no state beyond
 *     a per-device cache of the compute-unit count and the fixed scratch array
 *     of mqa_decode_noalloc.
 *   - Layouts are dense and row-major; the head dimension d_h is innermost and
 *     contiguous.  Every tensor pointer must be 16-byte aligned.
 *   - q, o, Q, O, k_new, v_new and the cache share one element type
 *     (mqa_dtype); accumulation is fp32 throughout.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *     is asynchronous on that stream and never synchronises, except
 *     mqa_check_lens.
 *   - Return value: MQA_OK (0) or a negative mqa_status.  Argument errors are
 *     detected on the host before anything is enqueued; nothing is launched
 *     when an error is returned.  Conditions that live in device memory
 *     (lens values) cannot be reported without a synchronisation and are
 *     handled as documented per call.
 *   - Supported: d_h in {64, 128}; heads per group h/G <= 32; G divides h.
 */
#ifndef MQA_H
#define MQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MQA_F32 = 0, MQA_BF16 = 1 } mqa_dtype;

typedef enum {
  MQA_OK = 0,
  MQA_ERR_NULL = -1,      /* a required pointer is NULL                            */
  MQA_ERR_SHAPE = -2,     /* b/n/h/G/m_cap out of range, G does not divide h, h/G>32 */
  MQA_ERR_DHEAD = -3,     /* d_h not in {64, 128}                                  */
  MQA_ERR_ALIGN = -4,     /* a tensor pointer is not 16-byte aligned               */
  MQA_ERR_WORKSPACE = -5, /* workspace missing, misaligned or smaller than needed  */
  MQA_ERR_LAUNCH = -6,    /* the HIP runtime refused a launch / query              */
  MQA_ERR_DTYPE = -7,     /* unknown mqa_dtype                                     */
  MQA_ERR_LENS = -8       /* mqa_check_lens: some lens[b] outside [0, m_cap]       */
} mqa_status;

/* A preallocated, growing K/V cache.  k and v each hold [b][m_cap][G][d_h]
 * elements of `dtype`; row (b, p, g) is d_h contiguous elements.  The number
 * of valid positions of sequence b lives in a separate device int32 lens[b]. */
typedef struct {
  void* k;
  void* v;
  int32_t b;      /* sequences                          */
  int32_t m_cap;  /* capacity in positions per sequence */
  int32_t G;      /* K/V heads (groups)                 */
  int32_t d_h;    /* head dimension                     */
  int32_t dtype;  /* mqa_dtype                          */
} mqa_cache;

/* mqa_kv_append -- the incremental concat of one new K/V row per sequence
 * (paper review, section 3: new_K = concat(prev_K, k), new_V likewise).
 *   k_new, v_new : device [b][G][d_h], cache dtype.
 *   lens         : device int32 [b], read and updated in place:
 *                  K[b, lens[b], :, :] = k_new[b]; V likewise; lens[b] += 1.
 *   err_flag     : optional device int32; a sequence whose cache is full
 *                  (lens[b] >= m_cap) or whose lens[b] < 0 is left untouched
 *                  and *err_flag is set to 1 (never cleared by the library).
 * The copy is bit-exact.  Call it BEFORE mqa_decode: the new token attends to
 * itself, as in the pseudocode where the concat precedes the logits. */
int mqa_kv_append(const void* k_new, const void* v_new, const mqa_cache* cache,
                  int32_t* lens, int32_t* err_flag, void* stream);

/* mqa_kv_reorder -- the cache reorder of beam decoding (the study notes'
 * section 6.2 reports beam-4 decoding; the pages do not spell out its
 * mechanics, and this is the plainest reading): the cache->b rows form
 * cache->b / beam groups of `beam` consecutive hypotheses, and before a step
 * every hypothesis i continues hypothesis src(i) = (i / beam) * beam +
 * parent[i] of its own group:
 *     K[i, j] = K[src(i), j], V[i, j] = V[src(i), j] for j < L(src(i)),
 *     lens[i] = lens[src(i)],
 * all read as they were before the call (L = lens clamped to [0, m_cap]).
 * Positions at or past L(src(i)) of row i keep their contents; a row whose
 * parent is itself is not touched.  In place: no second cache.
 *   lens     : device int32 [b], read and rewritten.
 *   parent   : device int32 [b], beam-local indices in [0, beam).  A parent
 *              outside that range leaves row i and lens[i] as they were and
 *              sets *err_flag (optional device int32) to 1.
 *   beam     : 1 .. 16, dividing cache->b (else MQA_ERR_SHAPE).
 * Two launches on `stream` (rows, then lens).  The copy is bit-exact.  A beam
 * step is mqa_kv_reorder followed by mqa_append_decode. */
int mqa_kv_reorder(const mqa_cache* cache, int32_t* lens, const int32_t* parent, int32_t beam,
                   int32_t* err_flag, void* stream);

/* mqa_kv_reorder_to -- mqa_kv_reorder with the permuted lengths written to a
 * separate array: lens_out[i] = lens_in[src(i)] (lens_out[i] = lens_in[i]
 * for a bad parent), K and V rows reordered in place exactly as above.
 * lens_in is only read, so one launch suffices; a beam loop alternates two
 * lens arrays (reorder from one into the other, then mqa_append_decode on
 * the other).  lens_out must not overlap lens_in (equal pointers:
 * MQA_ERR_SHAPE); other arguments and errors as for mqa_kv_reorder. */
int mqa_kv_reorder_to(const mqa_cache* cache, const int32_t* lens_in, int32_t* lens_out,
                      const int32_t* parent, int32_t beam, int32_t* err_flag, void* stream);

/* Bytes of device workspace a decode needs for `h` query heads over `cache`:
 * a small schedule header (b + 1 ints) followed by the split-K partial
 * results.  Depends only on the shapes, never on the device or on lens.
 * Returns 0 when the arguments are invalid. */
size_t mqa_decode_workspace_size(int32_t h, const mqa_cache* cache);

/* mqa_decode -- one decode step (study notes section 4:
 * o_i = softmax(q_i K^T * scale) V; paper review section 3 einsums
 * "bhk,bmk->bhm", softmax, "bhm,bmv->bhv").  Two kernel launches: the
 * split-K attention, then the exact merge of segments it split; one launch
 * when the cache holds at most 8 tiles of 32 positions (m_cap <= 256),
 * where every sequence is kept whole in one workgroup.
 *   q      : device [b][h][d_h].
 *   lens   : device int32 [b] (read only); sequence b attends over positions
 *            [max(0, L - window), L) with L = clamp(lens[b], 0, m_cap).
 *            Positions at or beyond L are never read.  L == 0 gives o = 0.
 *   scale  : logit multiplier (1/sqrt(d_h) in the study notes; the paper
 *            review's pseudocode uses 1).
 *   window : 0 = attend over the whole cache; w > 0 = local attention over the
 *            last w positions (study notes section 6.4: current + 31 previous
 *            is w = 32).
 *   o      : device [b][h][d_h], written.
 *   workspace, ws_bytes : device scratch of >= mqa_decode_workspace_size()
 *            bytes, 16-byte aligned; needs no initialisation; clobbered.
 *            Calls that share a workspace must be ordered (same stream, or
 *            synchronised). */
int mqa_decode(const void* q, int32_t h, const mqa_cache* cache, const int32_t* lens,
               float scale, int32_t window, void* o, void* workspace, size_t ws_bytes,
               void* stream);

/* mqa_append_decode -- mqa_kv_append followed by mqa_decode with identical
 * results, but without the separate append launch (the attention kernel
 * reads the new row and stores it into the cache): sequence b attends over its cache
 * plus the new row (k_new[b], v_new[b]) at position lens[b]; the new row is
 * stored into the cache and lens[b] is incremented.  A sequence whose cache
 * is full (lens[b] >= m_cap) or whose lens[b] < 0 gets no new row, keeps its
 * lens, attends over clamp(lens[b], 0, m_cap) positions, and sets *err_flag
 * (optional) to 1. */
int mqa_append_decode(const void* q, const void* k_new, const void* v_new, int32_t h,
                      const mqa_cache* cache, int32_t* lens, int32_t* err_flag, float scale,
                      int32_t window, void* o, void* workspace, size_t ws_bytes, void* stream);

/* mqa_decode_ex -- the general form of the two calls above.  k_new / v_new
 * NULL selects mqa_decode, non-NULL selects mqa_append_decode.  ev_begin /
 * ev_end are optional hipEvent_t handles (NULL = skip) recorded on `stream`
 * immediately before and after the decode kernel, so a caller can time that
 * kernel (the dominant one of the step) alone; they must belong to the
 * stream's device. */
int mqa_decode_ex(const void* q, const void* k_new, const void* v_new, int32_t h,
                  const mqa_cache* cache, int32_t* lens, int32_t* err_flag, float scale,
                  int32_t window, void* o, void* workspace, size_t ws_bytes, void* stream,
                  void* ev_begin, void* ev_end);

/* mqa_decode_noalloc -- mqa_decode_ex (k_new / v_new NULL: a plain decode;
 * non-NULL: the fused append) without a caller workspace and without
 * allocating anything, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it).
 * The split-K records live in a fixed array of MQA_NOALLOC_SCRATCH_BYTES
 * inside the library, one per device, held until the process ends; its
 * address is looked up on the first call on each device.
 *   Results, arguments and errors as for mqa_decode_ex, plus:
 *   MQA_ERR_WORKSPACE : the shapes need more than MQA_NOALLOC_SCRATCH_BYTES of
 *                       records on this device (about 2 * CUs * occupancy
 *                       records of (h/G) * (d_h + 2) floats, plus 4 * (b + 4)
 *                       bytes); nothing is launched.
 *   MQA_ERR_LAUNCH    : the array's address could not be obtained.
 * Every call on one device shares that array and leaves it as it wrote it:
 * calls that overlap on one device (concurrent streams, or host threads
 * without ordering) race and give wrong results.  Order them on one stream. */
#define MQA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int mqa_decode_noalloc(const void* q, const void* k_new, const void* v_new, int32_t h,
                       const mqa_cache* cache, int32_t* lens, int32_t* err_flag, float scale,
                       int32_t window, void* o, void* stream);

/* mqa_prefill_causal -- causal attention over a whole prompt (study notes
 * section 1: O = softmax(Q K^T / sqrt(d_h) + M) V with M_ij = -inf for j > i;
 * paper review section 2.3 batched form with an additive mask).
 *   Q, O    : device [b][n][h][d_h];  K, V : device [b][n][G][d_h].
 *   cache   : optional; when non-NULL, K and V are also copied into
 *             cache->k / cache->v at positions [0, n) of every sequence
 *             (requires cache->b == b, G, d_h, dtype equal, n <= m_cap).
 *   lens    : optional device int32 [b]; when non-NULL every lens[b] is set to n.
 */
int mqa_prefill_causal(const void* Q, const void* K, const void* V, int32_t b, int32_t n,
                       int32_t h, int32_t G, int32_t d_h, int32_t dtype, float scale,
                       const mqa_cache* cache, int32_t* lens, void* O, void* stream);

/* mqa_attend -- n queries per sequence attending over a fixed memory of m
 * positions with no causal structure, as in encoder-decoder attention (the
 * study notes' section 6.1: the multi-query layers replace encoder-decoder
 * attention too; the paper review's section 2.3 batched form, weights =
 * softmax(logits + mask)):
 *     O[b,t,i,:] = sum_j w_j V[b,j,g(i),:],
 *     w = softmax_j over j < m of (scale * Q[b,t,i,:].K[b,j,g(i),:] + mask(b,i,t,j))
 *   Q, O  : device [b][n][h][d_h];  K, V : device [b][m][G][d_h] (the memory).
 *   mask  : optional device fp32, 4-byte aligned; mask(b,i,t,j) is read at
 *           mask[b*mask_sb + i*mask_sh + t*mask_sn + j] (element strides >= 0,
 *           key index contiguous; a stride of 0 broadcasts: the pages' full
 *           [b][h][n][m] mask has strides (h*n*m, n*m, m), a key-padding mask
 *           [b][m] has (m, 0, 0)).  NULL: no mask.  -inf hides a key; a row
 *           whose every key is hidden gives o = 0.
 *   No cache is touched.  One launch on `stream`. */
int mqa_attend(const void* Q, const void* K, const void* V, int32_t b, int32_t n, int32_t m,
               int32_t h, int32_t G, int32_t d_h, int32_t dtype, float scale, const float* mask,
               int64_t mask_sb, int64_t mask_sh, int64_t mask_sn, void* O, void* stream);

/* Debug helper: synchronises `stream`, copies lens to the host and returns
 * MQA_ERR_LENS if any lens[b] lies outside [0, m_cap], else MQA_OK. */
int mqa_check_lens(const int32_t* lens, int32_t b, int32_t m_cap, void* stream);

/* Measurement aid, not part of the attention path: reads `bytes` (a
 * multiple of 16; buf 16-byte aligned) of device memory once with a plain
 * streaming kernel, so a caller can time the practical HBM read rate the
 * decode is compared with.  `sink` is 4 bytes of device memory that is
 * written only when the XOR of everything read equals 0x5a5aa5a5 (never for
 * a zero- or one-filled buffer).  One launch on `stream`. */
int mqa_read_probe(const void* buf, size_t bytes, void* sink, void* stream);

/* Static, human-readable text for a status code. */
const char* mqa_strerror(int status);

/* ABI version of this header (major * 100 + minor). */
int mqa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MQA_H */
