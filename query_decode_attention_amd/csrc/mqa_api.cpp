// mqa_api.cpp -- the C ABI of libmqa.so (declared in include/mqa.h): argument
// validation on the host, then asynchronous launches on the caller's stream.
// Nothing here allocates device memory or synchronises, except
// mqa_check_lens, which exists to synchronise.
#include "mqa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <vector>

#include "mqa_internal.h"
#include "mqa_reorder.h"
#include "mqa_attend.h"

namespace mqa {

int current_device_cus(int* device_out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (device_out) *device_out = dev;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace mqa

namespace {

static_assert(MQA_NOALLOC_SCRATCH_BYTES == mqa::kNoAllocScratchBytes,
              "the header states the library's scratch size");

constexpr int kMaxHeadsPerGroup = 32;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) { return dtype == MQA_F32 ? 4 : 2; }

// Shape checks of a cache descriptor (no pointer checks).
int check_cache_shape(const mqa_cache* c) {
  if (!c) return MQA_ERR_NULL;
  if (c->dtype != MQA_F32 && c->dtype != MQA_BF16) return MQA_ERR_DTYPE;
  if (c->d_h != 64 && c->d_h != 128) return MQA_ERR_DHEAD;
  if (c->b < 0 || c->m_cap < 1 || c->G < 1) return MQA_ERR_SHAPE;
  // flat tile and schedule-unit indices are 32-bit on the device
  const int64_t units = (int64_t)c->b * c->G * ((c->m_cap + 31) / 32 + mqa::kMaxSegLead);
  if (units >= ((int64_t)1 << 30)) return MQA_ERR_SHAPE;
  return MQA_OK;
}

// Shape and pointer checks shared by every call that takes a cache.
int check_cache(const mqa_cache* c) {
  const int rc = check_cache_shape(c);
  if (rc != MQA_OK) return rc;
  if (c->b > 0) {
    if (!c->k || !c->v) return MQA_ERR_NULL;
    if (!aligned16(c->k) || !aligned16(c->v)) return MQA_ERR_ALIGN;
  }
  return MQA_OK;
}

int check_heads(int32_t h, int32_t G) {
  if (h < 1 || G < 1 || h % G != 0) return MQA_ERR_SHAPE;
  if (h / G > kMaxHeadsPerGroup) return MQA_ERR_SHAPE;
  return MQA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MQA_OK : MQA_ERR_LAUNCH; }

// In place (lens_out null, two launches) or into lens_out (one launch).
int kv_reorder(const mqa_cache* cache, int32_t* lens, int32_t* lens_out, bool out_of_place,
               const int32_t* parent, int32_t beam, int32_t* err_flag, void* stream) {
  int rc = check_cache(cache);
  if (rc != MQA_OK) return rc;
  if (beam < 1 || beam > mqa::kMaxBeam || cache->b % beam != 0) return MQA_ERR_SHAPE;
  if (cache->b == 0) return MQA_OK;
  if (!lens || !parent || (out_of_place && !lens_out)) return MQA_ERR_NULL;
  if (out_of_place && lens_out == lens) return MQA_ERR_SHAPE;
  mqa::ReorderParams p;
  p.k = static_cast<char*>(cache->k);
  p.v = static_cast<char*>(cache->v);
  p.lens = lens;
  p.lens_out = lens_out;
  p.parent = parent;
  p.err_flag = err_flag;
  p.b = cache->b;
  p.m_cap = cache->m_cap;
  p.beam = beam;
  p.row_bytes = cache->G * cache->d_h * elem_size(cache->dtype);
  return launch_status(mqa::launch_kv_reorder(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int mqa_abi_version(void) { return 205; }

const char* mqa_strerror(int status) {
  switch (status) {
    case MQA_OK: return "success";
    case MQA_ERR_NULL: return "a required pointer is NULL";
    case MQA_ERR_SHAPE: return "invalid shape (b, n, h, G, m_cap) or h/G > 32 or G does not divide h";
    case MQA_ERR_DHEAD: return "unsupported head dimension (d_h must be 64 or 128)";
    case MQA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case MQA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MQA_ERR_LAUNCH: return "the HIP runtime refused a launch or query";
    case MQA_ERR_DTYPE: return "unknown element type";
    case MQA_ERR_LENS: return "some lens[b] lies outside [0, m_cap]";
    default: return "unknown status";
  }
}

int mqa_kv_append(const void* k_new, const void* v_new, const mqa_cache* cache, int32_t* lens,
                  int32_t* err_flag, void* stream) {
  int rc = check_cache(cache);
  if (rc != MQA_OK) return rc;
  if (cache->b == 0) return MQA_OK;
  if (!k_new || !v_new || !lens) return MQA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return MQA_ERR_ALIGN;
  mqa::AppendParams p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k = cache->k;
  p.v = cache->v;
  p.lens = lens;
  p.err_flag = err_flag;
  p.b = cache->b;
  p.m_cap = cache->m_cap;
  p.row_bytes = cache->G * cache->d_h * elem_size(cache->dtype);
  return launch_status(mqa::launch_kv_append(p, static_cast<hipStream_t>(stream)));
}


int mqa_kv_reorder(const mqa_cache* cache, int32_t* lens, const int32_t* parent, int32_t beam,
                   int32_t* err_flag, void* stream) {
  return kv_reorder(cache, lens, nullptr, false, parent, beam, err_flag, stream);
}

int mqa_kv_reorder_to(const mqa_cache* cache, const int32_t* lens_in, int32_t* lens_out,
                      const int32_t* parent, int32_t beam, int32_t* err_flag, void* stream) {
  return kv_reorder(cache, const_cast<int32_t*>(lens_in), lens_out, true, parent, beam, err_flag,
                    stream);
}

size_t mqa_decode_workspace_size(int32_t h, const mqa_cache* cache) {
  if (check_cache_shape(cache) != MQA_OK || check_heads(h, cache->G) != MQA_OK) return 0;
  return mqa::decode_workspace_bytes(cache->b, h, cache->G, cache->d_h, cache->m_cap);
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points (everything but the workspace)
// and the launch parameters; *skip is set when there is nothing to launch.
int decode_params(const void* q, const void* k_new, const void* v_new, int32_t h,
                  const mqa_cache* cache, int32_t* lens, int32_t* err_flag, float scale,
                  int32_t window, void* o, mqa::DecodeParams* p, bool* skip) {
  *skip = false;
  int rc = check_cache(cache);
  if (rc != MQA_OK) return rc;
  rc = check_heads(h, cache->G);
  if (rc != MQA_OK) return rc;
  if (window < 0) return MQA_ERR_SHAPE;
  if ((k_new == nullptr) != (v_new == nullptr)) return MQA_ERR_NULL;
  if (cache->b == 0) {
    *skip = true;
    return MQA_OK;
  }
  if (!q || !o || !lens) return MQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(o)) return MQA_ERR_ALIGN;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return MQA_ERR_ALIGN;
  p->q = q;
  p->k = cache->k;
  p->v = cache->v;
  p->lens = lens;
  p->k_new = k_new;
  p->v_new = v_new;
  p->err_flag = err_flag;
  p->o = o;
  p->ws = nullptr;
  p->b = cache->b;
  p->h = h;
  p->G = cache->G;
  p->dh = cache->d_h;
  p->m_cap = cache->m_cap;
  p->window = window;
  p->dtype = cache->dtype;
  p->scale = scale;
  return MQA_OK;
}

}  // namespace

extern "C" {

int mqa_decode_ex(const void* q, const void* k_new, const void* v_new, int32_t h,
                  const mqa_cache* cache, int32_t* lens, int32_t* err_flag, float scale,
                  int32_t window, void* o, void* workspace, size_t ws_bytes, void* stream,
                  void* ev_begin, void* ev_end) {
  mqa::DecodeParams p;
  bool skip = false;
  int rc = decode_params(q, k_new, v_new, h, cache, lens, err_flag, scale, window, o, &p, &skip);
  if (rc != MQA_OK || skip) return rc;
  const size_t need = mqa::decode_workspace_bytes(cache->b, h, cache->G, cache->d_h, cache->m_cap);
  if (!workspace || !aligned16(workspace) || ws_bytes < need) return MQA_ERR_WORKSPACE;
  p.ws = workspace;
  p.ev_begin = static_cast<hipEvent_t>(ev_begin);
  p.ev_end = static_cast<hipEvent_t>(ev_end);
  return launch_status(mqa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int mqa_decode_noalloc(const void* q, const void* k_new, const void* v_new, int32_t h,
                       const mqa_cache* cache, int32_t* lens, int32_t* err_flag, float scale,
                       int32_t window, void* o, void* stream) {
  mqa::DecodeParams p;
  bool skip = false;
  int rc = decode_params(q, k_new, v_new, h, cache, lens, err_flag, scale, window, o, &p, &skip);
  if (rc != MQA_OK || skip) return rc;
  size_t need = 0;
  if (mqa::decode_launch_workspace_bytes(p, &need) != hipSuccess) return MQA_ERR_LAUNCH;
  if (need > mqa::kNoAllocScratchBytes) return MQA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (mqa::noalloc_scratch(&ws) != hipSuccess) return MQA_ERR_LAUNCH;
  p.ws = ws;
  return launch_status(mqa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int mqa_decode(const void* q, int32_t h, const mqa_cache* cache, const int32_t* lens, float scale,
               int32_t window, void* o, void* workspace, size_t ws_bytes, void* stream) {
  return mqa_decode_ex(q, nullptr, nullptr, h, cache, const_cast<int32_t*>(lens), nullptr, scale,
                       window, o, workspace, ws_bytes, stream, nullptr, nullptr);
}

int mqa_append_decode(const void* q, const void* k_new, const void* v_new, int32_t h,
                      const mqa_cache* cache, int32_t* lens, int32_t* err_flag, float scale,
                      int32_t window, void* o, void* workspace, size_t ws_bytes, void* stream) {
  if (cache && cache->b > 0 && (!k_new || !v_new)) return MQA_ERR_NULL;
  return mqa_decode_ex(q, k_new, v_new, h, cache, lens, err_flag, scale, window, o, workspace,
                       ws_bytes, stream, nullptr, nullptr);
}

int mqa_prefill_causal(const void* Q, const void* K, const void* V, int32_t b, int32_t n,
                       int32_t h, int32_t G, int32_t d_h, int32_t dtype, float scale,
                       const mqa_cache* cache, int32_t* lens, void* O, void* stream) {
  if (dtype != MQA_F32 && dtype != MQA_BF16) return MQA_ERR_DTYPE;
  if (d_h != 64 && d_h != 128) return MQA_ERR_DHEAD;
  if (b < 0 || n < 1) return MQA_ERR_SHAPE;
  int rc = check_heads(h, G);
  if (rc != MQA_OK) return rc;
  // prefill grid: b * G row blocks of >= 8 rows
  if ((int64_t)b * G * ((n + 7) / 8) >= ((int64_t)1 << 31)) return MQA_ERR_SHAPE;
  if (cache) {
    rc = check_cache(cache);
    if (rc != MQA_OK) return rc;
    if (cache->b != b || cache->G != G || cache->d_h != d_h || cache->dtype != dtype ||
        n > cache->m_cap)
      return MQA_ERR_SHAPE;
  }
  if (b == 0) return MQA_OK;
  if (!Q || !K || !V || !O) return MQA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return MQA_ERR_ALIGN;
  mqa::PrefillParams p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.cache_k = cache ? cache->k : nullptr;
  p.cache_v = cache ? cache->v : nullptr;
  p.lens = lens;
  p.b = b;
  p.n = n;
  p.h = h;
  p.G = G;
  p.dh = d_h;
  p.dtype = dtype;
  p.m_cap = cache ? cache->m_cap : n;
  p.scale = scale;
  return launch_status(mqa::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

int mqa_attend(const void* Q, const void* K, const void* V, int32_t b, int32_t n, int32_t m,
               int32_t h, int32_t G, int32_t d_h, int32_t dtype, float scale, const float* mask,
               int64_t mask_sb, int64_t mask_sh, int64_t mask_sn, void* O, void* stream) {
  if (dtype != MQA_F32 && dtype != MQA_BF16) return MQA_ERR_DTYPE;
  if (d_h != 64 && d_h != 128) return MQA_ERR_DHEAD;
  if (b < 0 || n < 1 || m < 1) return MQA_ERR_SHAPE;
  int rc = check_heads(h, G);
  if (rc != MQA_OK) return rc;
  if ((int64_t)b * G * ((n + 7) / 8) >= ((int64_t)1 << 31)) return MQA_ERR_SHAPE;
  if (mask && (mask_sb < 0 || mask_sh < 0 || mask_sn < 0)) return MQA_ERR_SHAPE;
  if (b == 0) return MQA_OK;
  if (!Q || !K || !V || !O) return MQA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return MQA_ERR_ALIGN;
  if (mask && (reinterpret_cast<uintptr_t>(mask) & 3u)) return MQA_ERR_ALIGN;
  mqa::AttendParams a;
  a.base.Q = Q;
  a.base.K = K;
  a.base.V = V;
  a.base.O = O;
  a.base.cache_k = a.base.cache_v = nullptr;
  a.base.lens = nullptr;
  a.base.b = b;
  a.base.n = n;
  a.base.h = h;
  a.base.G = G;
  a.base.dh = d_h;
  a.base.dtype = dtype;
  a.base.m_cap = m;
  a.base.scale = scale;
  a.m = m;
  a.mask = mask;
  a.msb = mask_sb;
  a.msh = mask_sh;
  a.msn = mask_sn;
  return launch_status(mqa::launch_attend(a, static_cast<hipStream_t>(stream)));
}

int mqa_read_probe(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink) return MQA_ERR_NULL;
  if (!aligned16(buf) || bytes % 16 != 0) return MQA_ERR_ALIGN;
  if (bytes == 0) return MQA_OK;
  return launch_status(mqa::launch_read_probe(buf, bytes, static_cast<uint32_t*>(sink),
                                              static_cast<hipStream_t>(stream)));
}

int mqa_check_lens(const int32_t* lens, int32_t b, int32_t m_cap, void* stream) {
  if (b < 0 || m_cap < 1) return MQA_ERR_SHAPE;
  if (b == 0) return MQA_OK;
  if (!lens) return MQA_ERR_NULL;
  std::vector<int32_t> host((size_t)b);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host.data(), lens, sizeof(int32_t) * (size_t)b, hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return MQA_ERR_LAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return MQA_ERR_LAUNCH;
  for (int32_t v : host)
    if (v < 0 || v > m_cap) return MQA_ERR_LENS;
  return MQA_OK;
}

}  // extern "C"
