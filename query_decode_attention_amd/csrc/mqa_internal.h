// mqa_internal.h -- host-side interface between the C-ABI layer (mqa_api.cpp)
// and the kernel launchers (mqa_decode.hip, mqa_prefill.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mqa {

// Largest split-K grid the decode may use; bounds the workspace.
constexpr int kMaxDecodeGrid = 2048;
// Upper bound of the decode schedule's lead-in units per segment; the cache
// shape check keeps b * G * (tiles per sequence + kMaxSegLead) below 2^30,
// so unit indices fit in 32 bits on the device.
constexpr int kMaxSegLead = 8;
// Cache positions per wave tile in the decode and prefill kernels.
constexpr int kTileRows = 32;

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* lens;     // written (+1) only when k_new is set
  const void* k_new;       // nullable: fused append
  const void* v_new;
  int32_t* err_flag;       // nullable
  void* o;
  void* ws;
  int b, h, G, dh, m_cap, window, dtype;
  float scale;
  hipEvent_t ev_begin = nullptr;  // optional, recorded around the split kernel
  hipEvent_t ev_end = nullptr;
};

struct AppendParams {
  const void* k_new;
  const void* v_new;
  void* k;
  void* v;
  int32_t* lens;
  int32_t* err_flag;
  int b, m_cap;
  int row_bytes;  // G * d_h * element size
};

struct PrefillParams {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  void* cache_k;  // nullable
  void* cache_v;
  int32_t* lens;  // nullable
  int b, n, h, G, dh, dtype, m_cap;
  float scale;
};

// Size in bytes of one split-K partial record for hg heads of width dh.
size_t decode_record_bytes(int hg, int dh);
// Byte offset of the first record in the workspace (after the schedule header).
size_t decode_records_offset(int b);
// Upper bound of the decode grid for these shapes (device independent).
int decode_grid_cap(int b, int G, int m_cap);
// Workspace bytes for mqa_decode.
size_t decode_workspace_bytes(int b, int h, int G, int dh, int m_cap);
// Workspace bytes that the decode launched for p on the current device
// actually touches (its header and the records of its real grid), at most
// decode_workspace_bytes of the same shapes.
hipError_t decode_launch_workspace_bytes(const DecodeParams& p, size_t* bytes);

// The decode workspace of mqa_decode_noalloc: a device array of fixed size
// in the library itself, one per device, shared by every such call on it.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
// Device address of the current device's copy (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

// Compute units of the current device (cached per device).
int current_device_cus(int* device_out);

}  // namespace mqa
