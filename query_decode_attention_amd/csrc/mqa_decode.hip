// mqa_decode.hip -- gfx950 kernels of one MQA/GQA decode step.
//
//   kv_append_kernel : the incremental concat of one new K/V row per sequence
//                      (paper review, section 3 multi-query pseudocode:
//                      new_K = concat(prev_K, k)), for callers that append
//                      separately.
//   decode_kernel    : optionally the append, then scores, online softmax and
//                      weighted V over every cached position (study notes
//                      section 4: o_i = softmax(q_i K^T * scale) V).
//   combine_kernel   : the exact merge of split segments, and the lens bump
//                      of a fused append.
//
// Work decomposition.  The visible positions of every (sequence b, group g)
// segment are cut into tiles of 32.  All segments form one flat list of U
// units -- a few lead-in units, then the segment's tiles -- and workgroup
// w of a grid of W takes units [U*w/W, U*(w+1)/W): every workgroup streams
// about the same number of bytes whatever the length mix (a few tiles fewer
// for each segment boundary its range crosses, see kSegLead).  Each wave
// derives this schedule from lens by itself (a DPP prefix sum over the
// wave) and keeps the lens entries it needs in registers, so the schedule
// costs no host synchronisation, no barrier and one read of lens.
//
// Pieces.  The part of a segment inside a workgroup's range is a piece.  The
// NW waves are shared out over the range's pieces, a piece's tiles go
// round-robin over its waves, and every wave streams one piece only: no wave
// waits for another until the range is done, and no partial result is
// stored while tiles still stream (on gfx9 a wave's next loads wait, in
// order, for the stores it issued before them, and under a read-saturated
// HBM a store takes microseconds to complete).  At the end all waves park
// their (max, sum, accumulator) in LDS and the workgroup folds the waves of
// each piece in a fixed order.  A segment that one workgroup covers
// completely is normalised and written; a piece of a segment shared with
// neighbouring workgroups becomes an fp32 partial record that the combine
// kernel merges.  The records cross from one workgroup to another only
// through the kernel boundary: publishing them inside the kernel would need
// an agent-scope release per workgroup, i.e. a write-back of an XCD's whole
// L2, which costs far more on gfx950 than a second small launch.
//
// Q.  Every wave loads its piece's Q^T operand itself, so no wave waits for
// another; the load shares a memory round trip with the wave's first tile.
// bf16 keeps the operand in registers for the whole piece; fp32 (twice as
// wide) copies it into the wave's own fold slot (free until the wave parks)
// and reads it chunk by chunk.
//
// Whole sequences.  When every cache holds at most kWholeMaxTiles tiles, the
// kernel is instantiated with WHOLE: workgroup w takes whole sequences (all
// their groups), reads only its own lens entries, finishes every segment
// itself and writes no partial record, so no combine kernel runs.
//
// Fused append.  With k_new/v_new, sequence b attends over L_old + 1
// positions; the row at L_old is read from k_new/v_new (never from the cache)
// and the wave that owns it stores it into the cache.  lens itself is bumped
// by the combine kernel, after every decode workgroup has read it (with
// WHOLE, by the workgroup that owns the sequence, at its end: no other
// workgroup reads that entry).
//
// One wave, one 32-position tile, all h/G <= 32 heads of the group:
//   S^T[32 pos][32 heads] = K_tile . Q^T        (MFMA; K rows are the A operand
//                                                loaded straight from HBM)
//   online softmax per head column (log2 domain, scale*log2(e) folded in)
//   V_tile^T via an exact 0/1-selection MFMA    (position-major rows become the
//                                                d-major A operand of PV)
//   O^T[d][heads] += V^T . P^T                   (MFMA; P stays in registers)
// Each K/V byte is read from HBM once and used by every head of its group.
#include <stdlib.h>

#include <mutex>

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

// ------------------------------------------------------------ decode: args ----

struct DecodeArgs {
  const char* q;
  char* k;               // cache; written only at the appended row
  char* v;
  int32_t* lens;         // read; with WHOLE and an append, +1 at the workgroup's end
  const char* k_new;     // nullable: no fused append
  const char* v_new;
  int32_t* err_flag;     // nullable
  char* o;
  float* records;        // [2 * grid][rec_floats] partial results
  int32_t* prefix;       // [b + 1] units before each sequence, then the count of
                         // non-empty sequences, the lead-in and the effective
                         // grid (written by workgroup 0 for the combine)
  int b, h, G, hg, m_cap, window;
  int rec_floats;
  float scale_log2;
};

// Visible range [j0, L) of sequence bi and the appended position (or -1).
struct SeqView {
  int j0, L, app_pos;
};

// From the raw lens entry of the sequence.
__device__ __forceinline__ SeqView seq_view_raw(const DecodeArgs& a, int raw) {
  int l = raw < 0 ? 0 : (raw > a.m_cap ? a.m_cap : raw);
  int app = -1;
  if (a.k_new && raw >= 0 && raw < a.m_cap) {
    app = raw;
    l = raw + 1;
  }
  SeqView s;
  s.L = l;
  s.j0 = (a.window > 0 && l > a.window) ? l - a.window : 0;
  s.app_pos = app;
  return s;
}

__device__ __forceinline__ int tiles_of(const SeqView& s) {
  return (s.L - s.j0 + kTileRows - 1) / kTileRows;
}

// Schedule units.  Every non-empty segment is `lead` virtual units (no
// positions) followed by its tiles, and workgroups split the units evenly.  A
// workgroup whose range reaches into a further segment thereby takes about
// `lead` fewer tiles, which pays for what a boundary costs it: its waves
// are split between two pieces (whole waves, so some take a tile more than
// an even split would give them), a second Q^T copy and a second record.
// (c3 kernel for lead-ins 0, 1, 2, 4, 6: 32.5, 32.1, 31.7, 31.5, 31.4 us.)
// A small step (at most one tile per
// wave of the launched grid) has no lead-in and up to one workgroup per
// kSmallUnits units: there every workgroup has about one round of loads, a
// CU streams only ~20 GB/s, and spreading the step over more CUs is worth
// more than avoiding boundaries.
constexpr int kSegLead = 6;
static_assert(kSegLead <= kMaxSegLead, "lead-in within the unit-index bound");
constexpr int kSmallUnits = 4;

// Workgroups that share the Tv units of `segs` non-empty segments: the
// launched grid, but no more than one per kSmallUnits units of a small step
// (one per NW units otherwise) unless there are more segments than that
// (short segments are better run side by side than one after another), and
// no more than Tv / (lead + 1), so that every range of units holds at least
// one tile.  The combine reads the value back.  32-bit arithmetic with
// constant divisors (Tv < 2^30 by the shape check).
template <int NW>
__device__ __forceinline__ int effective_grid(int Tv, int segs, int grid, bool small_step) {
  const unsigned T = (unsigned)Tv;
  unsigned w = small_step ? (T + kSmallUnits - 1) / kSmallUnits : (T + NW - 1) / NW;
  if (w < (unsigned)segs) w = (unsigned)segs;
  if (w > (unsigned)grid) w = (unsigned)grid;
  const unsigned cap = small_step ? T : T / (kSegLead + 1);  // small steps have no lead-in
  if (w > cap) w = cap;
  return (int)(w < 1 ? 1 : w);
}

// Lanes below this one whose bit is set in `mask` (a wave-wide ballot).
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// First unit of workgroup w out of W over T units, floor(T * w / W), and the
// workgroup whose range holds unit t (T > 0), ceil((t + 1) * W / T) - 1.
// With T < 2^30 and W <= kMaxDecodeGrid (2^11) both products are exact in a
// double, and a correctly rounded quotient cannot cross an integer (a
// non-integer quotient lies at least 1/W resp. 1/T from one, far more than
// its rounding error), so floor / ceil of the double quotient are exact; the
// double divide is much shorter than a 64-bit integer one.
static_assert(kMaxDecodeGrid <= 2048, "exact double quotients below need W <= 2^11");
__device__ __forceinline__ int wg_start(int T, int w, int W) {
  return (int)((double)T * (double)w / (double)W);
}
__device__ __forceinline__ int wg_of(int t, int T, int W) {
  return (int)__builtin_ceil((double)(t + 1) * (double)W / (double)T) - 1;
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  // Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round
  // trips): shifts by 1, 2, 4, 8 within each row of 16 lanes (0 shifted in),
  // then the last lane of row 0 / 2 is added to row 1 / 3 and the last lane
  // of row 1 to rows 2 and 3.
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Sum over the wave (uniform).
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

// Maximum over the wave of non-negative values (uniform); the same moves as
// wave_incl_scan, with max in place of +.
__device__ __forceinline__ int wave_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(x, 63);
}

// ------------------------------------------------------------ decode: tiles ----

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
    // issue every load of the tile before any use: one memory round trip
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      kr[c] = u32x4{0u, 0u, 0u, 0u};
      vr[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// This lane's chunks of the Q^T operand, read from LDS.
template <int NQ>
__device__ __forceinline__ void read_q(const u32x4 (*s_q)[64], int lane, u32x4 (&qr)[NQ]) {
#pragma unroll
  for (int c = 0; c < NQ; ++c) qr[c] = s_q[c][lane];
}

// Where the Q^T chunks of a tile's score product come from: registers read
// ahead (bf16), or LDS read chunk by chunk next to their product (fp32,
// whose operands are too wide to hold all at once).
struct QFromRegs {
  const u32x4* r;
  __device__ __forceinline__ u32x4 get(int c) const { return r[c]; }
};
struct QFromLds {
  const u32x4 (*s)[64];
  int lane;
  __device__ __forceinline__ u32x4 get(int c) const { return s[c][lane]; }
};

// One decode tile: scores, online softmax with the tail masked at L, and P.V
// with the V rows transposed in registers.
template <typename T, int DH, bool FULL, typename QSrc>
__device__ __forceinline__ void tile_update(WaveState<TileShape<T, DH>::ND>& st,
                                            const u32x4 (&kr)[TileShape<T, DH>::NQ],
                                            const u32x4 (&vr)[TileShape<T, DH>::NQ],
                                            const QSrc& q, const SelOps<T>& sel,
                                            float scale_log2, int pos0, int L, int half) {
  constexpr int ND = TileShape<T, DH>::ND;
  constexpr int NQ = TileShape<T, DH>::NQ;
  constexpr int VTC = TileShape<T, DH>::VTC;
  f32x16 s = {};
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    const u32x4 qc = q.get(c);
    if constexpr (sizeof(T) == 2) {
      s = mfma_bf16(as_bf16x8(kr[c]), as_bf16x8(qc), s);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma_f32(__uint_as_float(kr[c][e]), __uint_as_float(qc[e]), s);
    }
  }
  ProbTile<T> p;
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

// ----------------------------------------------------------- decode: merging ----

// LDS image of one wave's state, laid out so that lane i of every wave writes
// and reads consecutive 16-byte words (bank-conflict free).
template <int ND>
struct WaveSlot {
  f32x4 o[ND][4][64];
  float m[64];
  float l[64];
};

template <int ND>
__device__ __forceinline__ void park(const WaveState<ND>& st, WaveSlot<ND>& sl, int lane) {
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      sl.o[d][r4][lane] = f32x4{st.o[d][4 * r4], st.o[d][4 * r4 + 1], st.o[d][4 * r4 + 2],
                                st.o[d][4 * r4 + 3]};
  sl.m[lane] = st.m;
  sl.l[lane] = st.l;
}

// Word e of a slot is (d block, r4, lane): head = lane % 32 and
// d = 32*blk + 8*r4 + 4*(lane/32) .. +3.
struct SlotIndex {
  int blk, r4, lane;
  __device__ __forceinline__ explicit SlotIndex(int e) {
    lane = e & 63;
    r4 = (e >> 6) & 3;
    blk = e >> 8;
  }
  __device__ __forceinline__ int head() const { return lane & 31; }
  __device__ __forceinline__ int d() const { return 32 * blk + 8 * r4 + 4 * (lane >> 5); }
};

// Q^T operand of group g of sequence bi in LDS, lane order: chunk c of lane l
// is head l % 32, 16-byte chunk 2c + l / 32 of its row.  Columns of heads
// >= h/G repeat a real head, so they hold finite values; every head column
// has its own softmax and those columns are never written out.
__device__ __forceinline__ const char* q_row(const DecodeArgs& a, int bi, int g, int lane,
                                             int row_bytes) {
  const int row = lane & 31;
  const int qrow = row < a.hg ? row : row % a.hg;
  return a.q + ((size_t)bi * a.h + (size_t)g * a.hg + qrow) * row_bytes;
}

// The whole Q^T operand copied by one wave into an LDS region of its own
// (no other wave reads it, so no barrier is needed); complete once this
// wave's vmcnt reaches 0.
template <typename T, int DH>
__device__ __forceinline__ void copy_q_own(const DecodeArgs& a, u32x4 (*dst)[64], int bi, int g,
                                           int lane) {
  constexpr int NQ = TileShape<T, DH>::NQ;
  const int half = lane >> 5;
  const char* qp = q_row(a, bi, g, lane, DH * sizeof(T));
#pragma unroll
  for (int c = 0; c < NQ; ++c) load_to_lds(qp + (2 * c + half) * 16, &dst[c][0]);
}

// ------------------------------------------------------------ decode: kernel ----

// WHOLE: workgroup w takes sequences [b w / W, b (w + 1) / W), every group of
// each, whole: no partial records, and the lens bump after an append done
// here (see launch_decode_t).
template <typename T, int DH, int NW, bool WHOLE>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using S = TileShape<T, DH>;
  constexpr int NQ = S::NQ, ND = S::ND;
  constexpr int kWords = ND * 4 * 64;  // f32x4 words per slot
  static_assert(kWords % (NW * 64) == 0, "every thread folds the same number of words");
  __shared__ WaveSlot<ND> s_slot[NW];
  // A wave reads its piece's Q^T from its own fold slot, which it does not
  // need before it parks.
  static_assert(NQ * 64 * sizeof(u32x4) <= sizeof(WaveSlot<ND>), "Q^T fits a fold slot");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar
  const int row = lane & 31, half = lane >> 5;
  u32x4 (*const own_q)[64] = reinterpret_cast<u32x4 (*)[64]>(&s_slot[wave]);
  // lane constants of the V transpose (for b <= 64 set up while lens is in
  // flight, otherwise after the schedule)
  SelOps<T> sel;

  // ---- schedule (each wave on its own) ----
  // Three layouts of lens in the wave, by batch size: b <= 64, one entry per
  // lane; 64 < b <= 64 * kLensRegs ("block"), lane l holds the kLensRegs
  // consecutive entries from kLensRegs * l, so one round trip and one scan
  // over the lanes' block sums give every prefix; larger b, chunks of 64
  // entries (one per lane), read kLensRegs chunks at a time with all loads in
  // flight together (one memory round trip per 1024 sequences).
  constexpr int kLensRegs = 16;
  static_assert(kLensRegs == 16, "the block layout indexes lanes with >> 4");
  const int nchunks = (a.b + 63) / 64;
  const bool blk = nchunks > 1 && nchunks <= kLensRegs;
  int rawr[kLensRegs];
  auto load_block = [&]() {
#pragma unroll
    for (int k = 0; k < kLensRegs; ++k) {
      const int i = kLensRegs * lane + k;
      rawr[k] = a.lens[i < a.b ? i : a.b - 1];  // clamped: no branch between the loads
    }
  };
  // units of entry k of this lane's block in the block layout (0 past b)
  auto blk_tiles = [&](int k) {
    return kLensRegs * lane + k < a.b ? tiles_of(seq_view_raw(a, rawr[k])) : 0;
  };
  auto load_chunks = [&](int g0) {
    // unconditional loads of clamped indices (no branch between them, so they
    // are all in flight together); entries past b read as 0
#pragma unroll
    for (int k = 0; k < kLensRegs; ++k) {
      const int i = (g0 + k) * 64 + lane;
      if (g0 + k < nchunks)
        rawr[k] = a.lens[i < a.b ? i : a.b - 1];
      else
        rawr[k] = 0;
    }
#pragma unroll
    for (int k = 0; k < kLensRegs; ++k)
      if ((g0 + k) * 64 + lane >= a.b) rawr[k] = 0;
  };
  // Pass 1: tiles of every sequence (per group) and the non-empty count,
  // which fix the lead-in.  raw0 / v0 / incl0 (not in the block layout): lens
  // entry, tiles and their inclusive prefix for sequence `lane` (the first
  // 64), reused below.
  int tiles = 0, nonempty = 0, raw0 = 0, v0 = 0, incl0 = 0;
  // Tiles and non-empty sequences before lane's block (block layout) or
  // before chunk `lane` (chunk layout, up to 64 chunks), so that the range
  // search needs one block or chunk only.
  int ch_t = 0, ch_ne = 0;
  // (WHOLE: no pass over lens; each workgroup reads its own sequences' only)
  if constexpr (!WHOLE) {
  if (nchunks == 1) {  // b <= 64: one chunk, a compact path
    raw0 = lane < a.b ? a.lens[lane] : 0;
    sel.init(row, half);
    sel.pin();
    v0 = lane < a.b ? tiles_of(seq_view_raw(a, raw0)) : 0;
    incl0 = wave_incl_scan(v0);
    tiles = __builtin_amdgcn_readlane(incl0, 63);
    nonempty = __popcll(__ballot(v0 > 0));
  }
  if (__builtin_expect(blk, 0)) {
    load_block();
    int bt = 0, bne = 0;
#pragma unroll
    for (int k = 0; k < kLensRegs; ++k) {
      const int v = blk_tiles(k);
      bt += v;
      bne += v > 0 ? 1 : 0;
    }
    const int it = wave_incl_scan(bt), ine = wave_incl_scan(bne);
    ch_t = it - bt;
    ch_ne = ine - bne;
    tiles = __builtin_amdgcn_readlane(it, 63);
    nonempty = __builtin_amdgcn_readlane(ine, 63);
  }
  if (__builtin_expect(nchunks > kLensRegs, 0)) {
  for (int g0 = 0; g0 < nchunks; g0 += kLensRegs) {
    load_chunks(g0);
#pragma unroll
    for (int k = 0; k < kLensRegs; ++k) {
      if (g0 + k >= nchunks) break;
      const int c = (g0 + k) * 64;
      const int v = (c + lane < a.b) ? tiles_of(seq_view_raw(a, rawr[k])) : 0;
      const int incl = wave_incl_scan(v);
      if (c == 0) {
        raw0 = rawr[k];
        v0 = v;
        incl0 = incl;
      }
      if (lane == g0 + k) {
        ch_t = tiles;
        ch_ne = nonempty;
      }
      tiles += __builtin_amdgcn_readlane(incl, 63);
      nonempty += __popcll(__ballot(v > 0));
    }
  }
  }
  }
  tiles = __builtin_amdgcn_readfirstlane(tiles);
  nonempty = __builtin_amdgcn_readfirstlane(nonempty);
  const bool small = (int64_t)tiles * a.G <= (int64_t)NW * gridDim.x;
  const int lead = small ? 0 : kSegLead;
  const int total = tiles + lead * nonempty;                // units per group
  // Unit indices fit in 32 bits: the cache shape check bounds
  // b * G * (tiles per sequence + kMaxSegLead) below 2^30.
  const int Tt = total * a.G;  // units
  const int segs = nonempty * a.G;
  // Workgroups in use (see effective_grid): every wave has work, short
  // segments still run side by side.
  const int W = WHOLE ? 1 : effective_grid<NW>(Tt, segs, gridDim.x, small);
  const int t0 = WHOLE ? 0 : wg_start(Tt, blockIdx.x, W);
  const int t1 = WHOLE ? 0 : wg_start(Tt, blockIdx.x + 1, W);
  // Units of the sequences of one chunk: their tiles plus `lead` per non-empty
  // sequence; u_excl / u_incl are prefixes within the chunk.
  auto chunk_units = [&](int v, int incl, int& u, int& u_incl) {
    const uint64_t ne = __ballot(v > 0);
    u = v > 0 ? v + lead : 0;
    u_incl = incl + lead * (lanes_below(ne) + (v > 0 ? 1 : 0));
  };

  // lens entries of sequences cbase .. cbase + 63, one per lane: the segment
  // walk below reads lens from here, not from memory.
  int cbase = 0, craw = raw0;
  int b_cur = a.b;
  int seg_base = 0;
  // WHOLE: sequences [s_begin, s_end), every group of each; the lens cache
  // starts at s_begin
  int s_begin = a.b, s_end = a.b;
  int raw_first = 0;  // lens entries s_begin .. s_begin + 63, as read at the start
  if constexpr (WHOLE) {
    const int wb = (int)gridDim.x < a.b ? (int)gridDim.x : a.b;
    const int w = (int)blockIdx.x;
    if (w < wb) {
      s_begin = (int)((int64_t)a.b * w / wb);
      s_end = (int)((int64_t)a.b * (w + 1) / wb);
    }
    b_cur = s_begin;
    cbase = s_begin;
    craw = (s_begin + lane < a.b) ? a.lens[s_begin + lane] : 0;
    raw_first = craw;
  } else {
  if (t0 < t1 && nchunks == 1) {
    int u, u_incl;
    chunk_units(v0, incl0, u, u_incl);
    const uint64_t hit = __ballot(lane < a.b && u > 0 && (u_incl - u) * a.G <= t0 && t0 < u_incl * a.G);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      b_cur = __builtin_amdgcn_readfirstlane(src);
      seg_base = __builtin_amdgcn_readfirstlane(__shfl(u_incl - u, src, 64) * a.G);
    }
  } else if (__builtin_expect(t0 < t1 && blk, 0)) {
    // the block holding unit t0 from the per-block prefixes, then a uniform
    // walk over its entries (read from lane kh)
    const int u_before = ch_t + lead * ch_ne;  // units (per group) before lane's block
    const uint64_t cm = __ballot(kLensRegs * lane < a.b && u_before * a.G <= t0);
    const int kh = 63 - __builtin_clzll(cm);
    int run = __builtin_amdgcn_readlane(u_before, kh);
#pragma unroll
    for (int k = 0; k < kLensRegs; ++k) {
      const int bi = kLensRegs * kh + k;
      const int raw = __builtin_amdgcn_readlane(rawr[k], kh);
      const int v = bi < a.b ? tiles_of(seq_view_raw(a, raw)) : 0;
      const int u = v > 0 ? v + lead : 0;
      if (u > 0 && t0 < (run + u) * a.G) {
        b_cur = bi;
        seg_base = run * a.G;
        break;
      }
      run += u;
    }
    b_cur = __builtin_amdgcn_readfirstlane(b_cur);
    seg_base = __builtin_amdgcn_readfirstlane(seg_base);
    // the lane cache below (entries b_cur .. b_cur + 63) from the blocks:
    // entry j sits in register j % 16 of lane j / 16
    const int j = b_cur + lane;
    int x = 0;
#pragma unroll
    for (int k = 0; k < kLensRegs; ++k) {
      const int y = __builtin_amdgcn_ds_bpermute(((j >> 4) & 63) << 2, rawr[k]);
      if ((j & (kLensRegs - 1)) == k) x = y;
    }
    cbase = b_cur;
    craw = j < a.b ? x : 0;
  } else if (__builtin_expect(t0 < t1 && nchunks <= 64, 0)) {
    // the chunk holding unit t0 from the per-chunk prefixes, then one scan
    const int u_before = ch_t + lead * ch_ne;  // units (per group) before chunk `lane`
    const uint64_t cm = __ballot(lane < nchunks && u_before * a.G <= t0);
    const int kh = 63 - __builtin_clzll(cm);
    const int c = kh * 64;
    const int run = __builtin_amdgcn_readlane(u_before, kh);
    const int raw = a.lens[c + lane < a.b ? c + lane : a.b - 1];
    const int v = (c + lane < a.b) ? tiles_of(seq_view_raw(a, raw)) : 0;
    const int incl = wave_incl_scan(v);
    int u, u_incl;
    chunk_units(v, incl, u, u_incl);
    const int lo = (run + u_incl - u) * a.G, hi = (run + u_incl) * a.G;
    const uint64_t hit = __ballot(c + lane < a.b && u > 0 && lo <= t0 && t0 < hi);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      b_cur = __builtin_amdgcn_readfirstlane(c + src);
      seg_base = __builtin_amdgcn_readfirstlane((run + __shfl(u_incl - u, src, 64)) * a.G);
      cbase = c;
      craw = raw;
    }
  } else if (__builtin_expect(t0 < t1, 0)) {
    int run = 0;
    bool found = false;
    for (int g0 = 0; g0 < nchunks && !found; g0 += kLensRegs) {
      load_chunks(g0);
#pragma unroll
      for (int k = 0; k < kLensRegs; ++k) {
        if (g0 + k >= nchunks) break;
        const int c = (g0 + k) * 64;
        const int raw = rawr[k];
        int v = v0, incl = incl0;
        if (c > 0) {
          v = (c + lane < a.b) ? tiles_of(seq_view_raw(a, raw)) : 0;
          incl = wave_incl_scan(v);
        }
        int u, u_incl;
        chunk_units(v, incl, u, u_incl);
        const int lo = (run + u_incl - u) * a.G, hi = (run + u_incl) * a.G;
        const uint64_t hit = __ballot(c + lane < a.b && u > 0 && lo <= t0 && t0 < hi);
        if (hit) {
          const int src = __builtin_ctzll(hit);
          b_cur = c + src;
          seg_base = __builtin_amdgcn_readfirstlane((run + __shfl(u_incl - u, src, 64)) * a.G);
          cbase = c;
          craw = raw;
          found = true;
          break;
        }
        run += __builtin_amdgcn_readlane(u_incl, 63);
      }
    }
    b_cur = __builtin_amdgcn_readfirstlane(b_cur);
  }


  }
  if (WHOLE || nchunks != 1) sel.init(row, half);
  const size_t row_stride = (size_t)a.G * DH * sizeof(T);
  // lens entry of sequence bi (uniform), refilling the lane cache by chunks
  auto raw_of = [&](int bi) {
    if (bi < cbase || bi >= cbase + 64) {
      cbase = bi;
      craw = (bi + lane < a.b) ? a.lens[bi + lane] : 0;
    }
    return __builtin_amdgcn_readlane(craw, bi - cbase);  // uniform lane: no LDS trip
  };

  // A piece is the part of one (sequence, group) segment inside this
  // workgroup's range.  The waves are shared out over the pieces (up to NW of
  // them per round; one round unless the range crosses more than NW
  // segments), a piece's tiles go round-robin over its waves, and every wave
  // streams one piece only.  So no wave waits for another before the one fold
  // at the end of the round, and nothing is stored while tiles still stream
  // (a wave's next loads would wait for those stores to complete).
  int t = t0;
  int g_cur = 0;  // WHOLE: the next group of sequence b_cur
  auto more = [&]() { return WHOLE ? b_cur < s_end : (t < t1 && b_cur < a.b); };
  bool first_round = true;
  while (more()) {
    // ---- the pieces of this round; lane p describes piece p ----
    int np = 0;
    int p_b = 0, p_g = 0, p_raw = 0, p_ta = 0, p_te = 0, p_nb = 0;
    while (np < NW && more()) {
      const int raw = raw_of(b_cur);
      const SeqView sv = seq_view_raw(a, raw);
      const int nb = __builtin_amdgcn_readfirstlane((sv.L - sv.j0 + kTileRows - 1) / kTileRows);
      if (nb == 0) {
        ++b_cur;
        continue;
      }
      const int unit = nb + lead;  // units of one group of this sequence
      const int g = WHOLE ? g_cur : a.G == 1 ? 0 : (t - seg_base) / unit;  // MQA: no division
      const int seg0 = seg_base + g * unit + lead;  // its first tile
      int ta, te;
      if constexpr (WHOLE) {
        ta = 0;
        te = nb;
      } else {
        ta = (t > seg0 ? t : seg0) - seg0;
        te = (t1 < seg0 + nb ? t1 : seg0 + nb) - seg0;
        if (te <= ta) {  // the range ends inside this segment's lead-in units
          t = t1;
          break;
        }
      }
      if (lane == np) {
        p_b = b_cur;
        p_g = g;
        p_raw = raw;
        p_ta = ta;
        p_te = te;
        p_nb = nb;
      }
      ++np;
      t = seg0 + te;
      if constexpr (WHOLE) {
        if (++g_cur == a.G) {
          g_cur = 0;
          ++b_cur;
        }
      } else if (g == a.G - 1 && te == nb) {
        seg_base += a.G * unit;
        ++b_cur;
      }
    }
    if (np == 0) break;

    // ---- waves per piece ----
    // The smallest per-wave tile count k for which ceil(c_p / k) waves per
    // piece fit in NW; the spare waves go to the piece with the most tiles
    // (never more waves than tiles).  Piece p has waves [p_ws, p_ws + p_w).
    const int c = lane < np ? p_te - p_ta : 0;
    int p_w = 0, used = 0, p_ws = 0;
    if (np == 1) {  // the usual case: one piece, min(c, NW) waves
      const int c0 = __builtin_amdgcn_readfirstlane(c);
      used = c0 < NW ? c0 : NW;
      p_w = lane == 0 ? used : 0;
    } else {
      int k = (wave_sum(c) + NW - 1) / NW;
      for (;;) {
        p_w = (c + k - 1) / k;
        used = wave_sum(p_w);
        if (used <= NW) break;
        ++k;
      }
      const int cmax = wave_max(c);
      const int pbig = __builtin_ctzll(__ballot(lane < np && c == cmax));
      const int room = __builtin_amdgcn_readlane(c - p_w, pbig);
      const int give = NW - used < room ? NW - used : room;
      if (lane == pbig) p_w += give;
      used += give;
      p_ws = wave_incl_scan(p_w) - p_w;
    }
    // this wave's piece, or -1 (more waves than tiles)
    const int pw = wave >= used ? -1 : np == 1 ? 0 : __popcll(__ballot(lane < np && p_ws <= wave)) - 1;
    // For the fold: bit w of `runs` is set where a run of waves (a piece, or
    // the waves without one) starts; lane p of p_flags says whether piece p
    // is a whole segment (bit 0) and which record slot it takes (bit 1).
    int runs = (used < NW ? 1 << used : 0) | 1;  // piece 0 starts at wave 0
    if (np > 1) {
#pragma unroll
      for (int x = 1; x < NW; ++x)
        if (__ballot(lane < np && p_ws == x)) runs |= 1 << x;
    }
    const int p_flags =
        ((p_ta == 0 && p_te == p_nb) ? 1 : 0) | ((first_round && lane == 0) ? 0 : 2);

    // ---- this wave's tiles ----
    WaveState<ND> st;
    st.reset();
    if (pw >= 0) {
      const int bi = __builtin_amdgcn_readlane(p_b, pw);
      const int g = __builtin_amdgcn_readlane(p_g, pw);
      const int te = __builtin_amdgcn_readlane(p_te, pw);
      const int step = __builtin_amdgcn_readlane(p_w, pw);
      const SeqView sv = seq_view_raw(a, __builtin_amdgcn_readlane(p_raw, pw));
      const int j0 = __builtin_amdgcn_readfirstlane(sv.j0);
      const int L = __builtin_amdgcn_readfirstlane(sv.L);
      const int app_pos = __builtin_amdgcn_readfirstlane(sv.app_pos);
      const size_t seq_off = ((size_t)bi * a.m_cap * a.G + (size_t)g) * DH * sizeof(T);
      const size_t new_off = ((size_t)bi * a.G + (size_t)g) * DH * sizeof(T);
      // Row of this lane in tile tl: pointers (the appended row comes from
      // k_new / v_new) and whether it is visible.
      auto row_ptrs = [&](int tl, const char*& kp, const char*& vp) {
        const int pos = j0 + tl * kTileRows + row;
        const bool is_new = (pos == app_pos);
        kp = is_new ? a.k_new + new_off : a.k + seq_off + (size_t)pos * row_stride;
        vp = is_new ? a.v_new + new_off : a.v + seq_off + (size_t)pos * row_stride;
        return pos < L;
      };
      // The concat: the lane holding the appended row stores it into the
      // cache (in the segment's last tile, so no later load waits for it).
      auto store_new_row = [&](int tl, const u32x4 (&kr)[NQ], const u32x4 (&vr)[NQ]) {
        const int pos = j0 + tl * kTileRows + row;
        if (pos != app_pos) return;
        char* kc = a.k + seq_off + (size_t)pos * row_stride;
        char* vc = a.v + seq_off + (size_t)pos * row_stride;
#pragma unroll
        for (int cc = 0; cc < NQ; ++cc) {
          *reinterpret_cast<u32x4*>(kc + (2 * cc + half) * 16) = kr[cc];
          *reinterpret_cast<u32x4*>(vc + (2 * cc + half) * 16) = vr[cc];
        }
      };

      // Q^T of the piece: bf16 keeps it in registers for the whole piece (8
      // loads, no LDS); fp32 (twice as wide) copies it into this wave's own
      // fold slot.  Either way the loads share their memory round trip with
      // the first tile, whose wait covers them.
      u32x4 qreg[NQ];
      if constexpr (sizeof(T) == 2) {
        const char* qp = q_row(a, bi, g, lane, DH * sizeof(T));
#pragma unroll
        for (int c = 0; c < NQ; ++c) qreg[c] = *reinterpret_cast<const u32x4*>(qp + (2 * c + half) * 16);
      } else {
        copy_q_own<T, DH>(a, own_q, bi, g, lane);
      }
      // this lane's byte offset in a tile (row, 16-byte half), so that a
      // tile load is a uniform base plus one 32-bit offset per lane
      const uint32_t lane_off = (uint32_t)row * (uint32_t)row_stride + (uint32_t)half * 16u;
      // Every tile of the piece is whole and free of the appended row except
      // perhaps the segment's last one (ragged, and/or holding the appended
      // row); that one is taken after the loop by the wave it falls to.
      const int nb = __builtin_amdgcn_readlane(p_nb, pw);
      const int last0 = j0 + (nb - 1) * kTileRows;
      const bool special = te == nb && (last0 + kTileRows > L || app_pos >= last0);
      const int te_whole = special ? te - 1 : te;
      int tile = __builtin_amdgcn_readlane(p_ta, pw) + (wave - __builtin_amdgcn_readlane(p_ws, pw));
      // The Q^T copy lands with the wave's first tile, which waits for both;
      // from the second tile on, the Q^T reads from LDS are issued right
      // behind the tile's loads and complete while those are in flight.
      auto whole_tile = [&](bool first_tile) {
        const int pos0 = j0 + tile * kTileRows;
        u32x4 kr[NQ], vr[NQ];
        // uniform base of the tile plus a 32-bit offset per lane
        const size_t base = seq_off + (size_t)pos0 * row_stride;
        load_kv<NQ, true>(a.k + base + lane_off, a.v + base + lane_off, true, 0, kr, vr);
        if (first_tile) __builtin_amdgcn_s_waitcnt(0x0F70);
        if constexpr (sizeof(T) == 2) {
          tile_update<T, DH, true>(st, kr, vr, QFromRegs{qreg}, sel, a.scale_log2, pos0, L, half);
        } else {
          tile_update<T, DH, true>(st, kr, vr, QFromLds{own_q, lane}, sel, a.scale_log2, pos0, L,
                                   half);
        }
      };
      bool q_landed = false;
      if (tile < te_whole) {
        whole_tile(true);
        q_landed = true;
        for (tile += step; tile < te_whole; tile += step) whole_tile(false);
      }
      if (special && tile == te - 1) {
        u32x4 kr[NQ], vr[NQ];
        const char *kp, *vp;
        const bool valid = row_ptrs(tile, kp, vp);
        load_kv<NQ, false>(kp, vp, valid, half, kr, vr);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        q_landed = true;
        store_new_row(tile, kr, vr);
        // masked at L (a whole tile passes the mask unchanged)
        if constexpr (sizeof(T) == 2) {
          tile_update<T, DH, false>(st, kr, vr, QFromRegs{qreg}, sel, a.scale_log2,
                                    j0 + tile * kTileRows, L, half);
        } else {
          tile_update<T, DH, false>(st, kr, vr, QFromLds{own_q, lane}, sel, a.scale_log2,
                                    j0 + tile * kTileRows, L, half);
        }
      }
      if (!q_landed) __builtin_amdgcn_s_waitcnt(0x0F70);  // no tile: the copy still lands
    }

    // ---- fold: park in LDS, combine each run of waves in a fixed order ----
    park<ND>(st, s_slot[wave], lane);
    __syncthreads();
    {
      // Thread t folds the f32x4 words t, t + NW*64, ... of the slots; all of
      // them belong to head t % 32, whose per-run max, weights and sum it
      // derives itself.
      const int hd = threadIdx.x & 31;
      constexpr int KW = kWords / (NW * 64);  // words per thread
      // Every LDS read of the fold is issued up front, ahead of the scans and
      // the (scalar) branches of the stores, so that their latencies overlap.
      float m[NW], l0[NW], l1[NW], f[NW], M[NW], Ls[NW];
      f32x4 wd[KW][NW];
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        m[x] = s_slot[x].m[hd];
        l0[x] = s_slot[x].l[hd];
        l1[x] = s_slot[x].l[hd + 32];
      }
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) {
        const SlotIndex ix(threadIdx.x + kw * NW * 64);
#pragma unroll
        for (int x = 0; x < NW; ++x) wd[kw][x] = s_slot[x].o[ix.blk][ix.r4][ix.lane];
      }
      __builtin_amdgcn_sched_barrier(0);
      float run = kNegInf;
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        if (runs >> x & 1) run = kNegInf;
        run = fmaxf(run, m[x]);
        M[x] = run;
      }
#pragma unroll
      for (int x = NW - 2; x >= 0; --x)
        if (!(runs >> (x + 1) & 1)) M[x] = M[x + 1];
      float sum = 0.f;
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        f[x] = fast_exp2(m[x] - (M[x] == kNegInf ? 0.f : M[x]));
        if (runs >> x & 1) sum = 0.f;
        sum += (l0[x] + l1[x]) * f[x];
        Ls[x] = sum;
      }
#pragma unroll
      for (int x = NW - 2; x >= 0; --x)
        if (!(runs >> (x + 1) & 1)) Ls[x] = Ls[x + 1];
      // Every thread runs the loop (the piece descriptors are read across
      // lanes with readlane, which needs all lanes active); only heads below
      // h/G store.
      const bool real_head = hd < a.hg;
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) {
        const int e = threadIdx.x + kw * NW * 64;
        const SlotIndex ix(e);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < NW; ++x) {
          if (runs >> x & 1) acc = f32x4{0.f, 0.f, 0.f, 0.f};
          acc += wd[kw][x] * f[x];
          const bool run_end = (x == NW - 1) || (runs >> (x + 1) & 1);
          if (run_end && x < used) {
            const int pp = __popc((unsigned)runs & ((2u << x) - 1)) - 1;  // its piece
            const int bi = __builtin_amdgcn_readlane(p_b, pp);
            const int g = __builtin_amdgcn_readlane(p_g, pp);
            const int flags = __builtin_amdgcn_readlane(p_flags, pp);
            if (real_head) {
              if (flags & 1) {  // the whole segment: normalised output
                const float inv = 1.0f / Ls[x];
                T* op = reinterpret_cast<T*>(a.o) +
                        ((size_t)bi * a.h + (size_t)g * a.hg + hd) * DH + ix.d();
                store4(op, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
              } else {  // a partial record for the combine
                float* rec = a.records + ((size_t)blockIdx.x * 2 + (flags >> 1)) * a.rec_floats;
                *reinterpret_cast<f32x4*>(rec + (size_t)hd * DH + ix.d()) = acc;
                if (e < 32) {
                  rec[(size_t)a.hg * DH + hd] = M[x];
                  rec[(size_t)a.hg * DH + a.hg + hd] = Ls[x];
                }
              }
            }
          }
        }
      }
    }
    first_round = false;
    if (more()) __syncthreads();  // the slots are reused
  }

  if constexpr (WHOLE) {
    // This workgroup's sequences: zeros for those with nothing visible, and
    // after an append the lens bump (no other workgroup reads these entries,
    // and this one has read them for the last time).  A full cache or a
    // negative length keeps its lens and sets the error flag, as the combine
    // does otherwise.
    for (int c0 = s_begin + wave * 64; c0 < s_end; c0 += NW * 64) {
      const int bi = c0 + lane;
      // (the first 64 entries as read at the start: no second round trip)
      const int raw = bi >= s_end ? 0 : c0 == s_begin ? raw_first : a.lens[bi];
      uint64_t empty = __ballot(bi < s_end && tiles_of(seq_view_raw(a, raw)) == 0);
      while (empty) {
        const int be = c0 + __builtin_ctzll(empty);
        empty &= empty - 1;
        T* op = reinterpret_cast<T*>(a.o) + (size_t)be * a.h * DH;
        for (int e = lane; e < a.h * DH / 4; e += 64) store4(op + 4 * e, 0.f, 0.f, 0.f, 0.f);
      }
      if (a.k_new && bi < s_end) {
        if (raw >= 0 && raw < a.m_cap)
          a.lens[bi] = raw + 1;
        else if (a.err_flag)
          *a.err_flag = 1;
      }
    }
    return;
  }

  // Workgroup 0 writes the schedule header for the combine and zeros the rows
  // of sequences with nothing visible.  Both are stores; they come after the
  // streaming, because a wave's loads wait for the stores it issued earlier.
  if (blockIdx.x == 0 && wave == 0) {  // the units prefix, for the combine
    if (blk) {  // one round trip and one scan, as in pass 1
      load_block();
      int uk[kLensRegs], s = 0;
#pragma unroll
      for (int k = 0; k < kLensRegs; ++k) {
        const int v = blk_tiles(k);
        uk[k] = v > 0 ? v + lead : 0;
        s += uk[k];
      }
      int run = wave_incl_scan(s) - s;
#pragma unroll
      for (int k = 0; k < kLensRegs; ++k) {
        const int i = kLensRegs * lane + k;
        if (i < a.b) a.prefix[i] = run;
        run += uk[k];
      }
    } else {  // one chunk per lane set; up to kLensRegs chunks per round trip
      int run = 0;
      for (int g0 = 0; g0 < nchunks; g0 += kLensRegs) {
        if (nchunks > 1) load_chunks(g0);
#pragma unroll
        for (int k = 0; k < kLensRegs; ++k) {
          if (g0 + k >= nchunks) break;
          const int c = (g0 + k) * 64;
          int v = v0, incl = incl0;
          if (nchunks > 1) {
            v = (c + lane < a.b) ? tiles_of(seq_view_raw(a, rawr[k])) : 0;
            incl = wave_incl_scan(v);
          }
          int u, u_incl;
          chunk_units(v, incl, u, u_incl);
          if (c + lane < a.b) a.prefix[c + lane] = run + u_incl - u;
          run += __builtin_amdgcn_readlane(u_incl, 63);
        }
      }
    }
    if (lane == 0) {
      a.prefix[a.b] = total;
      a.prefix[a.b + 1] = nonempty;
      a.prefix[a.b + 2] = lead;
      a.prefix[a.b + 3] = W;
    }
  }

  // Sequences with nothing visible get zeros; wave k of workgroup 0 checks
  // sequences k*64 .. k*64+63, NW*64 at a time, and writes their rows.
  if (blockIdx.x == 0) {
    constexpr int kZ = 4;  // chunks per round trip
    for (int c0 = wave * 64; c0 < a.b; c0 += kZ * NW * 64) {
      int rz[kZ];
#pragma unroll
      for (int z = 0; z < kZ; ++z) {
        const int c = c0 + z * NW * 64, i = c + lane;
        rz[z] = 0;
        if (c == 0 && nchunks == 1) rz[z] = raw0;
        else if (c < a.b) rz[z] = a.lens[i < a.b ? i : a.b - 1];
      }
#pragma unroll
      for (int z = 0; z < kZ; ++z) {
        const int c = c0 + z * NW * 64;
        if (c >= a.b) break;
        uint64_t empty = __ballot(c + lane < a.b && tiles_of(seq_view_raw(a, rz[z])) == 0);
        while (empty) {
          const int bi = c + __builtin_ctzll(empty);
          empty &= empty - 1;
          T* op = reinterpret_cast<T*>(a.o) + (size_t)bi * a.h * DH;
          for (int e = lane; e < a.h * DH / 4; e += 64) store4(op + 4 * e, 0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  }
}

// --------------------------------------------------------- combine kernel ----

struct CombineArgs {
  const int32_t* prefix;
  const float* records;
  int32_t* lens;         // bumped when the decode appended
  int32_t* err_flag;     // nullable
  char* o;
  int b, h, G, hg, m_cap, rec_floats;
  int append;
};

// Merge of the partial records of one (sequence, group) segment:
// M = max_k m_k, weights f_k = exp2(m_k - M), o = sum_k f_k acc_k / sum_k f_k l_k
// (the softmax re-associated exactly).  Thread (head, d4) fetches a whole
// batch of records at once -- its float4 of every accumulator plus the head's
// max and sum, which the 32 threads of a head read at one address -- so a
// batch costs one memory round trip; there is no LDS and no barrier.
// Block (seg, y) handles the heads [y*HPB, (y+1)*HPB) of segment seg.
//
// Every workgroup in [wf, wl] took tiles of this segment and wrote a record
// for it (every range of units holds a tile: the effective grid keeps ranges
// longer than a lead-in): slot 1 for wf when its range began in an earlier
// segment, slot 0 otherwise.
template <typename T, int DH, int NT>
__global__ __launch_bounds__(NT) void combine_kernel(CombineArgs a) {
  constexpr int kD4 = DH / 4;            // float4 words per head row
  constexpr int HPB = NT / kD4;          // heads per block
  constexpr int kBatch = 16;             // records per round trip

  // A block of its own (x = b*G, launched only when appending) bumps lens,
  // so that no merge waits behind its load and store.
  if ((int)blockIdx.x == a.b * a.G) {
    if (blockIdx.y != 0) return;
    int over = 0;
    for (int bi = threadIdx.x; bi < a.b; bi += NT) {
      const int raw = a.lens[bi];
      if (raw >= 0 && raw < a.m_cap) a.lens[bi] = raw + 1;
      else over = 1;
    }
    if (over && a.err_flag) *a.err_flag = 1;
    return;
  }

  const int seg = blockIdx.x;
  const int bi = a.G == 1 ? seg : seg / a.G, g = a.G == 1 ? 0 : seg % a.G;
  // every header entry in one memory round trip, before any branch on them:
  // scalar loads (the header is uniform and read-only here)
  using cint = const __attribute__((address_space(4))) int32_t;
  cint* const hdr = (cint*)(a.prefix);
  const int p_bi = hdr[bi];
  const int p_next = hdr[bi + 1];
  const int p_total = hdr[a.b];
  const int lead = hdr[a.b + 2];  // as the decode chose it
  const int W = hdr[a.b + 3];
  // (kept ahead of the early return: the compiler would sink the loads of
  // the last three below it, a second round trip)
  asm volatile("" : : "s"(p_bi), "s"(p_next), "s"(p_total), "s"(lead), "s"(W));
  const int unit = p_next - p_bi;      // lead-in units + tiles, or 0
  if (unit == 0) return;
  const int nb = unit - lead;
  const int Tt = p_total * a.G;  // units (below 2^30 by the shape check)
  const int U0 = p_bi * a.G + g * unit;  // first unit
  const int S0 = U0 + lead;              // first tile
  const int wf = wg_of(S0, Tt, W), wl = wg_of(S0 + nb - 1, Tt, W);
  if (wf == wl) return;  // one workgroup covered the segment and wrote it
  // wf's range began in an earlier segment (whose last tile is unit U0 - 1)
  const int first_slot = (wg_start(Tt, wf, W) < U0) ? 1 : 0;

  const int hl = threadIdx.x / kD4, d4 = threadIdx.x % kD4;
  const int hd = blockIdx.y * HPB + hl;
  if (hd >= a.hg) return;
  const float* acc_at = a.records + (size_t)hd * DH + 4 * d4;
  const float* m_at = a.records + (size_t)a.hg * DH + hd;
  const float* l_at = m_at + a.hg;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float M = kNegInf, lsum = 0.f;
  for (int w0 = wf; w0 <= wl; w0 += kBatch) {
    f32x4 x[kBatch];
    float m[kBatch], l[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int w = w0 + u;
      x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[u] = kNegInf;
      l[u] = 0.f;
      if (w <= wl) {
        const size_t r = (size_t)(2 * w + (w == wf ? first_slot : 0)) * a.rec_floats;
        x[u] = *reinterpret_cast<const f32x4*>(acc_at + r);
        m[u] = m_at[r];
        l[u] = l_at[r];
      }
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) Mn = fmaxf(Mn, m[u]);
    const float Ms = (Mn == kNegInf) ? 0.f : Mn;
    const float sc = fast_exp2(M - Ms);
    acc *= sc;
    lsum *= sc;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float f = fast_exp2(m[u] - Ms);
      acc += x[u] * f;
      lsum += l[u] * f;
    }
    M = Mn;
  }
  const float inv = 1.0f / lsum;
  T* op = reinterpret_cast<T*>(a.o) + ((size_t)bi * a.h + (size_t)g * a.hg + hd) * DH + 4 * d4;
  store4(op, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
}

// ------------------------------------------------------------------- host ----

size_t decode_record_bytes(int hg, int dh) {
  size_t f = (size_t)hg * dh + 2 * (size_t)hg;
  f = (f + 3) & ~(size_t)3;  // 16-byte multiple
  return f * sizeof(float);
}

// Schedule header: the [b + 1] units prefix, the count of non-empty
// sequences, the lead-in and the effective grid, padded to 256 bytes.
size_t decode_records_offset(int b) {
  return (((size_t)b + 4) * sizeof(int32_t) + 255) & ~(size_t)255;
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
// Threads per combine block: a block merges kCombineThreads / (d_h / 4)
// heads of one segment.  Small blocks spread the records of a small step over
// many CUs (a CU streams only ~20 GB/s).
constexpr int kCombineThreads = 128;
// Cache capacity (tiles) up to which a decode takes whole sequences per
// workgroup and skips the combine (see launch_decode_t).
constexpr int kWholeMaxTiles = 8;

// Workgroups of the decode launch for these shapes on the current device:
// CUs x occupancy, cut to the largest grid the shapes can use.
template <typename T, int DH>
hipError_t decode_grid_t(const DecodeParams& p, int* grid_out) {
  auto kern = decode_kernel<T, DH, kDecodeWaves, false>;
  int dev = 0;
  const int cus = current_device_cus(&dev);
  if (cus <= 0) return hipErrorInvalidDevice;
  static int occ_cache[64];
  int occ = (dev >= 0 && dev < 64) ? occ_cache[dev] : 0;
  if (occ <= 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kDecodeWaves * 64, 0);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    if (dev >= 0 && dev < 64) occ_cache[dev] = occ;
  }
  int grid = cus * occ;
  // Tuning override of the grid (workgroups); never above the cap.
  static const int grid_env = [] {
    const char* e = getenv("MQA_DECODE_GRID");
    return e ? atoi(e) : 0;
  }();
  if (grid_env > 0) grid = grid_env;
  const int cap = decode_grid_cap(p.b, p.G, p.m_cap);
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  *grid_out = grid;
  return hipSuccess;
}

hipError_t decode_grid(const DecodeParams& p, int* grid) {
  if (p.dtype == 1) {
    if (p.dh == 128) return decode_grid_t<__bf16, 128>(p, grid);
    return decode_grid_t<__bf16, 64>(p, grid);
  }
  if (p.dh == 128) return decode_grid_t<float, 128>(p, grid);
  return decode_grid_t<float, 64>(p, grid);
}

template <typename T, int DH>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  int grid = 0;
  if (hipError_t e = decode_grid_t<T, DH>(p, &grid); e != hipSuccess) return e;

  DecodeArgs a;
  a.q = (const char*)p.q;
  a.k = (char*)p.k;
  a.v = (char*)p.v;
  a.lens = const_cast<int32_t*>(p.lens);
  a.k_new = (const char*)p.k_new;
  a.v_new = (const char*)p.v_new;
  a.err_flag = p.err_flag;
  a.o = (char*)p.o;
  a.prefix = (int32_t*)p.ws;
  a.records = (float*)((char*)p.ws + decode_records_offset(p.b));
  a.b = p.b;
  a.h = p.h;
  a.G = p.G;
  a.hg = p.h / p.G;
  a.m_cap = p.m_cap;
  a.window = p.window;
  a.rec_floats = (int)(decode_record_bytes(a.hg, DH) / sizeof(float));
  a.scale_log2 = (float)((double)p.scale * 1.4426950408889634);
  // Short caches: workgroup w takes sequences [b w / W, b (w + 1) / W) whole
  // (every group), reading only their lens entries, so it writes no partial
  // record and bumps their lens itself after an append: the combine is not
  // launched.  (With longer caches, a count split would leave the work too
  // uneven.)
  const bool whole = (p.m_cap + kTileRows - 1) / kTileRows <= kWholeMaxTiles;
  hipError_t e;
  if (p.ev_begin && (e = hipEventRecord(p.ev_begin, s)) != hipSuccess) return e;
  if (whole)
    hipLaunchKernelGGL((decode_kernel<T, DH, kDecodeWaves, true>), dim3(grid),
                       dim3(kDecodeWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, DH, kDecodeWaves, false>), dim3(grid),
                       dim3(kDecodeWaves * 64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_end && (e = hipEventRecord(p.ev_end, s)) != hipSuccess) return e;
  if (whole) return hipSuccess;

  CombineArgs ca;
  ca.prefix = a.prefix;
  ca.records = a.records;
  ca.lens = a.lens;
  ca.err_flag = a.err_flag;
  ca.o = a.o;
  ca.b = p.b;
  ca.h = p.h;
  ca.G = p.G;
  ca.hg = a.hg;
  ca.m_cap = p.m_cap;
  ca.rec_floats = a.rec_floats;
  ca.append = p.k_new != nullptr;
  constexpr int kHeadsPerBlock = kCombineThreads / (DH / 4);
  dim3 cgrid((unsigned)(p.b * p.G + (ca.append ? 1 : 0)),
             (unsigned)((a.hg + kHeadsPerBlock - 1) / kHeadsPerBlock));
  hipLaunchKernelGGL((combine_kernel<T, DH, kCombineThreads>), cgrid, dim3(kCombineThreads), 0, s,
                     ca);
  return hipGetLastError();
}

}  // namespace

hipError_t decode_launch_workspace_bytes(const DecodeParams& p, size_t* bytes) {
  int grid = 0;
  if (hipError_t e = decode_grid(p, &grid); e != hipSuccess) return e;
  const int hg = p.h / p.G;
  *bytes = decode_records_offset(p.b) + 2 * (size_t)grid * decode_record_bytes(hg, p.dh);
  return hipSuccess;
}

// The fixed workspace of the decode variant that allocates nothing.  Host
// code never passes this name to a kernel (on the host it only stands in for
// the symbol): it passes the device address that noalloc_scratch looked up.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (p.dtype == 1) {
    if (p.dh == 128) return launch_decode_t<__bf16, 128>(p, s);
    return launch_decode_t<__bf16, 64>(p, s);
  }
  if (p.dh == 128) return launch_decode_t<float, 128>(p, s);
  return launch_decode_t<float, 64>(p, s);
}

}  // namespace mqa
