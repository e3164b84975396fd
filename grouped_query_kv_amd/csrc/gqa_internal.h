// Internal interface between the validating host layer (gqa_api.cpp) and the
// kernel launchers (*.hip). Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gqa.h"

namespace gqa {

// Everything a launcher needs, already validated against the host lengths.
struct Problem {
  int B, S, H, Hkv, G, D, M;
  int dtype;              // gqa_dtype
  int window;             // -1 off, else 1..M
  int cap;                // an evicting sequence keeps min(L, max(0, cap - S)) rows: M, or W when greedy
  float scale;            // resolved (never 0)
  // rotary (rot == 0: none)
  int rot;
  const float* cos;
  const float* sin;
  int rot_rows;
  int interleaved;
  // absolute position of each sequence's buffer row 0 (nullptr: 0); rotary
  // positions are offset_b + L_b + i (host copy for planning, device copy
  // for kernels that cannot take it in their arguments)
  const int32_t* off_host = nullptr;
  const int32_t* off_dev = nullptr;
  // tensors
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  void* out;
  const int32_t* lens_dev;
  const int32_t* lens_host;
  // additive bias (bias == nullptr: none): element of (b, h, i, column) at
  // b * bias_bs + h * bias_hs + i * bias_T + column (strides 0 broadcast)
  const void* bias = nullptr;
  int64_t bias_bs = 0, bias_hs = 0;
  int bias_T = 0;
  // windowed chunk on the MFMA prefill (stage_k != nullptr): M is the
  // staging frame's row count (M + S of the cache); keys from each
  // sequence's 64-aligned past length on are read from the frame, earlier
  // ones from k_cache/v_cache, whose row count is cache_rows
  const void* stage_k = nullptr;
  const void* stage_v = nullptr;
  int cache_rows = 0;
  // separate past buffers read by the split-KV decode, which writes every
  // past row it reads into k_cache/v_cache at the same row (past_k !=
  // nullptr; past_rows rows per (b, kv head)); only when the decode reads
  // rows [0, L_b) of every sequence (no eviction, window off or covering)
  const void* past_k = nullptr;
  const void* past_v = nullptr;
  int past_rows = 0;
};

// Workspace carving (byte offsets from the workspace base). The layout is a
// function of the shape only, so one allocation serves every call.
struct WorkspaceLayout {
  size_t counters;        // int32 [B, Hkv, hg_max] merge counters (kept zero)
  size_t counters_bytes;
  size_t scratch;         // shared by decode partials and eviction halos
  size_t scratch_bytes;
  size_t decode_halo;     // fused-eviction halo rows, after the decode partials
  size_t prefill_counters;  // int32 [prefill row blocks] split counters (kept zero)
  size_t prefill_counters_bytes;
  size_t prefill_partials;  // split partials of the prefill kernel (in the scratch area)
  // windowed chunk (S > 1, a window, some sequence evicting): K and V staging
  // frames [B, Hkv, stage_rows, D], stage_rows = M + S, in which attention
  // sees each sequence before its eviction (0 bytes when not needed)
  size_t stage_k, stage_v, stage_bytes;
  int stage_rows;
  size_t total;
};

// Prefill: 256 query rows per workgroup. When a call has too few row blocks
// to fill the chip, each row block's key tiles are cut into up to
// kPrefillMaxSplits ranges taken by separate workgroups and merged by the
// last one to finish; the host sizes the ranges to the lengths (the plan in
// the launch). A range's partial holds, for each of the 512 lanes, its 64
// unnormalised output values, the row's exponent base and its weight sum
// (fp32).
constexpr int kPrefillWgRows = 256;
constexpr int kPrefillTargetWorkgroups = 256;   // one per CU
constexpr int kPrefillMaxSplits = 4;            // slots per row block in the workspace
constexpr int kPrefillPlanMax = 512;            // workgroups a split plan can list
constexpr size_t kPrefillSlotFloats = 512 * 32 + 2 * 512;

// A function of the shape only (the workspace is sized from it): whether the
// row blocks may be split, i.e. they fill less than three quarters of the
// chip and the buffer holds at least 8 tiles of 64 keys per extra range.
inline bool prefill_may_split(int64_t B, int64_t S, int64_t G, int64_t Hkv, int64_t M) {
  const int64_t items = ((S * G + kPrefillWgRows - 1) / kPrefillWgRows) * B * Hkv;
  if (items <= 0 || 4 * items >= 3 * kPrefillTargetWorkgroups) return false;
  return ((M + 63) / 64) / 8 >= 2;
}

// Decode: fast split-KV kernel limits.
#ifndef GQA_DECODE_WG_WAVES
#define GQA_DECODE_WG_WAVES 8
#endif
constexpr int kDecodeWaves = GQA_DECODE_WG_WAVES;  // waves per workgroup
#ifndef GQA_DECODE_WORKGROUPS
#define GQA_DECODE_WORKGROUPS 256
#endif
constexpr int kDecodeMaxWorkgroups = GQA_DECODE_WORKGROUPS;  // per launch: one per CU, all resident
constexpr int kDecodeMaxWorkers = kDecodeMaxWorkgroups * kDecodeWaves;  // waves taking a slice
constexpr int kDecodeMaxHG = 16;         // query heads per unit (the 16 MFMA columns)
constexpr int kDecodeArgBatch = 64;      // largest batch the fast decode plans in its arguments

// Eviction (parallel form): chunks of kEvictChunkRows rows, one thread per
// 16-byte column of a chunk; halo copies are used up to kEvictHaloMax
// dropped rows, the serial form beyond.
constexpr int kEvictHaloMax = 4;          // largest drop the parallel eviction handles
constexpr int kEvictThreads = 256;
constexpr int kEvictUnitsPerThread = 16;  // serial eviction: units per thread per pass
#ifndef GQA_EVICT_CHUNK_ROWS
#define GQA_EVICT_CHUNK_ROWS 128
#endif
#ifndef GQA_EVICT_ROWS_IN_FLIGHT
#define GQA_EVICT_ROWS_IN_FLIGHT 8
#endif
constexpr int kEvictChunkRows = GQA_EVICT_CHUNK_ROWS;       // rows per chunk of the parallel eviction
constexpr int kEvictRowsInFlight = GQA_EVICT_ROWS_IN_FLIGHT;  // rows of one column a thread has in flight

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Every tensor the kernels read or write in 16-byte vector units (Q, the new
// K/V rows, the caches, the output, a separate past) must start at a
// multiple of this many bytes.
constexpr int kTensorAlign = 16;

// Rows a sequence of length L keeps before its S new rows: all of them when
// they fit, else the min(L, max(0, cap - S)) most recent (cap = M keeps the
// min(L + S, M) most recent tokens in all; cap = W < M is greedy eviction).
inline int kept_rows_host(int L, int S, int M, int cap) {
  if (L + S <= M) return L;
  const int k = cap - S > 0 ? cap - S : 0;
  return L < k ? L : k;
}

// Eviction copy unit and rows per workgroup chunk for a row of `row_bytes`.
struct EvictGeometry {
  int unit;        // bytes moved per access: 16, 4 or 2
  int chunk_rows;  // rows per workgroup chunk (>= 1)
};
inline EvictGeometry evict_geometry(int row_bytes) {
  EvictGeometry g;
  g.unit = (row_bytes % 16 == 0) ? 16 : ((row_bytes % 4 == 0) ? 4 : 2);
  g.chunk_rows = kEvictChunkRows;
  return g;
}

// `window` is the call's local_window_size (-1 when off); with a window and
// S > 1 the layout includes the staging frames.
WorkspaceLayout workspace_layout(const gqa_shape& s, int window);

// The device scratch of gqa_attention_decode_noalloc: a static array of
// GQA_NOALLOC_SCRATCH_BYTES per GPU. Its first kStaticCounterArea bytes hold
// only merge counters (decode counters from 0, prefill split counters from
// kStaticCounterArea / 2), zeroed once per device and left at zero by every
// successful call; the other regions of a call's layout start at
// kStaticCounterArea.
constexpr size_t kStaticCounterArea = size_t(64) << 10;

// The current device's static scratch for one call: its device address and
// whether its counter area must be zeroed first (the device's first call,
// or the first after a call that failed in a launch).
struct StaticScratch {
  int device = -1;
  void* ptr = nullptr;
  bool clear = false;
};
// Look up (once per device, with hipGetSymbolAddress) the scratch of the
// current device. GQA_ERR_HIP if the device or the symbol is unavailable.
gqa_status static_scratch_begin(StaticScratch* sc);
// After the call's launches: a call that zeroed the counters leaves them
// zero for the next one; a call that failed in a launch marks them dirty.
void static_scratch_end(const StaticScratch& sc, gqa_status st);

// Zero `bytes` (a multiple of 16) at `p` with a fill kernel on `st`.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

// Record a failure message for gqa_last_error() (printf-style).
gqa_status set_error(gqa_status s, const char* fmt, ...);

// Rows of the staging frame the windowed chunk path fills before attention:
// key tiles of the attention kernels start at multiples of this, so every
// row of a visited tile holds a real key.
constexpr int kStageAlignRows = 64;

// Copy rows [lo_b, min(L_b, src_rows)) of every (b, kv head) of K and V
// from buffers of src_rows rows per head to buffers of dst_rows rows per
// head, at the same row numbers; lo_b = 0 with window <= 0, else
// max(0, L_b - window + 1) rounded down to kStageAlignRows. max_len is the
// largest L_b (host copy), which sizes the grid.
hipError_t launch_copy_prefix(const void* src_k, const void* src_v, int src_rows, void* dst_k,
                              void* dst_v, int dst_rows, const int32_t* lens_dev, int B, int Hkv,
                              int row_bytes, int window, int max_len, hipStream_t st);

// Launchers. They assume validated arguments and return the first HIP error.
hipError_t launch_append(const Problem& p, bool evicted_lengths, hipStream_t st);

// Eviction for `incoming` tokens; max_drop = max_b d_b from the host lengths.
hipError_t launch_evict(const Problem& p, int incoming, int max_drop, void* ws,
                        const WorkspaceLayout& lay, hipStream_t st);

// Plain attention (any dtype, D <= 256): reads keys from the cache, which
// must already hold this call's appended rows.
hipError_t launch_attention_simple(const Problem& p, hipStream_t st);

// Fast decode (fp16/bf16, D == 128 or 64, S == 1): fused append + split-KV + merge.
bool decode_fast_supported(const Problem& p);
// Eviction folded into the decode (the window covers the buffer, one head
// group per kv head): each kept row is moved by the wave that reads it.
bool decode_fused_evict_supported(const Problem& p);
hipError_t launch_decode_fast(const Problem& p, void* ws, const WorkspaceLayout& lay,
                              hipStream_t st, bool fuse_evict);

// Fast prefill (fp16/bf16, D == 128 or 64): MFMA flash attention over the cache.
bool prefill_fast_supported(const Problem& p);
hipError_t launch_prefill_fast(const Problem& p, void* ws, const WorkspaceLayout& lay,
                               hipStream_t st);

}  // namespace gqa
