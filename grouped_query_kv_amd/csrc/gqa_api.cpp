// Host side of the C ABI: argument validation (complete before any launch),
// workspace carving and kernel dispatch. See include/gqa.h for the contract.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "gqa_internal.h"

namespace gqa {
namespace {

thread_local char g_err[512] = "";

gqa_status fail(gqa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gqa_status hip_fail(hipError_t e, const char* where) {
  return fail(GQA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

int elem_bytes(int dtype) { return dtype == GQA_FP32 ? 4 : 2; }

enum Entry { kAppend, kPrefill, kDecode };

// Shape checks shared by every entry point.
gqa_status check_shape(const gqa_shape* s, bool need_heads) {
  if (!s) return fail(GQA_ERR_INVALID_ARG, "shape is NULL");
  if (s->dtype != GQA_FP32 && s->dtype != GQA_FP16 && s->dtype != GQA_BF16)
    return fail(GQA_ERR_INVALID_ARG, "unknown dtype %d", s->dtype);
  if (s->batch < 0) return fail(GQA_ERR_INVALID_ARG, "batch %d < 0", s->batch);
  if (s->kv_num_heads < 1) return fail(GQA_ERR_INVALID_ARG, "kv_num_heads %d < 1", s->kv_num_heads);
  if (need_heads) {
    if (s->num_heads < 1) return fail(GQA_ERR_INVALID_ARG, "num_heads %d < 1", s->num_heads);
    if (s->num_heads % s->kv_num_heads)
      return fail(GQA_ERR_INVALID_ARG, "num_heads %d not a multiple of kv_num_heads %d",
                  s->num_heads, s->kv_num_heads);
  }
  if (s->head_size < 1 || s->head_size > 256)
    return fail(GQA_ERR_INVALID_ARG, "head_size %d outside 1..256", s->head_size);
  if (s->max_seq_len < 1) return fail(GQA_ERR_INVALID_ARG, "max_seq_len %d < 1", s->max_seq_len);
  return GQA_OK;
}

gqa_status check_lengths(const gqa_shape* s, const int32_t* host, const int32_t* dev) {
  if (s->batch == 0) return GQA_OK;
  if (!host) return fail(GQA_ERR_INVALID_ARG, "seqlens_k_host is NULL");
  if (!dev) return fail(GQA_ERR_INVALID_ARG, "seqlens_k_dev is NULL");
  for (int b = 0; b < s->batch; ++b)
    if (host[b] < 0 || host[b] > s->max_seq_len)
      return fail(GQA_ERR_INVALID_ARG, "seqlens_k[%d] = %d outside 0..%d", b, host[b],
                  s->max_seq_len);
  return GQA_OK;
}

// Full validation of an append / attention call; fills `p` on success.
gqa_status validate(Entry entry, const gqa_shape* s, const gqa_options* o, const void* q,
                    const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* lens_host, const int32_t* lens_dev, void* out,
                    Problem* p, bool* needs_evict, int* max_drop) {
  gqa_status st = check_shape(s, true);
  if (st != GQA_OK) return st;
  if (!o) return fail(GQA_ERR_INVALID_ARG, "options is NULL");
  const int B = s->batch, S = s->new_tokens, D = s->head_size, M = s->max_seq_len;
  if (S < 0) return fail(GQA_ERR_INVALID_ARG, "new_tokens %d < 0", S);
  if (entry != kAppend && S < 1) return fail(GQA_ERR_INVALID_ARG, "new_tokens must be >= 1");
  if (entry == kDecode && S != 1) return fail(GQA_ERR_INVALID_ARG, "decode needs new_tokens == 1");
  const int W = o->local_window_size;
  if (!(W == -1 || (W >= 1 && W <= M)))
    return fail(GQA_ERR_INVALID_ARG, "local_window_size %d not -1 or 1..%d", W, M);
  if (!isfinite(o->scale)) return fail(GQA_ERR_INVALID_ARG, "scale is not finite");
  st = check_lengths(s, lens_host, lens_dev);
  if (st != GQA_OK) return st;
  const bool rot = o->cos_cache != nullptr || o->sin_cache != nullptr;
  const bool offsets = o->position_offset_host != nullptr || o->position_offset_dev != nullptr;
  if (offsets && B > 0 && (!o->position_offset_host || !o->position_offset_dev))
    return fail(GQA_ERR_INVALID_ARG,
                "position_offset_host and position_offset_dev must be given together");
  int64_t maxpos = 0;            // largest offset_b + L_b
  for (int b = 0; b < B; ++b) {
    const int64_t off = offsets ? o->position_offset_host[b] : 0;
    if (off < 0)
      return fail(GQA_ERR_INVALID_ARG, "position_offset[%d] = %lld < 0", b, (long long)off);
    maxpos = std::max(maxpos, off + lens_host[b]);
  }
  if (rot) {
    if (!o->cos_cache || !o->sin_cache)
      return fail(GQA_ERR_INVALID_ARG, "cos_cache and sin_cache must be given together");
    if (D % 2) return fail(GQA_ERR_INVALID_ARG, "rotary needs an even head_size (got %d)", D);
    if (B > 0 && S > 0 && maxpos + S > (int64_t)o->rotary_rows)
      return fail(GQA_ERR_INVALID_ARG, "rotary table has %d rows, positions reach %lld",
                  o->rotary_rows, (long long)(maxpos + S - 1));
  }
  const bool work = B > 0 && S > 0;
  if (work) {
    if (!k_new || !v_new || !k_cache || !v_cache)
      return fail(GQA_ERR_INVALID_ARG, "a K/V pointer is NULL");
    if (entry != kAppend && (!q || !out)) return fail(GQA_ERR_INVALID_ARG, "q or out is NULL");
    const uintptr_t bits = uintptr_t(k_new) | uintptr_t(v_new) | uintptr_t(k_cache) |
                           uintptr_t(v_cache) |
                           (entry != kAppend ? uintptr_t(q) | uintptr_t(out) : uintptr_t(0));
    if (bits & (kTensorAlign - 1))
      return fail(GQA_ERR_INVALID_ARG, "q, k_new, v_new, the caches and out must be %d-byte aligned",
                  kTensorAlign);
  }
  const bool windowed = W > 0 && entry != kAppend;
  const bool greedy = o->greedy_eviction != 0 && entry != kAppend;
  if (greedy && !windowed)
    return fail(GQA_ERR_INVALID_ARG, "greedy_eviction needs a window (local_window_size > 0)");
  const int cap = greedy ? W : M;
  *needs_evict = false;
  *max_drop = 0;
  if (windowed) {
    if (S > M) return fail(GQA_ERR_INVALID_ARG, "new_tokens %d > max_seq_len %d", S, M);
    for (int b = 0; b < B; ++b)
      *max_drop = std::max(*max_drop, lens_host[b] - kept_rows_host(lens_host[b], S, M, cap));
    *needs_evict = *max_drop > 0;
  } else {
    for (int b = 0; b < B; ++b)
      if (int64_t(lens_host[b]) + S > M)
        return fail(GQA_ERR_NO_ROOM, "sequence %d: %d past + %d new > max_seq_len %d", b,
                    lens_host[b], S, M);
  }
  const int64_t H = s->num_heads;
  const bool biased = o->attention_bias != nullptr && entry != kAppend;
  if (biased) {
    if (o->bias_batch != 1 && o->bias_batch != B)
      return fail(GQA_ERR_INVALID_ARG, "bias_batch %d is neither 1 nor batch %d", o->bias_batch, B);
    if (o->bias_heads != 1 && o->bias_heads != H)
      return fail(GQA_ERR_INVALID_ARG, "bias_heads %d is neither 1 nor num_heads %d",
                  o->bias_heads, (int)H);
    int64_t need = 1;
    for (int b = 0; b < B; ++b) need = std::max(need, int64_t(lens_host[b]) + S);
    if (o->bias_total < need)
      return fail(GQA_ERR_INVALID_ARG, "bias_total %d < %lld (past + new tokens)", o->bias_total,
                  (long long)need);
  }
  Problem& P = *p;
  P.bias = biased ? o->attention_bias : nullptr;
  P.bias_T = biased ? o->bias_total : 0;
  P.bias_hs = biased && o->bias_heads != 1 ? int64_t(S) * o->bias_total : 0;
  P.bias_bs = biased && o->bias_batch != 1 ? int64_t(o->bias_heads) * S * o->bias_total : 0;
  P.B = B; P.S = S; P.H = s->num_heads; P.Hkv = s->kv_num_heads; P.G = P.H / P.Hkv;
  P.D = D; P.M = M; P.dtype = s->dtype; P.window = W; P.cap = cap;
  P.scale = o->scale != 0.0f ? o->scale : 1.0f / sqrtf((float)D);
  P.rot = rot; P.cos = o->cos_cache; P.sin = o->sin_cache; P.rot_rows = o->rotary_rows;
  P.interleaved = o->rotary_interleaved != 0;
  P.off_host = offsets && B > 0 ? o->position_offset_host : nullptr;
  P.off_dev = offsets && B > 0 ? o->position_offset_dev : nullptr;
  P.q = q; P.k_new = k_new; P.v_new = v_new; P.k_cache = k_cache; P.v_cache = v_cache;
  P.out = out; P.lens_dev = lens_dev; P.lens_host = lens_host;
  return GQA_OK;
}

gqa_status check_workspace(const gqa_shape* s, int window, void* ws, size_t bytes,
                           WorkspaceLayout* lay) {
  *lay = workspace_layout(*s, window);
  if (lay->total == 0) return GQA_OK;
  if (!ws) return fail(GQA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", lay->total);
  if (bytes < lay->total)
    return fail(GQA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", bytes, lay->total);
  return GQA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Attention over one call's rows on the buffers the Problem names (the new
// rows already appended there).
hipError_t attend(const Problem& P, void* ws, const WorkspaceLayout& lay, hipStream_t hs) {
  return prefill_fast_supported(P) ? launch_prefill_fast(P, ws, lay, hs)
                                   : launch_attention_simple(P, hs);
}

// S > 1 with a window where some sequence must evict. Queries early in the
// chunk see keys the eviction drops, so attention runs first over each
// sequence as it stands before the eviction (past ++ new): in staging frames
// of M + S rows per (b, kv head) in the workspace, where buffer row = position
// in the sequence, so rotary positions stay L_b + i. Only the past rows the
// window can reach are copied in (from the tile holding L_b - W + 1 on). The
// cache itself then takes the ordinary eviction and the append at the
// compacted lengths, exactly as a one-token step does.
gqa_status windowed_chunk(const Problem& P, int max_drop, void* ws, const WorkspaceLayout& lay,
                          hipStream_t hs) {
  char* base = static_cast<char*>(ws);
  Problem F = P;
  F.M = lay.stage_rows;
  F.cap = F.M;             // the frame holds past ++ new: nothing is evicted there
  F.k_cache = base + lay.stage_k;
  F.v_cache = base + lay.stage_v;
  const int row_bytes = P.D * elem_bytes(P.dtype);
  int max_len = 0;
  for (int b = 0; b < P.B; ++b) max_len = std::max(max_len, P.lens_host[b]);
  // the MFMA kernel reads whole 64-key tiles of the past from the cache
  // itself and only the tile holding L_b and the new rows from the frame;
  // the plain kernel reads everything from the frame, from the tile the
  // window reaches on
  const bool direct = prefill_fast_supported(F);
  // on the MFMA route only a partial tile at L_b has rows to copy
  bool partial = !direct;
  for (int b = 0; b < P.B && !partial; ++b) partial = P.lens_host[b] % kStageAlignRows != 0;
  hipError_t e = hipSuccess;
  if (partial)
    e = launch_copy_prefix(P.k_cache, P.v_cache, P.M, F.k_cache, F.v_cache, F.M, P.lens_dev, P.B,
                           P.Hkv, row_bytes, direct ? 1 : P.window, max_len, hs);
  if (e != hipSuccess) return hip_fail(e, "staging copy");
  e = launch_append(F, false, hs);
  if (e != hipSuccess) return hip_fail(e, "staging append");
  if (direct) {
    Problem A = F;
    A.stage_k = F.k_cache;
    A.stage_v = F.v_cache;
    A.k_cache = P.k_cache;
    A.v_cache = P.v_cache;
    A.cache_rows = P.M;
    e = launch_prefill_fast(A, ws, lay, hs);
  } else {
    e = attend(F, ws, lay, hs);
  }
  if (e != hipSuccess) return hip_fail(e, "attention");
  e = launch_evict(P, P.S, max_drop, ws, lay, hs);
  if (e != hipSuccess) return hip_fail(e, "eviction");
  e = launch_append(P, true, hs);
  if (e != hipSuccess) return hip_fail(e, "append");
  return GQA_OK;
}

// The layout of a call moved into the static scratch: counters into the
// counter area, every other region after it (same order, same sizes).
gqa_status static_layout(const WorkspaceLayout& lay, WorkspaceLayout* out) {
  constexpr size_t half = kStaticCounterArea / 2;
  if (lay.counters_bytes > half || lay.prefill_counters_bytes > half)
    return fail(GQA_ERR_WORKSPACE, "the call needs %zu + %zu bytes of merge counters, the static "
                "scratch holds %zu + %zu", lay.counters_bytes, lay.prefill_counters_bytes, half, half);
  const size_t delta = kStaticCounterArea - lay.scratch;   // lay.scratch == lay.counters_bytes
  const size_t need = lay.total + delta;
  if (need > size_t(GQA_NOALLOC_SCRATCH_BYTES))
    return fail(GQA_ERR_WORKSPACE, "the call needs %zu bytes of scratch, the static scratch holds "
                "%zu", need, size_t(GQA_NOALLOC_SCRATCH_BYTES));
  WorkspaceLayout s = lay;
  s.counters = 0;
  s.prefill_counters = half;
  s.scratch += delta;
  s.decode_halo += delta;
  s.prefill_partials += delta;
  if (s.stage_bytes) {
    s.stage_k += delta;
    s.stage_v += delta;
  }
  s.total = need;
  *out = s;
  return GQA_OK;
}

// Whether the split-KV decode can read a call's past rows straight from
// separate past buffers and write them to the cache itself: one new token,
// the MFMA decode, nothing evicted, and every row [0, L_b) attended (no
// window, or one that reaches row 0 of every sequence).
bool past_reads_fused(const Problem& P, bool needs_evict) {
  if (P.S != 1 || needs_evict || !decode_fast_supported(P)) return false;
  if (P.window > 0)
    for (int b = 0; b < P.B; ++b)
      if (P.lens_host[b] + 1 > P.window) return false;
  return true;
}

// The kernels of one validated call, on the workspace `ws` carved as `lay`.
// S == 1 takes the split-KV decode route.
gqa_status execute(const Problem& P, bool needs_evict, int max_drop, void* ws,
                   const WorkspaceLayout& lay, hipStream_t hs) {
  hipError_t e;
  if (needs_evict && P.S > 1) return windowed_chunk(P, max_drop, ws, lay, hs);
  const bool fast_decode = P.S == 1 && decode_fast_supported(P);
  const bool fuse_evict = needs_evict && fast_decode && decode_fused_evict_supported(P);
  if (needs_evict && !fuse_evict) {
    e = launch_evict(P, P.S, max_drop, ws, lay, hs);
    if (e != hipSuccess) return hip_fail(e, "eviction");
  }
  const bool evicted_lengths = P.window > 0;
  if (fast_decode) {
    e = launch_decode_fast(P, ws, lay, hs, fuse_evict);
    if (e != hipSuccess) return hip_fail(e, "decode");
    return GQA_OK;
  }
  e = launch_append(P, evicted_lengths, hs);
  if (e != hipSuccess) return hip_fail(e, "append");
  // After an eviction the MFMA kernel still finds each sequence's keys (it
  // applies the same kept-rows rule), but a bias column is then the buffer
  // row plus the dropped count, which its aligned four-column bias loads
  // cannot follow: such calls take the plain kernel.
  e = (needs_evict && P.bias) ? launch_attention_simple(P, hs) : attend(P, ws, lay, hs);
  if (e != hipSuccess) return hip_fail(e, "attention");
  return GQA_OK;
}

// The whole op for one call: validation and the workspace check first (no
// device call before both pass), then the kernels. With static_scratch the
// workspace is the current device's static scratch instead of `ws`.
gqa_status run_attention(Entry entry, const gqa_shape* shape, const gqa_options* opts,
                         const void* q, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, const int32_t* lens_host, const int32_t* lens_dev,
                         void* out, void* ws, size_t ws_bytes, void* stream,
                         bool static_scratch = false, const void* past_k = nullptr,
                         const void* past_v = nullptr, int past_rows = 0) {
  g_err[0] = '\0';
  Problem P;
  bool needs_evict;
  int max_drop;
  gqa_status st = validate(entry, shape, opts, q, k_new, v_new, k_cache, v_cache, lens_host,
                           lens_dev, out, &P, &needs_evict, &max_drop);
  if (st != GQA_OK) return st;
  if (past_k) {
    // the split-KV decode copies the past rows on its way (the caller
    // checked that it reads all of them)
    if (!past_reads_fused(P, needs_evict))
      return fail(GQA_ERR_INVALID_ARG, "fused past copy requested for a call that cannot take it");
    P.past_k = past_k;
    P.past_v = past_v;
    P.past_rows = past_rows;
  }
  WorkspaceLayout lay;
  if (static_scratch) {
    st = static_layout(workspace_layout(*shape, P.window), &lay);
  } else {
    st = check_workspace(shape, P.window, ws, ws_bytes, &lay);
  }
  if (st != GQA_OK) return st;
  if (P.B == 0) return GQA_OK;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (!static_scratch) return execute(P, needs_evict, max_drop, ws, lay, hs);
  StaticScratch sc;
  st = static_scratch_begin(&sc);
  if (st != GQA_OK) return st;
  if (sc.clear) {
    const hipError_t e = launch_zero(sc.ptr, kStaticCounterArea, hs);
    if (e != hipSuccess) {
      static_scratch_end(sc, GQA_ERR_HIP);
      return hip_fail(e, "static scratch counter clear");
    }
  }
  st = execute(P, needs_evict, max_drop, sc.ptr, lay, hs);
  static_scratch_end(sc, st);
  return st;
}

}  // namespace

gqa_status set_error(gqa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

WorkspaceLayout workspace_layout(const gqa_shape& s, int window) {
  WorkspaceLayout l{};
  const int64_t B = s.batch, H = s.num_heads, Hkv = s.kv_num_heads, D = s.head_size;
  const bool staged = window > 0 && s.new_tokens > 1;
  // the windowed chunk path runs the attention kernels on staging frames of
  // M + S rows, so the partials and halos below are sized for that many
  const int64_t M = s.max_seq_len + (staged ? s.new_tokens : 0);
  if (B <= 0 || Hkv <= 0 || D <= 0 || M <= 0) return l;
  const int64_t G = H > 0 && H % Hkv == 0 ? H / Hkv : 1;
  // decode merge counters, one per (b, kv head, head group)
  const int64_t hg = (G + kDecodeMaxHG - 1) / kDecodeMaxHG;
  l.counters = 0;
  l.counters_bytes = align256(size_t(B * Hkv * hg) * sizeof(int32_t));
  // decode partials: one slot of [HG_max, D + 2] fp32 per (workgroup, unit)
  // pair that can meet: at most (workgroups + units) slots
  // (slots are laid out for head size 128, which D = 64 shares)
  int64_t partial = 0;
  const bool fast_decode = (D == 128 || D == 64) && s.dtype != GQA_FP32;
  if (fast_decode)
    partial = (kDecodeMaxWorkgroups + B * Hkv * hg) * int64_t(kDecodeMaxHG) * (128 + 2) * 4;
  // eviction halos: [B, Hkv, 2, chunks, halo rows, row bytes]
  const int64_t row_bytes = D * (s.dtype == GQA_FP32 ? 4 : 2);
  const EvictGeometry eg = evict_geometry((int)row_bytes);
  const int64_t chunks = (M + eg.chunk_rows - 1) / eg.chunk_rows;
  const int64_t halo = B * Hkv * 2 * chunks * kEvictHaloMax * row_bytes;
  // fused-eviction halo rows (decode): one K and one V row per worker, in the dtype
  int64_t dhalo = 0;
  if (fast_decode) dhalo = 2 * int64_t(kDecodeMaxWorkers) * D * 2;
  // prefill split partials: [row blocks, splits] slots (only when splitting;
  // a one-token shape that the split-KV decode serves never runs the prefill)
  int64_t pf_items = 0, pf_partial = 0;
  const bool decode_only = s.new_tokens == 1;
  if ((D == 128 || D == 64) && s.dtype != GQA_FP32 && s.new_tokens > 0 && !decode_only) {
    if (prefill_may_split(B, s.new_tokens, G, Hkv, M)) {
      pf_items = ((s.new_tokens * G + kPrefillWgRows - 1) / kPrefillWgRows) * B * Hkv;
      // the plan may give one row block up to kPrefillMaxSplits ranges
      pf_partial = pf_items * kPrefillMaxSplits * int64_t(kPrefillSlotFloats) * 4;
    }
  }
  l.scratch = l.counters_bytes;
  l.decode_halo = l.scratch + align256(size_t(partial));
  // the scratch area is reused: an eviction before the prefill kernel has
  // finished with it (stream order), and decode runs in calls of its own
  l.prefill_partials = l.scratch;
  l.scratch_bytes = align256(std::max({size_t(halo), align256(size_t(partial)) + size_t(dhalo),
                                       size_t(pf_partial)}));
  l.prefill_counters = l.scratch + l.scratch_bytes;
  l.prefill_counters_bytes = align256(size_t(pf_items) * sizeof(int32_t));
  l.total = l.prefill_counters + l.prefill_counters_bytes;
  if (staged) {
    l.stage_rows = int(M);
    l.stage_bytes = align256(size_t(B * Hkv * M * row_bytes));
    l.stage_k = l.total;
    l.stage_v = l.stage_k + l.stage_bytes;
    l.total = l.stage_v + l.stage_bytes;
  }
  return l;
}

}  // namespace gqa

using namespace gqa;

extern "C" {

size_t gqa_workspace_bytes(const gqa_shape* shape, const gqa_options* opts) {
  if (!shape) return 0;
  return workspace_layout(*shape, opts ? opts->local_window_size : -1).total;
}

gqa_status gqa_append_kv(const gqa_shape* shape, const gqa_options* opts, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache,
                         const int32_t* seqlens_k_host, const int32_t* seqlens_k_dev,
                         void* stream) {
  g_err[0] = '\0';
  Problem P;
  bool needs_evict;
  int max_drop;
  gqa_status st = validate(kAppend, shape, opts, nullptr, k_new, v_new, k_cache, v_cache,
                           seqlens_k_host, seqlens_k_dev, nullptr, &P, &needs_evict, &max_drop);
  if (st != GQA_OK) return st;
  if (P.B == 0 || P.S == 0) return GQA_OK;
  hipError_t e = launch_append(P, false, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append");
  return GQA_OK;
}

gqa_status gqa_attention_prefill(const gqa_shape* shape, const gqa_options* opts, const void* q,
                                 const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, const int32_t* seqlens_k_host,
                                 const int32_t* seqlens_k_dev, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return run_attention(kPrefill, shape, opts, q, k_new, v_new, k_cache, v_cache, seqlens_k_host,
                       seqlens_k_dev, out, workspace, workspace_bytes, stream);
}

gqa_status gqa_attention_decode(const gqa_shape* shape, const gqa_options* opts, const void* q,
                                const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, const int32_t* seqlens_k_host,
                                const int32_t* seqlens_k_dev, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return run_attention(kDecode, shape, opts, q, k_new, v_new, k_cache, v_cache, seqlens_k_host,
                       seqlens_k_dev, out, workspace, workspace_bytes, stream);
}

gqa_status gqa_attention_present(const gqa_shape* shape, const gqa_options* opts, const void* q,
                                 const void* k_new, const void* v_new, const void* past_key,
                                 const void* past_value, int32_t past_rows, void* present_key,
                                 void* present_value, const int32_t* seqlens_k_host,
                                 const int32_t* seqlens_k_dev, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  // the whole op's own validation (shape, options, present lengths, room,
  // workspace) comes first; nothing is launched before every check passed
  Problem P;
  bool needs_evict;
  int max_drop;
  gqa_status st = validate(kPrefill, shape, opts, q, k_new, v_new, present_key, present_value,
                           seqlens_k_host, seqlens_k_dev, out, &P, &needs_evict, &max_drop);
  if (st != GQA_OK) return st;
  if (past_rows < 0) return fail(GQA_ERR_INVALID_ARG, "past_rows %d < 0", past_rows);
  int max_len = 0;
  for (int b = 0; b < P.B; ++b) {
    if (seqlens_k_host[b] > past_rows)
      return fail(GQA_ERR_INVALID_ARG, "seqlens_k[%d] = %d > past_rows %d", b, seqlens_k_host[b],
                  past_rows);
    max_len = std::max(max_len, seqlens_k_host[b]);
  }
  const bool same = past_key == present_key || past_value == present_value;
  if (same && (past_key != present_key || past_value != present_value || past_rows != P.M))
    return fail(GQA_ERR_INVALID_ARG,
                "past and present share a buffer only as a whole (same K and V, same rows)");
  if (!same && max_len > 0 && (!past_key || !past_value))
    return fail(GQA_ERR_INVALID_ARG, "past_key or past_value is NULL");
  if (!same && ((uintptr_t(past_key) | uintptr_t(past_value)) & (kTensorAlign - 1)))
    return fail(GQA_ERR_INVALID_ARG, "past_key and past_value must be %d-byte aligned", kTensorAlign);
  WorkspaceLayout lay;
  st = check_workspace(shape, P.window, workspace, workspace_bytes, &lay);
  if (st != GQA_OK) return st;
  if (P.B == 0) return GQA_OK;
  if (!same && past_reads_fused(P, needs_evict)) {
    // one new token on the split-KV decode: it reads every past row once
    // anyway, so it writes them into present as it goes (no separate copy)
    return run_attention(kPrefill, shape, opts, q, k_new, v_new, present_key, present_value,
                         seqlens_k_host, seqlens_k_dev, out, workspace, workspace_bytes, stream,
                         false, past_key, past_value, past_rows);
  }
  if (!same) {
    hipError_t e = launch_copy_prefix(past_key, past_value, past_rows, present_key, present_value,
                                      P.M, seqlens_k_dev, P.B, P.Hkv,
                                      P.D * elem_bytes(P.dtype), -1, max_len,
                                      reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "past copy");
  }
  return run_attention(kPrefill, shape, opts, q, k_new, v_new, present_key, present_value,
                       seqlens_k_host, seqlens_k_dev, out, workspace, workspace_bytes, stream);
}

gqa_status gqa_evict_window(const gqa_shape* shape, int32_t incoming, void* k_cache,
                            void* v_cache, const int32_t* seqlens_k_host,
                            const int32_t* seqlens_k_dev, int32_t* seqlens_after_host,
                            void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  gqa_status st = check_shape(shape, false);
  if (st != GQA_OK) return st;
  const int B = shape->batch, M = shape->max_seq_len;
  if (incoming < 0 || incoming > M)
    return fail(GQA_ERR_INVALID_ARG, "incoming %d outside 0..%d", incoming, M);
  st = check_lengths(shape, seqlens_k_host, seqlens_k_dev);
  if (st != GQA_OK) return st;
  if (B > 0 && !seqlens_after_host) return fail(GQA_ERR_INVALID_ARG, "seqlens_after_host is NULL");
  int max_drop = 0;
  for (int b = 0; b < B; ++b)
    max_drop = std::max<int64_t>(max_drop, int64_t(seqlens_k_host[b]) + incoming - M);
  if (max_drop > 0 && (!k_cache || !v_cache)) return fail(GQA_ERR_INVALID_ARG, "cache is NULL");
  if (max_drop > 0 && ((uintptr_t(k_cache) | uintptr_t(v_cache)) & (kTensorAlign - 1)))
    return fail(GQA_ERR_INVALID_ARG, "the caches must be %d-byte aligned", kTensorAlign);
  WorkspaceLayout lay;
  st = check_workspace(shape, -1, workspace, workspace_bytes, &lay);
  if (st != GQA_OK) return st;
  if (max_drop > 0) {
    Problem P{};
    P.B = B; P.S = incoming; P.H = shape->kv_num_heads; P.Hkv = shape->kv_num_heads; P.G = 1;
    P.D = shape->head_size; P.M = M; P.dtype = shape->dtype; P.window = M; P.cap = M;
    P.k_cache = k_cache; P.v_cache = v_cache; P.lens_dev = seqlens_k_dev;
    P.lens_host = seqlens_k_host;
    hipError_t e = launch_evict(P, incoming, max_drop, workspace, lay,
                                reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "eviction");
  }
  for (int b = 0; b < B; ++b) seqlens_after_host[b] = std::min(seqlens_k_host[b], M - incoming);
  return GQA_OK;
}

const char* gqa_status_string(gqa_status s) {
  switch (s) {
    case GQA_OK: return "ok";
    case GQA_ERR_NO_ROOM: return "no room to append: past + new exceeds max_seq_len";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GQA_ERR_WORKSPACE: return "workspace missing or too small";
    case GQA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* gqa_last_error(void) { return g_err; }

gqa_status gqa_attention_decode_noalloc(const gqa_shape* shape, const gqa_options* opts,
                                        const void* q, const void* k_new, const void* v_new,
                                        void* k_cache, void* v_cache,
                                        const int32_t* seqlens_k_host,
                                        const int32_t* seqlens_k_dev, void* out, void* stream) {
  return run_attention(kDecode, shape, opts, q, k_new, v_new, k_cache, v_cache, seqlens_k_host,
                       seqlens_k_dev, out, nullptr, 0, stream, true);
}

}  // extern "C"
