// Flash-style attention for S >= 1 new tokens, fp16/bf16, head_size 128 or 64
// (the template parameter D).
//
// One workgroup (8 waves) takes one (b, kv head) and 256 query rows, where
// the rows of a kv head are its (position i, local head j) pairs flattened as
// r = i * G + j: the G query heads that share the kv head share every K/V
// tile the workgroup holds in LDS, whatever G is. Each wave owns 32 rows.
//
// Per 64-key tile (the gemm0 -> softmax -> gemm1 chain of the "KV Cache"
// discussion's worked example, on gfx950 MFMA 32x32x16):
//   S^T = K Q^T   A = K rows from LDS, B = Q^T held in registers (rotated
//                 on load in fp32 when rotary is on);
//                 lane (row, half) gets 32 keys of its row;
//   online softmax per row, in registers (one cross-lane step);
//   O^T += V^T P^T  A = V^T through transposing LDS reads, B = P^T straight
//                 from the S^T registers.
// The eight waves form two groups that alternate between the matrix
// products and the softmax (see prefill_kernel), so the two waves sharing a
// SIMD keep its matrix core and its vector unit busy at the same time.
// Keys run from the workgroup's window start to its last row's own position:
// the tile loop ends at the sequence's length (the early exit on the key-block
// loop from the discussion's notes), each wave skips the tiles no row of its
// own can see, and the causal/window mask is applied only on tiles that are
// not fully visible to all of the wave's rows. K/V rows past the valid length
// are never read from memory (the tile loads return zeros there), so P and V
// entries of masked keys are exact zeros.
#include <algorithm>
#include <atomic>
#include <vector>

#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// MFMA 32x32x16 for the storage dtype, the packed fp32 -> dtype conversion
// (v_cvt_pk_*_f32, nearest-even) and a two-element sum on the dot unit.
template <class T> struct Mma32;
template <> struct Mma32<F16> {
  __device__ static inline f32x16 run(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    const f16x2 v = {static_cast<_Float16>(x), static_cast<_Float16>(y)};
    return __builtin_bit_cast(uint32_t, v);
  }
  // acc + lo + hi of a packed pair
  __device__ static inline float dot_ones(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                  __builtin_bit_cast(f16x2, 0x3C003C00u), acc, false);
  }
};
template <> struct Mma32<BF16> {
  __device__ static inline f32x16 run(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    const bf16x2 v = {static_cast<__bf16>(x), static_cast<__bf16>(y)};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static inline float dot_ones(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
  }
};

constexpr int kPrefillArgBatch = 64;          // batches whose lengths travel in the arguments
constexpr int kBK = 64;                       // keys per tile
#ifndef GQA_PREFILL_SETPRIO
#define GQA_PREFILL_SETPRIO 2                 // wave priority while issuing matrix products
#endif
#ifndef GQA_PREFILL_PLAN_PCT
#define GQA_PREFILL_PLAN_PCT 100              // split plan: workgroups per 100 CUs
#endif
#ifndef GQA_PREFILL_READ_AHEAD
#define GQA_PREFILL_READ_AHEAD 4              // LDS operand reads issued ahead of their product
#endif
constexpr int kWaves = 8;                     // two groups of four (one wave of each per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kWgRows = 32 * kWaves;          // query rows per workgroup
static_assert(kWgRows == kPrefillWgRows && kThreads == 512, "split slots assume 512 lanes x 256 rows");
constexpr float kLog2e = 1.4426950408889634f;
// A split partial: [512 x 32] words of o / l (two 16-bit values each, lane
// fastest), then the 512 lanes' running maxima and weight sums in fp32.
constexpr int kSlotM = 512 * 32;
constexpr int kSlotL = 512 * 33;
static_assert(kSlotL + 512 == int(kPrefillSlotFloats), "split slot layout");
// The running maximum used in the exponent is refreshed only when a score
// exceeds it by more than this many binary orders, so weights stay <= 2^8:
// exact in fp32, representable in fp16/bf16 with full relative precision.
constexpr float kRescaleSlack = 8.f;

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  uint16_t* out;
  const int32_t* lens;
  const float* cosv;
  const float* sinv;
  int B, S, H, Hkv, G, M, W;
  int cap;            // an evicting sequence keeps min(L, max(0, cap - S)) rows (M, or W when greedy)
  // windowed chunk: keys from each sequence's 64-aligned past length on come
  // from the staging frame (M rows per (b, kv head), row = key), earlier
  // keys from the cache (kv_rows rows per (b, kv head)); without a frame
  // everything comes from the cache and kv_rows = M
  const uint16_t* k_stage;
  const uint16_t* v_stage;
  int kv_rows;
  int rot, rot_rows, interleaved;
  int n_rb;           // row blocks per (b, kv head)
  float scale_log2;   // |scale| * log2(e)
  uint32_t q_sign;    // 0x80008000 when the scale is negative: Q is negated (exact)
  int n_items0;       // n_rb * B * Hkv row blocks
  float* partials;    // splitting: [row block][kPrefillMaxSplits] slots of kPrefillSlotFloats
  int* counters;      // splitting: per row block, finished ranges (kept zero)
  int plan_n;         // > 0: workgroup w takes plan[w] = row block | range << 16 | ranges << 24
  uint32_t plan[kPrefillPlanMax];
  const uint16_t* bias;   // additive bias: (b, h, i, column) at b bias_bs + h bias_hs + i bias_T + column
  int64_t bias_bs, bias_hs;
  int bias_T;             // a multiple of 4 (four columns per 8-byte load)
  float bias_mul;         // log2(e) / scale_log2 = 1 / |scale|: a bias in units of the raw scores
  int hl_ok;          // past lengths below are valid (B <= kPrefillArgBatch)
  int hl[kPrefillArgBatch];   // past lengths from the host (the same values as lens)
  const int32_t* offs;        // absolute position of buffer row 0 (nullptr: 0), device
  int ho[kPrefillArgBatch];   // the same from the host, valid with hl_ok
};

// The cos/sin values one lane needs for its row's D / 16 B-operand chunks;
// chunk ks holds dims 16 ks + 8 c + e. Rotate-half pairs (d, d + D / 2) are
// chunks (ks, ks + D / 32) of the same lane and use entry 8 ks + e (table
// index 16 ks + 8 c + e); interleaved pairs are neighbours inside a chunk
// and use entry 4 ks + e / 2 (table index 8 ks + 4 c + e / 2). Either way a
// lane needs D / 4 entries (D / 16 float4 of each table); all its 16-byte
// loads are issued together, before any of them is used.
struct RotVals {
  float4 c0, c1, c2, c3, c4, c5, c6, c7;
  float4 s0, s1, s2, s3, s4, s5, s6, s7;
};

template <int D>
__device__ __forceinline__ void load_rot(RotVals& r, const float* cosr, const float* sinr, int c,
                                         int interleaved) {
  const float4* cv = reinterpret_cast<const float4*>(cosr);
  const float4* sv = reinterpret_cast<const float4*>(sinr);
  // float4 index of entry 4 m: rotate-half 4 (m / 2) + 2 c + m % 2, interleaved 2 m + c
  const int o0 = interleaved ? c : 2 * c;
  const int st = interleaved ? 2 : 1;
  auto idx = [&](int m) { return interleaved ? o0 + st * m : 4 * (m >> 1) + o0 + (m & 1); };
  r.c0 = cv[idx(0)]; r.c1 = cv[idx(1)]; r.c2 = cv[idx(2)]; r.c3 = cv[idx(3)];
  r.s0 = sv[idx(0)]; r.s1 = sv[idx(1)]; r.s2 = sv[idx(2)]; r.s3 = sv[idx(3)];
  if (D == 128) {
    r.c4 = cv[idx(4)]; r.c5 = cv[idx(5)]; r.c6 = cv[idx(6)]; r.c7 = cv[idx(7)];
    r.s4 = sv[idx(4)]; r.s5 = sv[idx(5)]; r.s6 = sv[idx(6)]; r.s7 = sv[idx(7)];
  } else {
    r.c4 = r.c5 = r.c6 = r.c7 = r.s4 = r.s5 = r.s6 = r.s7 = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__device__ __forceinline__ float rot_entry(const RotVals& r, int i, bool sine) {
  // i is a compile-time constant after unrolling: picks one register
  const float4 v = sine ? (i < 4 ? r.s0 : i < 8 ? r.s1 : i < 12 ? r.s2 : i < 16 ? r.s3 :
                           i < 20 ? r.s4 : i < 24 ? r.s5 : i < 28 ? r.s6 : r.s7)
                        : (i < 4 ? r.c0 : i < 8 ? r.c1 : i < 12 ? r.c2 : i < 16 ? r.c3 :
                           i < 20 ? r.c4 : i < 24 ? r.c5 : i < 28 ? r.c6 : r.c7);
  const int k = i & 3;
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Rotate one row's 8 B-operand chunks in place with the loaded values, in
// fp32: each output is a fused multiply-add on the rounded other product,
// then nearest-even to the dtype. Q only enters the scores, so this
// rounding (at most one fp32 ulp from the exact expression before the
// dtype rounding) shows only in the outputs, which are held to their
// tolerance; K rows written to the cache use the exact rule of
// rotate_pair. The fp64 form here was about a third of each workgroup's
// start (fp64 conversions run at a quarter of the fp32 rate).
template <class T, int D>
__device__ __forceinline__ void apply_rot_q(uint4 (&qv)[D / 16], const RotVals& r, int interleaved) {
  using Bits = typename T::bits;
  auto lo = [](uint32_t w) { return T::to_float(Bits(w & 0xFFFFu)); };
  auto hi = [](uint32_t w) { return T::to_float(Bits(w >> 16)); };
  if (!interleaved) {
    // pairs (chunk ks element e, chunk ks + D / 32 element e): two per word
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t& wx = (&qv[ks].x)[j];
        uint32_t& wy = (&qv[ks + D / 32].x)[j];
        const float c0 = rot_entry(r, 8 * ks + 2 * j, false), s0 = rot_entry(r, 8 * ks + 2 * j, true);
        const float c1 = rot_entry(r, 8 * ks + 2 * j + 1, false);
        const float s1 = rot_entry(r, 8 * ks + 2 * j + 1, true);
        const float x0 = lo(wx), x1 = hi(wx), y0 = lo(wy), y1 = hi(wy);
        const float ys0 = y0 * s0, ys1 = y1 * s1, xs0 = x0 * s0, xs1 = x1 * s1;
        wx = Mma32<T>::pack2(fmaf(x0, c0, -ys0), fmaf(x1, c1, -ys1));
        wy = Mma32<T>::pack2(fmaf(y0, c0, xs0), fmaf(y1, c1, xs1));
      }
  } else {
    // pairs are the two elements of a word
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t& w = (&qv[ks].x)[j];
        const float cc = rot_entry(r, 4 * ks + j, false), ss = rot_entry(r, 4 * ks + j, true);
        const float x = lo(w), y = hi(w);
        const float ys = y * ss, xs = x * ss;
        w = Mma32<T>::pack2(fmaf(x, cc, -ys), fmaf(y, cc, xs));
      }
  }
}

// ---------------------------------------------------------------------------
// Tiles in LDS. K and V tiles are row-major, 64 keys x 2 D bytes, filled
// straight from HBM by buffer_load_dwordx4 ... lds (no register staging): one
// instruction moves 1 KB, lane i writing 16-byte slot i (four 256-byte rows
// at D = 128, eight 128-byte rows at D = 64). The buffer range ends at the
// valid length, so rows past it read as zeros. Within a row the D / 8
// 16-byte chunks are XOR-swizzled per key so that the operand reads below
// are free of bank conflicts (64 banks of 4 bytes: 16 lanes of a b128 read,
// 32 lanes of a b64 read per cycle, 256 bytes either way):
//   D = 128  K: chunk ^ (key & 15)          (b128 reads of 16 consecutive keys)
//            V: chunk ^ 4 (key & 3)         (transposing b64 reads, 4 keys x 2 dim groups)
//   D = 64   K: chunk ^ ((key >> 1) & 7)    (two keys per 256 bytes: 2 x 8 chunks)
//            V: chunk ^ 4 ((key >> 1) & 1)  (4 keys x 4 chunks x 2 halves)
// ---------------------------------------------------------------------------
template <int D> constexpr int tile_bytes() { return kBK * D * 2; }   // 16 KB or 8 KB

template <int D> __device__ inline int swz_k(int key) { return D == 128 ? key & 15 : (key >> 1) & 7; }
template <int D> __device__ inline int swz_v(int key) {
  return D == 128 ? (key & 3) << 2 : ((key >> 1) & 1) << 2;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Per-lane byte offsets of the tile loads, relative to the tile's first key.
// Wave w moves rows 8 w .. 8 w + 7 of a tile. D = 128: rows 8 w + 4 q +
// lane / 16 (q = 0, 1); the K swizzle depends on the row only through
// key & 15 = (8 w + 4 q + lane / 16) & 15 (tiles start at multiples of 64),
// the V swizzle only through lane / 16. D = 64: one instruction, row
// 8 w + lane / 8, chunk lane % 8.
struct LoadOffsets {
  int k[2];
  int v;         // V: one pattern; quad q adds 1024 q
};

template <int D>
__device__ inline LoadOffsets load_offsets(int wave, int lane) {
  LoadOffsets lo;
  if (D == 128) {
    const int lr = lane >> 4, slot = lane & 15;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rrow = 8 * wave + 4 * q + lr;
      lo.k[q] = rrow * 256 + 16 * (slot ^ swz_k<D>(rrow));
    }
    lo.v = (8 * wave + lr) * 256 + 16 * (slot ^ swz_v<D>(lr));
  } else {
    const int rrow = 8 * wave + (lane >> 3), slot = lane & 7;
    lo.k[0] = rrow * 128 + 16 * (slot ^ swz_k<D>(rrow));
    lo.k[1] = lo.k[0];
    lo.v = rrow * 128 + 16 * (slot ^ swz_v<D>(rrow));
  }
  return lo;
}

// Issue this wave's share (8 rows) of one tile: quad q covers rows
// 8 w + 4 q .. + 3. The instruction's immediate offset moves both the
// memory address and the LDS destination, so V (one offset pattern) steps
// through its quads with it from one LDS base; K (a different swizzle per
// quad) uses per-quad lane offsets and LDS bases. Each tile gets its own
// buffer range, starting at its first key and ending at the valid length:
// the range check covers the lane and immediate offsets but not the scalar
// one, so the tile base goes into the descriptor.
template <bool kIsV, int Q>
__device__ inline void quad_load(__amdgpu_buffer_rsrc_t rsrc, unsigned char* tile,
                                 const LoadOffsets& lo, int wave) {
  if (kIsV)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + 8 * wave * 256), 16, lo.v, 0,
                                             1024 * Q, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + (8 * wave + 4 * Q) * 256),
                                             16, lo.k[Q], 0, 0, 0);
}

template <bool kIsV, int D>
__device__ inline void tile_load(const uint16_t* base, int kvalid, unsigned char* tile, int t0,
                                 const LoadOffsets& lo, int wave) {
  t0 = __builtin_amdgcn_readfirstlane(t0);      // the tile start is wave-uniform
  const int rows = max(0, kvalid - t0);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base + int64_t(t0) * D), 0, rows * D * 2, 0x00020000);
  if (D == 128) {
    quad_load<kIsV, 0>(rsrc, tile, lo, wave);
    quad_load<kIsV, 1>(rsrc, tile, lo, wave);
  } else {
    // the wave's eight 128-byte rows in one instruction
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + 8 * wave * 128), 16,
                                             kIsV ? lo.v : lo.k[0], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Online softmax of one 64-key tile of S^T for the lane's row (32 scores
// here, the other 32 in lane ^ 32), then P^T packed as the PV B operand.
// ---------------------------------------------------------------------------
struct RowState {
  float m_run;   // running max of score * cs (-inf before the first visible key)
  float m_use;   // reference max in the exponent (finite)
  float l;       // this lane's share of the sum of the packed weights
};

// The lane's bias values of one tile: columns tb + 4 c + 32 h + 8 j + e in
// member 4 h + j (four halves each), matching the lane's scores.
struct BiasTile {
  uint2 v[8];
};

template <class T, bool kMask, bool kBias, int D>
__device__ inline void softmax_tile(f32x16 (&s)[2], RowState& rs, f32x16 (&o)[D / 32], uint4 (&pk)[4],
                                    float cs, int lim_hi, int span, const BiasTile& bt,
                                    float bias_mul) {
  if (kBias) {
    // the bias joins the raw score scaled by 1 / |scale|, so that the
    // exponent cs * s becomes scale * q.k + bias (in log2 units)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint2 w = bt.v[4 * h + (v >> 2)];
        const uint32_t x = (v & 2) ? w.y : w.x;
        const float bv = T::to_float(typename T::bits((x >> (16 * (v & 1))) & 0xFFFFu));
        s[h][v] = fmaf(bv, bias_mul, s[h][v]);
      }
  }
  if (kMask) {
    // key offset within the lane's keys: 32 h + 8 (v / 4) + v % 4; visible iff
    // 0 <= lim_hi - offset <= span (causal limit and window start together)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = 32 * h + 8 * (v >> 2) + (v & 3);
        s[h][v] = uint32_t(lim_hi - off) <= uint32_t(span) ? s[h][v] : -INFINITY;
      }
  }
  // NaN-propagating maximum: unlike fmaxf it needs no quieting of each
  // operand, so the chain folds into one three-input max per two scores
  // four independent chains, then a tree: short dependency paths
  float mc[4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) mc[c4] = __builtin_elementwise_maximum(s[0][c4], s[1][c4]);
#pragma unroll
  for (int v = 4; v < 16; ++v)
    mc[v & 3] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mc[v & 3], s[0][v]), s[1][v]);
  float tmax = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mc[0], mc[1]),
                                             __builtin_elementwise_maximum(mc[2], mc[3]));
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                     false, false);
    tmax = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const float tm = tmax * cs;
  if (__any(tm > rs.m_run + kRescaleSlack)) {
    const float m_new = fmaxf(rs.m_run, tm);
    const float use_new = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(rs.m_use - use_new);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
    rs.l *= alpha;
    rs.m_run = m_new;
    rs.m_use = use_new;
  }
  const float mu = rs.m_use;
  float lp[4] = {0.f, 0.f, 0.f, 0.f};   // the tile's row sum in four chains
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 8 * (u & 1) + 2 * e;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][v], cs, -mu));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][v + 1], cs, -mu));
      w[e] = Mma32<T>::pack2(p0, p1);
      lp[e] = Mma32<T>::dot_ones(w[e], lp[e]);
    }
    pk[u] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  rs.l += (lp[0] + lp[1]) + (lp[2] + lp[3]);
}

// S^T (64 keys) = K Q^T for the lane's row; A = K rows (key 32 h + col,
// dims 16 kk + 8 c .. + 7), B = Q^T.
template <class T, int D>
__device__ inline void scores_tile(const unsigned char* kt, const uint4 (&qv)[D / 16],
                                   f32x16 (&s)[2], int col, int c) {
  // the two 32-key halves are independent accumulation chains: alternate
  // them so that consecutive products never wait on each other (keys col
  // and 32 + col share their swizzle)
  const unsigned char* k0 = kt + col * (2 * D);
  const unsigned char* k1 = kt + (32 + col) * (2 * D);
  const int sw = swz_k<D>(col);
  s[0] = Mma32<T>::run(*reinterpret_cast<const uint4*>(k0 + 16 * (c ^ sw)), qv[0], f32x16{});
  s[1] = Mma32<T>::run(*reinterpret_cast<const uint4*>(k1 + 16 * (c ^ sw)), qv[0], f32x16{});
#pragma unroll
  for (int kk = 1; kk < D / 16; ++kk) {
    s[0] = Mma32<T>::run(*reinterpret_cast<const uint4*>(k0 + 16 * ((2 * kk + c) ^ sw)), qv[kk], s[0]);
    s[1] = Mma32<T>::run(*reinterpret_cast<const uint4*>(k1 + 16 * ((2 * kk + c) ^ sw)), qv[kk], s[1]);
  }
  // operand reads kPrefetch products ahead
  __builtin_amdgcn_sched_group_barrier(0x100, GQA_PREFILL_READ_AHEAD, 0);
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// O^T += V^T P^T over the tile's 64 keys. The A operand (lane: dim d =
// 32 dt + lane % 32, keys in the P^T order 16 u + 8 (e / 4) + 4 c + e % 4) comes
// from two transposing reads: in each 16-lane group, lane j points at key
// kb + j / 4, dims 4 (j % 4) .. + 3 of the group's 16 dims, and lane 4 a + e
// receives dim 4 a + e of the four keys.
template <class T, int D>
__device__ inline void pv_tile(const unsigned char* vt, const uint4 (&pk)[4], f32x16 (&o)[D / 32],
                               int lane) {
  const int j = lane & 15, c = lane >> 5, g1 = (lane >> 4) & 1;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      uint32_t w[4];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int key = 16 * u + 8 * r + 4 * c + (j >> 2);
        const int ch = 4 * dt + 2 * g1 + ((j & 3) >> 1);
        const unsigned char* ptr = vt + key * (2 * D) + 16 * (ch ^ swz_v<D>(key)) + 8 * (j & 1);
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ptr));
        const uint2 xx = __builtin_bit_cast(uint2, x);
        w[2 * r] = xx.x;
        w[2 * r + 1] = xx.y;
      }
      o[dt] = Mma32<T>::run(make_uint4(w[0], w[1], w[2], w[3]), pk[u], o[dt]);
    }
  }
  // operand reads kPrefetch products ahead of the products that use them
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * GQA_PREFILL_READ_AHEAD, 0);
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// One workgroup = 8 waves x 32 query rows of one (b, kv head): group 0
// (waves 0-3) and group 1 (waves 4-7), one wave of each on every SIMD.
// Every 64-key tile t takes two phases, separated by workgroup barriers:
//   phase 2t:     group 0: O += V(t-1) P(t-1), S(t) = K(t) Q^T   (matrix cores)
//                 group 1: softmax of S(t-1) -> P(t-1)            (vector units)
//   phase 2t + 1: group 0: softmax of S(t) -> P(t)
//                 group 1: O += V(t-1) P(t-1), S(t) = K(t) Q^T
// so the two waves sharing a SIMD always work on different units. K(t+1)
// and V(t) go to the free LDS buffers at the start of phase 2t (the tiles
// they replace were last read in phase 2t - 1) and are waited for at the
// end of phase 2t + 1.
template <class T, int D>
__device__ inline void products(int t, int wt0, int wt1, const unsigned char* kt,
                                const unsigned char* vt, const uint4 (&qv)[D / 16],
                                const uint4 (&pk)[4], f32x16 (&o)[D / 32], f32x16 (&sc)[2], int col,
                                int c, int lane) {
#if GQA_PREFILL_SETPRIO
  __builtin_amdgcn_s_setprio(GQA_PREFILL_SETPRIO);
#endif
  if (t - 1 >= wt0 && t - 1 < wt1) pv_tile<T, D>(vt, pk, o, lane);
  if (t >= wt0 && t < wt1) scores_tile<T, D>(kt, qv, sc, col, c);
#if GQA_PREFILL_SETPRIO
  __builtin_amdgcn_s_setprio(0);
#endif
}

template <class T, bool kBias, int D>
__device__ inline void softmax_step(int t, int wt0, int wt1, f32x16 (&sc)[2], RowState& rs,
                                    f32x16 (&o)[D / 32], uint4 (&pk)[4], float cs, int my_p, int span,
                                    int w_full_lo, int w_full_hi, int c, const BiasTile& bt,
                                    float bias_mul) {
  if (t < wt0 || t >= wt1) return;
  const int tb = t * kBK;
  const bool full = tb + kBK - 1 <= w_full_hi && tb >= w_full_lo;
  const int lim_hi = my_p - (tb + 4 * c);
  if (full)
    softmax_tile<T, false, kBias, D>(sc, rs, o, pk, cs, lim_hi, span, bt, bias_mul);
  else
    softmax_tile<T, true, kBias, D>(sc, rs, o, pk, cs, lim_hi, span, bt, bias_mul);
}

// The bias values of tile t for the lane's row. Columns are clamped to the
// last aligned group below bias_T: past the causal limit the scores are
// masked whatever the value, and below it every column is < L + S <= T.
__device__ inline void bias_load(BiasTile& bt, const uint16_t* brow, int t, int c, int T) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int col = t * kBK + 4 * c + 32 * h + 8 * j;
      col = col <= T - 4 ? col : T - 4;
      bt.v[4 * h + j] = *reinterpret_cast<const uint2*>(brow + col);
    }
}

template <class T, bool kBias, int D>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(PrefillArgs a) {
  constexpr int kTileBytes = tile_bytes<D>();
  constexpr int kRowBytes = 2 * D;
  // four separately declared tiles, each used at fixed places of the
  // two-iteration loop body: the compiler can then tell the tiles being read
  // from the tiles being filled by direct-to-LDS loads and does not wait for
  // those loads before every read
  __shared__ __attribute__((aligned(1024))) unsigned char k_even[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_odd[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_even[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_odd[kTileBytes];
  __shared__ int sh_last;                       // split merge: this workgroup finished last

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
#ifndef GQA_PREFILL_GROUP_ODD
  const int grp = wave >> 2;
#else
  const int grp = wave & 1;
#endif
  const int col = lane & 31, c = lane >> 5;     // S^T column (= the lane's row), k half
  const int units = a.B * a.Hkv;
  // workgroup -> (row block, key range, ranges of that row block): from the
  // host's plan (sized to the lengths) when splitting, else one row block
  // each, longest first
  int item = int(blockIdx.x), split = 0, nsplit = 1;
  if (a.plan_n > 0) {
    const uint32_t e = a.plan[blockIdx.x];
    item = int(e & 0xFFFFu);
    split = int((e >> 16) & 0xFFu);
    nsplit = int(e >> 24);
  }
  const int bg = item % units;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.G, S = a.S;

  // one row block: the whole tile loop for 256 query rows
  auto row_block = [&](const int rb) {
  const int nrows = S * G;
  // past lengths come from the arguments when the host could pass them
  // (no dependent load before the first tile and the rotary tables); a
  // device read is marked wave-uniform
  int len_raw;
  if (a.hl_ok) {
    len_raw = a.hl[b];                 // a scalar read of the argument block
    asm volatile("" : "+s"(len_raw));  // keeps it apart from the device read below
  } else {
    len_raw = __builtin_amdgcn_readfirstlane(a.lens[b]);
  }
  // rows kept before the new ones (the append already ran, after any
  // eviction): the same rule as the eviction kernels
  const int L = clamp_len(kept_rows(clamp_len(len_raw, 0, a.M), S, a.M, a.cap), 0, a.M - S);
  const int kvalid = L + S;

  const int r0 = rb * kWgRows;
  const int wr0 = r0 + 32 * wave;
  const bool wave_has_rows = wr0 < nrows;
  const int r = wr0 + col;
  const bool row_ok = r < nrows;
  const int my_i = row_ok ? r / G : S - 1;
  const int my_h = g * G + (row_ok ? r % G : 0);
  const int my_p = L + my_i;                                // causal limit
  const int my_ws = a.W > 0 ? max(0, my_p - a.W + 1) : 0;   // window start

  // workgroup and wave key ranges (tiles)
  const int wg_ilo = r0 / G, wg_ihi = min(S - 1, (r0 + kWgRows - 1) / G);
  const int w_ilo = min(S - 1, wr0 / G), w_ihi = min(S - 1, (wr0 + 31) / G);
  const int wg_kstart = a.W > 0 ? max(0, L + wg_ilo - a.W + 1) : 0;
  const int wg_kend = L + wg_ihi + 1;
  const int w_kstart = a.W > 0 ? max(0, L + w_ilo - a.W + 1) : 0;
  const int w_kend = L + w_ihi + 1;
  const int w_full_lo = a.W > 0 ? L + w_ihi - a.W + 1 : 0;  // keys >= this: no window cut
  const int w_full_hi = L + w_ilo;                          // keys <= this: no causal cut
  // this split's share of the row block's tiles (all of them without a split)
  const int rb_t0 = wg_kstart / kBK, rb_t1 = (wg_kend + kBK - 1) / kBK;
  const int t_begin = __builtin_amdgcn_readfirstlane(rb_t0 + (rb_t1 - rb_t0) * split / nsplit);
  const int t_end = __builtin_amdgcn_readfirstlane(rb_t0 + (rb_t1 - rb_t0) * (split + 1) / nsplit);
  const int wt0 = wave_has_rows ? max(w_kstart / kBK, t_begin) : t_end;
  const int wt1 = wave_has_rows ? min((w_kend + kBK - 1) / kBK, t_end) : t_end;

  const int64_t kvbase = (int64_t(b) * a.Hkv + g) * a.kv_rows * D;
  const uint16_t* kc = a.k_cache + kvbase;
  const uint16_t* vc = a.v_cache + kvbase;
  // tiles at or past `stage_from` come from the staging frame (same key rows)
  const int stage_from = a.k_stage ? (L & ~(kBK - 1)) : INT_MAX;
  const int64_t sbase = (int64_t(b) * a.Hkv + g) * a.M * D;
  const uint16_t* k_frame = a.k_stage ? a.k_stage + sbase : kc;
  const uint16_t* v_frame = a.k_stage ? a.v_stage + sbase : vc;

  const LoadOffsets lo = load_offsets<D>(wave, lane);
  tile_load<false, D>(t_begin * kBK < stage_from ? kc : k_frame, kvalid, k_even, t_begin * kBK, lo,
                      wave);

  // ---- Q^T (B operand): lane holds Q[row][16 ks + 8 c + e] ----
  uint4 qv[D / 16];
  {
    const uint16_t* qrow = a.q + ((int64_t(b) * S + my_i) * a.H + my_h) * D + 8 * c;
    // lanes past the last row read a valid row (my_i = S - 1): rows never
    // mix, and those lanes store nothing, so no load waits on a branch
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qv[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks);
    if (a.rot) {
      int off = 0;
      if (a.hl_ok) {
        off = a.ho[b];
        asm volatile("" : "+s"(off));
      } else if (a.offs) {
        off = __builtin_amdgcn_readfirstlane(a.offs[b]);
      }
      const int pos = clamp_len(len_raw + off + my_i, 0, a.rot_rows - 1);
      RotVals rv;
      load_rot<D>(rv, a.cosv + int64_t(pos) * (D / 2), a.sinv + int64_t(pos) * (D / 2), c,
                  a.interleaved);
      apply_rot_q<T, D>(qv, rv, a.interleaved);
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qv[ks].x ^= a.q_sign; qv[ks].y ^= a.q_sign; qv[ks].z ^= a.q_sign; qv[ks].w ^= a.q_sign;
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  RowState rs{-INFINITY, 0.f, 0.f};
  const float cs = a.scale_log2;
  const int span = my_p - my_ws;
  f32x16 sc[2];
  uint4 pk[4];

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Tile t (j = t - t_begin) uses K buffer j % 2 and V(t - 1) in buffer
  // (j + 1) % 2, and fills K(t + 1) into buffer (j + 1) % 2 and V(t) into
  // buffer j % 2. The two groups run separate loops with the same barriers
  // (s_barrier counts arrivals, not program locations).
  // Phase barriers order execution only: every LDS read of a tile is
  // consumed by a product before its wave reaches the barrier, so a bare
  // s_barrier (no memory fence, which would wait for the direct-to-LDS loads
  // still in flight) suffices in the middle of a tile. At the end of a tile
  // each wave first waits for its own loads, so the next tiles are complete
  // in LDS once everyone has passed.
  auto phase_barrier = []() { __builtin_amdgcn_s_barrier(); };
  auto tiles_landed_barrier = []() {
    // vmcnt(0), expcnt and lgkmcnt left alone; as a builtin the compiler
    // sees that the direct-to-LDS loads have completed
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_s_barrier();
  };
  auto loads = [&](int t, unsigned char* kn, unsigned char* vn) {
    if (t + 1 < t_end)
      tile_load<false, D>((t + 1) * kBK < stage_from ? kc : k_frame, kvalid, kn, (t + 1) * kBK, lo,
                          wave);
    if (t < t_end)
      tile_load<true, D>(t * kBK < stage_from ? vc : v_frame, kvalid, vn, t * kBK, lo, wave);
  };
  // bias of tile t for this lane's row: group 0 issues it before the step's
  // tile loads and uses it after the products (its wait then does not take
  // in the tile loads issued later); group 1 issues it before its products
  // and uses it in the next step, after that step's full wait
  BiasTile bt;
  const uint16_t* brow = nullptr;
  if (kBias) brow = a.bias + b * a.bias_bs + int64_t(my_h) * a.bias_hs + int64_t(my_i) * a.bias_T;
  auto bias_tile = [&](int t) {
    if (kBias && t >= wt0 && t < wt1) bias_load(bt, brow, t, c, a.bias_T);
  };
  auto step0 = [&](int t, const unsigned char* kt, const unsigned char* vt, unsigned char* kn,
                   unsigned char* vn) {
    bias_tile(t);
    loads(t, kn, vn);
    products<T, D>(t, wt0, wt1, kt, vt, qv, pk, o, sc, col, c, lane);
    phase_barrier();
    softmax_step<T, kBias, D>(t, wt0, wt1, sc, rs, o, pk, cs, my_p, span, w_full_lo, w_full_hi, c,
                              bt, a.bias_mul);
    tiles_landed_barrier();
  };
  auto step1 = [&](int t, const unsigned char* kt, const unsigned char* vt, unsigned char* kn,
                   unsigned char* vn) {
    loads(t, kn, vn);
    softmax_step<T, kBias, D>(t - 1, wt0, wt1, sc, rs, o, pk, cs, my_p, span, w_full_lo, w_full_hi,
                              c, bt, a.bias_mul);
    phase_barrier();
    bias_tile(t);
    products<T, D>(t, wt0, wt1, kt, vt, qv, pk, o, sc, col, c, lane);
    tiles_landed_barrier();
  };
  if (grp == 0) {
    for (int t = t_begin; t <= t_end; t += 2) {
      step0(t, k_even, v_odd, k_odd, v_even);
      if (t + 1 <= t_end) step0(t + 1, k_odd, v_even, k_even, v_odd);
    }
  } else {
    for (int t = t_begin; t <= t_end; t += 2) {
      step1(t, k_even, v_odd, k_odd, v_even);
      if (t + 1 <= t_end) step1(t + 1, k_odd, v_even, k_even, v_odd);
    }
  }

  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs.l), __float_as_uint(rs.l),
                                                    false, false);
  float l_row = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);   // the row's weight sum
  if (nsplit > 1) {
    // publish this split's partial, count it in; the last split to finish
    // merges all of them in split order (the same sum whoever is last). The
    // partial output goes out normalised (o / l, a convex combination of V
    // rows, so within the dtype's range) and rounded to the dtype, two
    // values per word: half the bytes of the fp32 accumulators, which all
    // splits write and the last one reads at the same moment at the end of
    // the launch. The merging split rounds its own values the same way.
    float* slots = a.partials + int64_t(item) * kPrefillMaxSplits * int64_t(kPrefillSlotFloats);
    float* mine = slots + int64_t(split) * kPrefillSlotFloats;
    const float inv_l = l_row > 0.f ? 1.f / l_row : 0.f;
    auto packed = [&](int dt, int v2) {
      return Mma32<T>::pack2(o[dt][2 * v2] * inv_l, o[dt][2 * v2 + 1] * inv_l);
    };
    uint32_t* mine_o = reinterpret_cast<uint32_t*>(mine);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v2 = 0; v2 < 8; ++v2)
        __hip_atomic_store(mine_o + (wave * 32 + dt * 8 + v2) * 64 + lane, packed(dt, v2),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mine + kSlotM + tid, rs.m_use, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mine + kSlotL + tid, l_row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // release/acquire handoff: the workgroup barrier orders every thread's
    // partial stores before the count; the counting thread's increment
    // releases them at agent scope (each increment continues the release
    // sequence of the earlier ones), and the thread whose increment
    // completes the count acquires at agent scope before the barrier that
    // carries it to the whole workgroup. Only that workgroup pays for the
    // acquire (an L2 invalidate, which would also drop K/V lines the other
    // workgroups on its XCD still read).
    __syncthreads();
    if (tid == 0) {
      const int prev = __hip_atomic_fetch_add(a.counters + item, 1, __ATOMIC_RELEASE,
                                              __HIP_MEMORY_SCOPE_AGENT);
      sh_last = prev == nsplit - 1;
      if (sh_last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(a.counters + item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (!sh_last) return;
    // the other splits' partials from memory, this split's own from its
    // registers (the values it stored), all weighed in split order
    float mj[kPrefillMaxSplits], lj[kPrefillMaxSplits];
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPrefillMaxSplits; ++j) {
      mj[j] = -INFINITY;
      lj[j] = 0.f;
      if (j < nsplit) {
        const float* sj = slots + int64_t(j) * kPrefillSlotFloats;
        mj[j] = j == split ? rs.m_use
                           : __hip_atomic_load(sj + kSlotM + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lj[j] = j == split ? l_row
                           : __hip_atomic_load(sj + kSlotL + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lj[j] > 0.f) M = fmaxf(M, mj[j]);   // a split that saw no key of the row adds nothing
      }
    }
    float l_acc = 0.f;
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;
    using Bits = typename T::bits;
#pragma unroll
    for (int j = 0; j < kPrefillMaxSplits; ++j) {
      if (j >= nsplit) break;
      const float wj = lj[j] > 0.f ? __builtin_amdgcn_exp2f(mj[j] - M) : 0.f;
      l_acc = fmaf(lj[j], wj, l_acc);
      const float cj = lj[j] * wj;          // weight of the normalised partial
      const uint32_t* sj = reinterpret_cast<const uint32_t*>(slots + int64_t(j) * kPrefillSlotFloats);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v2 = 0; v2 < 8; ++v2) {
          const uint32_t w = j == split ? packed(dt, v2)
                                        : __hip_atomic_load(sj + (wave * 32 + dt * 8 + v2) * 64 + lane,
                                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          acc[dt][2 * v2] = fmaf(T::to_float(Bits(w & 0xFFFFu)), cj, acc[dt][2 * v2]);
          acc[dt][2 * v2 + 1] = fmaf(T::to_float(Bits(w >> 16)), cj, acc[dt][2 * v2 + 1]);
        }
    }
    l_row = l_acc;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = acc[dt];
  }
  // ---- the output. A lane holds dims 32 dt + 8 v4 + 4 c .. + 3 of its row,
  // so storing from registers writes 16-byte pieces of 32 rows per
  // instruction; instead the wave's 32 rows go through its own 64 D bytes
  // of LDS (the tiles are free: every wave has passed the last tile's
  // barrier) and each store instruction writes 1 KB of whole rows. Chunks
  // are XOR-swizzled by row like the K tile. ----
  const float inv = row_ok ? 1.f / l_row : 0.f;
  unsigned char* stage = (wave < 2 ? k_even : wave < 4 ? k_odd : wave < 6 ? v_even : v_odd) +
                         (wave & 1) * (kTileBytes / 2);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      uint2 w;
      w.x = Mma32<T>::pack2(o[dt][4 * v4] * inv, o[dt][4 * v4 + 1] * inv);
      w.y = Mma32<T>::pack2(o[dt][4 * v4 + 2] * inv, o[dt][4 * v4 + 3] * inv);
      *reinterpret_cast<uint2*>(stage + col * kRowBytes + (((4 * dt + v4) ^ swz_k<D>(col)) << 4) +
                                8 * c) = w;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // lane: row kRowsPer k + lane / kChunks of the wave, chunk lane % kChunks
  constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  constexpr int kRowsPer = 64 / kChunks;         // rows per store instruction
  const int ch = lane % kChunks;
  int out_i = (wr0 + lane / kChunks) / G;
  int out_j = wr0 + lane / kChunks - out_i * G;
#pragma unroll
  for (int k = 0; k < 32 / kRowsPer; ++k) {
    const int rr = kRowsPer * k + lane / kChunks;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + rr * kRowBytes + ((ch ^ swz_k<D>(rr)) << 4));
    if (wr0 + rr < nrows)
      *reinterpret_cast<uint4*>(a.out + ((int64_t(b) * S + out_i) * a.H + g * G + out_j) * D + 8 * ch) = v;
    out_j += kRowsPer;
    while (out_j >= G) {
      out_j -= G;
      ++out_i;
    }
  }
  };

  row_block(a.n_rb - 1 - item / units);      // longest row blocks first
}

}  // namespace

bool prefill_fast_supported(const Problem& p) {
  // buffer ranges are 32-bit byte counts; cos/sin rows are read as float4
  const bool rot_aligned = !p.rot || ((reinterpret_cast<uintptr_t>(p.cos) |
                                       reinterpret_cast<uintptr_t>(p.sin)) & 15) == 0;
  // a bias is read four columns per 8-byte load
  const bool bias_ok = !p.bias || (p.bias_T % 4 == 0 && (reinterpret_cast<uintptr_t>(p.bias) & 7) == 0);
  return (p.D == 128 || p.D == 64) && (p.dtype == GQA_FP16 || p.dtype == GQA_BF16) &&
         p.M <= (1 << 23) &&
         rot_aligned && bias_ok;
}

namespace {
template <int D>
void launch_prefill_kernel(const Problem& p, const PrefillArgs& a, int blocks, hipStream_t st) {
  const bool fp16 = p.dtype == GQA_FP16;
  if (p.bias && fp16)
    hipLaunchKernelGGL((prefill_kernel<F16, true, D>), dim3(blocks), dim3(kThreads), 0, st, a);
  else if (p.bias)
    hipLaunchKernelGGL((prefill_kernel<BF16, true, D>), dim3(blocks), dim3(kThreads), 0, st, a);
  else if (fp16)
    hipLaunchKernelGGL((prefill_kernel<F16, false, D>), dim3(blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<BF16, false, D>), dim3(blocks), dim3(kThreads), 0, st, a);
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = kPrefillTargetWorkgroups;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}
}  // namespace

hipError_t launch_prefill_fast(const Problem& p, void* ws, const WorkspaceLayout& lay,
                               hipStream_t st) {
  PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k_cache = static_cast<const uint16_t*>(p.k_cache);
  a.v_cache = static_cast<const uint16_t*>(p.v_cache);
  a.out = static_cast<uint16_t*>(p.out);
  a.lens = p.lens_dev;
  a.cosv = p.cos; a.sinv = p.sin;
  a.B = p.B; a.S = p.S; a.H = p.H; a.Hkv = p.Hkv; a.G = p.G; a.M = p.M; a.W = p.window;
  a.cap = p.cap;
  a.k_stage = static_cast<const uint16_t*>(p.stage_k);
  a.v_stage = static_cast<const uint16_t*>(p.stage_v);
  a.kv_rows = p.stage_k ? p.cache_rows : p.M;
  a.rot = p.rot; a.rot_rows = p.rot_rows; a.interleaved = p.interleaved;
  a.n_rb = ceil_div(p.S * p.G, kWgRows);
  a.scale_log2 = fabsf(p.scale) * kLog2e;
  a.q_sign = p.scale < 0.f ? 0x80008000u : 0u;
  a.bias = static_cast<const uint16_t*>(p.bias);
  a.bias_bs = p.bias_bs; a.bias_hs = p.bias_hs; a.bias_T = p.bias_T;
  a.bias_mul = kLog2e / a.scale_log2;
  a.hl_ok = p.lens_host != nullptr && p.B <= kPrefillArgBatch;
  a.offs = p.off_dev;
  if (a.hl_ok)
    for (int b = 0; b < p.B; ++b) {
      a.hl[b] = p.lens_host[b];
      a.ho[b] = p.off_host ? p.off_host[b] : 0;
    }
  a.n_items0 = a.n_rb * p.B * p.Hkv;
  if (a.n_items0 == 0) return hipSuccess;
  int blocks = a.n_items0;
  if (prefill_may_split(p.B, p.S, p.G, p.Hkv, p.M) && p.lens_host != nullptr) {
    a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.prefill_partials);
    a.counters = reinterpret_cast<int*>(static_cast<char*>(ws) + lay.prefill_counters);
    // Key ranges sized to the lengths: the fewest ranges per row block (at
    // most kPrefillMaxSplits) that keep every range within T tiles, for the
    // smallest T whose total fits one workgroup per CU; longest ranges first.
    const int budget = std::min(kPrefillPlanMax,
                                std::max(device_cu_count() * GQA_PREFILL_PLAN_PCT / 100, a.n_items0));
    std::vector<int> tiles(a.n_items0);
    const int units = p.B * p.Hkv;
    int tmax = 1;
    for (int k = 0; k < a.n_items0; ++k) {
      const int rb = a.n_rb - 1 - k / units, b = (k % units) / p.Hkv;
      const int L = std::max(0, std::min(kept_rows_host(p.lens_host[b], p.S, p.M, p.cap), p.M - p.S));
      const int r0 = rb * kWgRows;
      const int ilo = r0 / p.G, ihi = std::min(p.S - 1, (r0 + kWgRows - 1) / p.G);
      const int kstart = p.window > 0 ? std::max(0, L + ilo - p.window + 1) : 0;
      const int kend = L + ihi + 1;
      tiles[k] = std::max(1, (kend + kBK - 1) / kBK - kstart / kBK);
      tmax = std::max(tmax, tiles[k]);
    }
    auto ranges = [&](int k, int T) { return std::min(kPrefillMaxSplits, (tiles[k] + T - 1) / T); };
    auto total = [&](int T) {
      int n = 0;
      for (int k = 0; k < a.n_items0; ++k) n += ranges(k, T);
      return n;
    };
    int lo = 1, hi = tmax;                 // total(hi) == n_items0 <= budget
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (total(mid) <= budget) hi = mid; else lo = mid + 1;
    }
    std::vector<int> order(a.n_items0);
    for (int k = 0; k < a.n_items0; ++k) order[k] = k;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
      return int64_t(tiles[x]) * ranges(y, lo) > int64_t(tiles[y]) * ranges(x, lo);
    });
    a.plan_n = 0;
    for (int k : order) {
      const int n = ranges(k, lo);
      for (int j = 0; j < n; ++j)
        a.plan[a.plan_n++] = uint32_t(k) | (uint32_t(j) << 16) | (uint32_t(n) << 24);
    }
    blocks = a.plan_n;
  }
  if (p.D == 128) launch_prefill_kernel<128>(p, a, blocks, st);
  else launch_prefill_kernel<64>(p, a, blocks, st);
  return hipGetLastError();
}

}  // namespace gqa
