// Flash-style attention for S >= 1 new tokens, fp16/bf16, head_size 128.
//
// One workgroup (4 waves) takes one (b, kv head) and 128 query rows, where
// the rows of a kv head are its (position i, local head j) pairs flattened as
// r = i * G + j: the G query heads that share the kv head share every K/V
// tile the workgroup stages in LDS, whatever G is. Each wave owns 32 rows.
//
// Per 64-key tile (the gemm0 -> softmax -> gemm1 chain of the "KV Cache"
// discussion's worked example, on gfx950 MFMA 32x32x16):
//   S^T = K Q^T   A = K rows from LDS, B = Q^T held in registers (rotated
//                 on load under the fp64 rule when rotary is on);
//                 lane (row, half) gets 16 keys of its row;
//   online softmax per row, in registers (one cross-lane step);
//   O^T += V^T P^T  A = V^T from LDS (staged transposed, keys permuted so one
//                 16-byte read gives the 8 keys the lane's P slice holds),
//                 B = P^T straight from the S^T registers.
// Keys run from the workgroup's window start to its last row's own position:
// the tile loop ends at the sequence's length (the early exit on the key-block
// loop from the discussion's notes), each wave skips the tiles no row of its
// own can see, and the causal/window mask is applied only on tiles that are
// not fully visible to all of the wave's rows. K/V rows past the valid length
// are never read from memory (zeros are staged instead), so P and V entries of
// masked keys are exact zeros.
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

constexpr int kD = 128;
constexpr int kBK = 64;                       // keys per tile
constexpr int kThreads = 256;
constexpr int kKStride = kD + 8;              // K tile row stride in halves (272 B)
constexpr int kKTile = kBK * kKStride;        // halves
constexpr int kVTile = kD * kBK;              // V^T tile, 128 B rows, swizzled
constexpr float kLog2e = 1.4426950408889634f;
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
  int rot, rot_rows, interleaved;
  int n_rb;           // row blocks per (b, kv head)
  float scale_log2;   // |scale| * log2(e)
  uint32_t q_sign;    // 0x80008000 when the scale is negative: Q is negated (exact)
};

// Rotate one row's 8 B-operand chunks in place. Chunk ks holds dims
// 16 ks + 8 c + e: rotate-half pairs (d, d + 64) are chunks (ks, ks + 4) of the
// same lane, interleaved pairs are neighbours inside a chunk.
template <class T>
__device__ inline void rotate_q(uint4 (&qv)[8], int c, const float* cosr, const float* sinr,
                                int interleaved) {
  using Bits = typename T::bits;
  auto get = [&](int ks, int e) -> Bits {
    const uint32_t w = (&qv[ks].x)[e >> 1];
    return Bits((w >> (16 * (e & 1))) & 0xFFFFu);
  };
  auto put = [&](int ks, int e, Bits v) {
    uint32_t& w = (&qv[ks].x)[e >> 1];
    const int sh = 16 * (e & 1);
    w = (w & ~(0xFFFFu << sh)) | (uint32_t(v) << sh);
  };
  if (!interleaved) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * ks + 8 * c + e;
        Bits x = get(ks, e), y = get(ks + 4, e);
        rotate_pair<T>(x, y, cosr[j], sinr[j]);
        put(ks, e, x);
        put(ks + 4, e, y);
      }
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int j = (16 * ks + 8 * c + e) >> 1;
        Bits x = get(ks, e), y = get(ks, e + 1);
        rotate_pair<T>(x, y, cosr[j], sinr[j]);
        put(ks, e, x);
        put(ks, e + 1, y);
      }
  }
}

// ---------------------------------------------------------------------------
// Staging of one 64-key tile. Thread (wave w, lane) moves keys 16 w + 4 qd + j
// (j = 0..3), dims 8 dg .. 8 dg + 7, of K and V, with dg and qd drawn from the
// lane bits so that each 16-lane group of a store covers 8 dim groups x 2 key
// quads: the V^T stores below are then free of bank conflicts. Rows at or past
// the valid length are not read; zeros are staged.
//
// V^T layout: row d holds the tile's 64 keys in MFMA k order (within every 16
// keys, key 8a + 4c + r sits at 8c + 4a + r, matching the P^T operand the
// score layout hands over), as eight 16-byte chunks whose order is XOR-swizzled
// by vt_swz(d) so that the lanes of a read (consecutive d) and of a store
// (d = 8 dg + e) hit distinct banks.
// ---------------------------------------------------------------------------
struct Stage {
  uint4 k[4];
  uint4 v[4];
};

__device__ inline int stage_dg(int tid) { return (tid & 7) | (((tid >> 4) & 1) << 3); }
__device__ inline int stage_kq(int tid) {
  return 4 * (tid >> 6) + ((((tid >> 3) & 1) << 1) | ((tid >> 5) & 1));
}
__device__ inline int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

__device__ inline void stage_load(Stage& st, const uint16_t* kc, const uint16_t* vc, int tb,
                                  int kvalid, int tid) {
  const int kq = stage_kq(tid), dg = stage_dg(tid);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = tb + 4 * kq + j;
    if (row < kvalid) {
      st.k[j] = *reinterpret_cast<const uint4*>(kc + int64_t(row) * kD + 8 * dg);
      st.v[j] = *reinterpret_cast<const uint4*>(vc + int64_t(row) * kD + 8 * dg);
    } else {
      st.k[j] = make_uint4(0, 0, 0, 0);
      st.v[j] = make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ inline void stage_store(const Stage& st, uint16_t* ks, uint16_t* vs, int tid) {
  const int kq = stage_kq(tid), dg = stage_dg(tid);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint4*>(ks + (4 * kq + j) * kKStride + 8 * dg) = st.k[j];
  const int u = kq >> 2, qd = kq & 3;                       // qd = 2a + c
  const int perm = ((qd & 1) << 1) | (qd >> 1);             // 2c + a
  const int chunk = 2 * u + (perm >> 1), sub = perm & 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1, sh = 16 * (e & 1);
    const uint32_t x0 = ((&st.v[0].x)[w] >> sh) & 0xFFFFu;
    const uint32_t x1 = ((&st.v[1].x)[w] >> sh) & 0xFFFFu;
    const uint32_t x2 = ((&st.v[2].x)[w] >> sh) & 0xFFFFu;
    const uint32_t x3 = ((&st.v[3].x)[w] >> sh) & 0xFFFFu;
    uint2 pk;
    pk.x = x0 | (x1 << 16);
    pk.y = x2 | (x3 << 16);
    const int d = 8 * dg + e;
    *reinterpret_cast<uint2*>(vs + d * kBK + 8 * (chunk ^ vt_swz(d)) + 4 * sub) = pk;
  }
}

// ---------------------------------------------------------------------------
// Online softmax of one 32-key half of S^T for the lane's row (16 scores here,
// the other 16 in lane ^ 32), then P^T packed as the PV B operand.
// ---------------------------------------------------------------------------
struct RowState {
  float m_run;   // running max of score * cs (-inf before the first visible key)
  float m_use;   // reference max in the exponent (finite)
  float l;       // this lane's share of the sum of the packed weights
};

template <class T, bool kMask>
__device__ inline void softmax_half(f32x16& s, RowState& rs, f32x16 (&o)[4], uint4 (&pk)[2],
                                    float cs, int lim_hi, int span) {
  if (kMask) {
    // key offset within the lane's keys: 8 (v / 4) + v % 4; visible iff
    // 0 <= lim_hi - offset <= span (causal limit and window start together)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int off = 8 * (v >> 2) + (v & 3);
      s[v] = uint32_t(lim_hi - off) <= uint32_t(span) ? s[v] : -INFINITY;
    }
  }
  float tmax = s[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, s[v]);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                     false, false);
    tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  const float tm = tmax * cs;
  if (__any(tm > rs.m_run + kRescaleSlack)) {
    const float m_new = fmaxf(rs.m_run, tm);
    const float use_new = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(rs.m_use - use_new);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
    rs.l *= alpha;
    rs.m_run = m_new;
    rs.m_use = use_new;
  }
  const float mu = rs.m_use;
  uint32_t w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * e], cs, -mu));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * e + 1], cs, -mu));
    w[e] = Mma32<T>::pack2(p0, p1);
    rs.l = Mma32<T>::dot_ones(w[e], rs.l);
  }
  pk[0] = make_uint4(w[0], w[1], w[2], w[3]);
  pk[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// S^T (32 keys of half h) = K Q^T for the lane's row
template <class T>
__device__ inline f32x16 scores_half(const uint16_t* ks, const uint4 (&qv)[8], int h, int col,
                                     int c) {
  const uint16_t* krow = ks + (32 * h + col) * kKStride + 8 * c;
  f32x16 sc = Mma32<T>::run(*reinterpret_cast<const uint4*>(krow), qv[0], f32x16{});
#pragma unroll
  for (int kk = 1; kk < 8; ++kk)
    sc = Mma32<T>::run(*reinterpret_cast<const uint4*>(krow + 16 * kk), qv[kk], sc);
  return sc;
}

// O^T += V^T P^T over the 32 keys of half h
template <class T>
__device__ inline void pv_half(const uint16_t* vs, const uint4 (&pk)[2], f32x16 (&o)[4], int h,
                               int col, int c) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d = 32 * dt + col;
    const uint16_t* vrow = vs + d * kBK;
    const int sw = vt_swz(d);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 va = *reinterpret_cast<const uint4*>(vrow + 8 * ((4 * h + 2 * u + c) ^ sw));
      o[dt] = Mma32<T>::run(va, pk[u], o[dt]);
    }
  }
}

// One 64-key tile for the lane's row: both score halves are issued before the
// first softmax so the second runs on the matrix cores meanwhile.
template <class T, bool kMask>
__device__ inline void tile_step(const uint16_t* ks, const uint16_t* vs, const uint4 (&qv)[8],
                                 f32x16 (&o)[4], RowState& rs, float cs, int lim_hi, int span,
                                 int col, int c) {
  f32x16 s0 = scores_half<T>(ks, qv, 0, col, c);
  f32x16 s1 = scores_half<T>(ks, qv, 1, col, c);
  uint4 pk[2];
  softmax_half<T, kMask>(s0, rs, o, pk, cs, lim_hi, span);
  pv_half<T>(vs, pk, o, 0, col, c);
  softmax_half<T, kMask>(s1, rs, o, pk, cs, lim_hi - 32, span);
  pv_half<T>(vs, pk, o, 1, col, c);
}

// One workgroup = 4 waves x 32 query rows of one (b, kv head).
template <class T>
__global__ void __launch_bounds__(kThreads, 2) prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKTile];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kVTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, c = lane >> 5;     // S^T column (= the lane's row), k half
  const int units = a.B * a.Hkv;
  const int rb = a.n_rb - 1 - int(blockIdx.x) / units;    // longest row blocks first
  const int bg = int(blockIdx.x) % units;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.G, S = a.S;
  const int nrows = S * G;
  const int L = clamp_len(a.lens[b], 0, a.M - S);
  const int kvalid = L + S;

  const int r0 = rb * 128;
  const int wr0 = r0 + 32 * wave;
  const bool wave_has_rows = wr0 < nrows;
  const int r = wr0 + col;
  const bool row_ok = r < nrows;
  const int my_i = row_ok ? r / G : S - 1;
  const int my_h = g * G + (row_ok ? r % G : 0);
  const int my_p = L + my_i;                                // causal limit
  const int my_ws = a.W > 0 ? max(0, my_p - a.W + 1) : 0;   // window start

  // workgroup and wave key ranges
  const int wg_ilo = r0 / G, wg_ihi = min(S - 1, (r0 + 127) / G);
  const int w_ilo = min(S - 1, wr0 / G), w_ihi = min(S - 1, (wr0 + 31) / G);
  const int wg_kstart = a.W > 0 ? max(0, L + wg_ilo - a.W + 1) : 0;
  const int wg_kend = L + wg_ihi + 1;
  const int w_kstart = a.W > 0 ? max(0, L + w_ilo - a.W + 1) : 0;
  const int w_kend = L + w_ihi + 1;
  const int w_full_lo = a.W > 0 ? L + w_ihi - a.W + 1 : 0;  // keys >= this: no window cut
  const int w_full_hi = L + w_ilo;                          // keys <= this: no causal cut

  // ---- Q^T (B operand): lane holds Q[row][16 ks + 8 c + e] ----
  uint4 qv[8];
  {
    const uint16_t* qrow = a.q + ((int64_t(b) * S + my_i) * a.H + my_h) * kD + 8 * c;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qv[ks] = row_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks) : make_uint4(0, 0, 0, 0);
    if (a.rot && row_ok) {
      const int pos = clamp_len(a.lens[b] + my_i, 0, a.rot_rows - 1);
      rotate_q<T>(qv, c, a.cosv + int64_t(pos) * (kD / 2), a.sinv + int64_t(pos) * (kD / 2),
                  a.interleaved);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qv[ks].x ^= a.q_sign; qv[ks].y ^= a.q_sign; qv[ks].z ^= a.q_sign; qv[ks].w ^= a.q_sign;
    }
  }

  const int64_t kvbase = (int64_t(b) * a.Hkv + g) * a.M * kD;
  const uint16_t* kc = a.k_cache + kvbase;
  const uint16_t* vc = a.v_cache + kvbase;

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  RowState rs{-INFINITY, 0.f, 0.f};
  const float cs = a.scale_log2;
  const int span = my_p - my_ws;

  const int t_begin = wg_kstart / kBK;
  const int t_end = (wg_kend + kBK - 1) / kBK;
  Stage st;
  stage_load(st, kc, vc, t_begin * kBK, kvalid, tid);
  stage_store(st, lds_k[0], lds_v[0], tid);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const int tb = t * kBK;
    const bool more = t + 1 < t_end;
    if (more) stage_load(st, kc, vc, tb + kBK, kvalid, tid);

    if (wave_has_rows && tb < w_kend && tb + kBK > w_kstart) {
      const bool full = tb + kBK - 1 <= w_full_hi && tb >= w_full_lo;
      const int lim_hi = my_p - (tb + 4 * c);
      if (full)
        tile_step<T, false>(lds_k[buf], lds_v[buf], qv, o, rs, cs, lim_hi, span, col, c);
      else
        tile_step<T, true>(lds_k[buf], lds_v[buf], qv, o, rs, cs, lim_hi, span, col, c);
    }
    if (more) stage_store(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
    __syncthreads();
  }

  if (!row_ok) return;
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs.l), __float_as_uint(rs.l),
                                                    false, false);
  const float inv = 1.f / (__uint_as_float(lsw[0]) + __uint_as_float(lsw[1]));
  uint16_t* orow = a.out + ((int64_t(b) * S + my_i) * a.H + my_h) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int d = 32 * dt + 8 * v4 + 4 * c;
      uint2 w;
      w.x = Mma32<T>::pack2(o[dt][4 * v4] * inv, o[dt][4 * v4 + 1] * inv);
      w.y = Mma32<T>::pack2(o[dt][4 * v4 + 2] * inv, o[dt][4 * v4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d) = w;
    }
}

}  // namespace

bool prefill_fast_supported(const Problem& p) {
  return p.D == 128 && (p.dtype == GQA_FP16 || p.dtype == GQA_BF16);
}

hipError_t launch_prefill_fast(const Problem& p, hipStream_t st) {
  PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k_cache = static_cast<const uint16_t*>(p.k_cache);
  a.v_cache = static_cast<const uint16_t*>(p.v_cache);
  a.out = static_cast<uint16_t*>(p.out);
  a.lens = p.lens_dev;
  a.cosv = p.cos; a.sinv = p.sin;
  a.B = p.B; a.S = p.S; a.H = p.H; a.Hkv = p.Hkv; a.G = p.G; a.M = p.M; a.W = p.window;
  a.rot = p.rot; a.rot_rows = p.rot_rows; a.interleaved = p.interleaved;
  a.n_rb = ceil_div(p.S * p.G, 128);
  a.scale_log2 = fabsf(p.scale) * kLog2e;
  a.q_sign = p.scale < 0.f ? 0x80008000u : 0u;
  const int blocks = a.n_rb * p.B * p.Hkv;
  if (blocks == 0) return hipSuccess;
  if (p.dtype == GQA_FP16)
    hipLaunchKernelGGL(prefill_kernel<F16>, dim3(blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_kernel<BF16>, dim3(blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace gqa
