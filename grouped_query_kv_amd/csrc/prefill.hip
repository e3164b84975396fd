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
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <class T> struct Mma32;
template <> struct Mma32<F16> {
  __device__ static inline f32x16 run(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> fp16 (nearest-even), packed
  __device__ static inline uint32_t pack2(float x, float y) {
    return uint32_t(F16::from_float(x)) | (uint32_t(F16::from_float(y)) << 16);
  }
};
template <> struct Mma32<BF16> {
  __device__ static inline f32x16 run(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    return uint32_t(BF16::from_float(x)) | (uint32_t(BF16::from_float(y)) << 16);
  }
};

constexpr int kD = 128;
constexpr int kBK = 64;                       // keys per tile
constexpr int kRows = 128;                    // query rows per workgroup
constexpr int kThreads = 256;
constexpr int kKStride = kD + 8;              // K tile row stride in halves (272 B)
constexpr int kVStride = kBK + 8;             // V^T tile row stride in halves (144 B)
constexpr int kKTile = kBK * kKStride;        // halves
constexpr int kVTile = kD * kVStride;         // halves
constexpr float kLog2e = 1.4426950408889634f;

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
  float scale_log2;
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

// Staging of one 64-key tile: thread (kq = tid / 16, dg = tid % 16) moves keys
// 4 kq .. 4 kq + 3, dims 8 dg .. 8 dg + 7, of K and V. Rows at or past the
// valid length are not read; zeros are staged.
struct Stage {
  uint4 k[4];
  uint4 v[4];
};

__device__ inline void stage_load(Stage& st, const uint16_t* kc, const uint16_t* vc, int tb,
                                  int kvalid, int tid) {
  const int kq = tid >> 4, dg = tid & 15;
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
  const int kq = tid >> 4, dg = tid & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint4*>(ks + (4 * kq + j) * kKStride + 8 * dg) = st.k[j];
  // V^T[d][pos]: within each 16 keys, key 8a + 4c + r sits at 8c + 4a + r
  const int u = kq >> 2, qd = kq & 3;                       // qd = 2a + c
  const int pos = 16 * u + 4 * (((qd & 1) << 1) | (qd >> 1));
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
    *reinterpret_cast<uint2*>(vs + (8 * dg + e) * kVStride + pos) = pk;
  }
}

template <class T>
__global__ void __launch_bounds__(kThreads, 2) prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKTile];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kVTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, c = lane >> 5;     // S^T column (= row of this wave), k half
  const int units = a.B * a.Hkv;
  const int rb = a.n_rb - 1 - int(blockIdx.x) / units;    // longest row blocks first
  const int bg = int(blockIdx.x) % units;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.G, S = a.S;
  const int nrows = S * G;
  const int L = clamp_len(a.lens[b], 0, a.M - S);
  const int kvalid = L + S;

  // rows of this workgroup / wave / lane
  const int r0 = rb * kRows;
  const int wr0 = r0 + 32 * wave;
  const bool wave_has_rows = wr0 < nrows;
  const int my_r = wr0 + col;
  const bool row_ok = my_r < nrows;
  const int my_i = row_ok ? my_r / G : S - 1;
  const int my_h = g * G + (row_ok ? my_r % G : 0);
  const int my_p = L + my_i;                              // causal limit
  const int my_ws = a.W > 0 ? my_p - a.W + 1 : 0;          // window start

  // workgroup and wave key ranges
  const int wg_ilo = r0 / G, wg_ihi = min(S - 1, (r0 + kRows - 1) / G);
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
  }

  const int64_t kvbase = (int64_t(b) * a.Hkv + g) * a.M * kD;
  const uint16_t* kc = a.k_cache + kvbase;
  const uint16_t* vc = a.v_cache + kvbase;

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

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

    const bool active = wave_has_rows && tb < w_kend && tb + kBK > w_kstart;
    if (active) {
      const uint16_t* ks = lds_k[buf];
      const uint16_t* vs = lds_v[buf];
      // ---- S^T = K Q^T: two 32-key halves of the tile ----
      f32x16 s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[h][v] = 0.f;
        const uint16_t* krow = ks + (32 * h + col) * kKStride + 8 * c;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          s[h] = Mma32<T>::run(*reinterpret_cast<const uint4*>(krow + 16 * kk), qv[kk], s[h]);
      }
      // ---- scale, mask (boundary tiles only), online softmax ----
      const bool full = tb + kBK - 1 <= w_full_hi && tb >= w_full_lo;
      float tmax = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = s[h][v] * a.scale_log2;
          if (!full) {
            const int key = tb + 32 * h + 8 * (v >> 2) + 4 * c + (v & 3);
            x = (key <= my_p && key >= my_ws) ? x : -INFINITY;
          }
          s[h][v] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      if (__any(m_new != m_run)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
      }
      l_run *= alpha;
      m_run = m_new;
      uint4 pk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = exp2f(s[u >> 1][8 * (u & 1) + e] - m_use);
          l_run += p[e];
        }
        pk[u].x = Mma32<T>::pack2(p[0], p[1]);
        pk[u].y = Mma32<T>::pack2(p[2], p[3]);
        pk[u].z = Mma32<T>::pack2(p[4], p[5]);
        pk[u].w = Mma32<T>::pack2(p[6], p[7]);
      }
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* vrow = vs + (32 * dt + col) * kVStride + 8 * c;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[dt] = Mma32<T>::run(*reinterpret_cast<const uint4*>(vrow + 16 * u), pk[u], o[dt]);
      }
    }
    if (more) stage_store(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
    __syncthreads();
  }

  if (!row_ok) return;
  l_run += __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_run;
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
  a.n_rb = ceil_div(p.S * p.G, kRows);
  a.scale_log2 = p.scale * kLog2e;
  const int blocks = a.n_rb * p.B * p.Hkv;
  if (blocks == 0) return hipSuccess;
  if (p.dtype == GQA_FP16)
    hipLaunchKernelGGL(prefill_kernel<F16>, dim3(blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_kernel<BF16>, dim3(blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace gqa
