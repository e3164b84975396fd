// Split-KV decode for fp16/bf16 with head_size 128 (one new token per
// sequence).
//
// The key axis of sequence b grows with every step and lives in a buffer of M
// rows ("KV Cache" discussion, notes): only rows [kstart, L'_b] are touched.
// They are cut into splits of `chunk` keys; one workgroup (4 waves) streams
// one split of one (b, kv head, head group) and the G query heads that share
// the kv head reuse every K/V row it loads.
//
//  * QK^T runs on MFMA 16x16x32 with keys as the M rows and the head group
//    padded to the 16 N columns (A = 16 keys x 32 dims straight from HBM,
//    B = Q^T held in registers for the whole split).
//  * Softmax is online per 64-key block; the block's P and the rescale
//    factors go through LDS to the PV layout, in which each lane owns 8 head
//    dimensions of 4 keys and accumulates P V on the VALU in fp32.
//  * The new token's K/V row is read from k_new/v_new (rotated if asked),
//    used directly, and written to row L'_b of the cache by the workgroup
//    holding the last split: the append is fused, nothing reads that row
//    from memory in this call.
//  * Each split ends with (unnormalised o, m, l) per head; the last workgroup
//    of a (b, kv head, head group) to finish (an atomic counter in the
//    workspace) merges them by log-sum-exp, writes the output and resets the
//    counter.
//
// Keys past the split end are clamped to a valid row and get p = 0 exactly,
// so no NaN from the unused part of the buffer can reach an accumulator.
#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class T> struct Mma;
template <> struct Mma<F16> {
  __device__ static inline f32x4 run(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<BF16> {
  __device__ static inline f32x4 run(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

constexpr int kD = 128;
constexpr int kBlock = kDecodeBlockKeys;   // 64 keys per wave iteration
constexpr int kTiles = kBlock / 16;        // 16-key MFMA tiles per block
constexpr int kSlotFloats = kDecodeMaxHG * (kD + 2);
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* out;
  const int32_t* lens;
  const float* cosv;
  const float* sinv;
  float* partials;
  int* counters;
  int B, H, Hkv, G, M, W;
  int rot, rot_rows, interleaved;
  int n_hg, hg_size;
  int chunk, max_splits;
  float scale_log2;
};

struct Range {
  int L, Lp, kstart, kend;
};

__device__ inline Range key_range(const DecodeArgs& a, int b) {
  Range r;
  r.L = clamp_len(a.lens[b], 0, a.M);
  r.Lp = r.L < a.M - 1 ? r.L : a.M - 1;   // row of the new token (after any eviction)
  r.kend = r.Lp + 1;
  r.kstart = a.W > 0 ? (r.kend - a.W > 0 ? r.kend - a.W : 0) : 0;
  return r;
}

__device__ inline int nsplit(const DecodeArgs& a, int b) {
  const Range r = key_range(a, b);
  return (r.kend - r.kstart + a.chunk - 1) / a.chunk;
}

// Rotate the 4 loaded 16-byte chunks of one 128-dim row in place. Chunk i
// holds dims 32 i + 8 q4 + e (e = 0..7): rotate-half pairs (d, d + 64) sit in
// chunks (i, i + 2) of the same lane; interleaved pairs sit in one chunk.
template <class T>
__device__ inline void rotate_row_chunks(uint4 (&c)[4], int q4, const float* cosr,
                                         const float* sinr, int interleaved) {
  using Bits = typename T::bits;
  Bits x[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] = Bits((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
  }
  if (!interleaved) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * i + 8 * q4 + e;
        rotate_pair<T>(x[i][e], x[i + 2][e], cosr[j], sinr[j]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int j = (32 * i + 8 * q4 + e) >> 1;
        rotate_pair<T>(x[i][e], x[i][e + 1], cosr[j], sinr[j]);
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i].x = uint32_t(x[i][0]) | (uint32_t(x[i][1]) << 16);
    c[i].y = uint32_t(x[i][2]) | (uint32_t(x[i][3]) << 16);
    c[i].z = uint32_t(x[i][4]) | (uint32_t(x[i][5]) << 16);
    c[i].w = uint32_t(x[i][6]) | (uint32_t(x[i][7]) << 16);
  }
}

template <class T>
__device__ inline void unpack8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = T::to_float(typename T::bits(w[k] & 0xFFFFu));
    f[2 * k + 1] = T::to_float(typename T::bits(w[k] >> 16));
  }
}

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <class T, int HG>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  constexpr int HP = HG < 4 ? 4 : HG;            // padded LDS row for vector reads
  __shared__ __attribute__((aligned(16))) float p_lds[kDecodeWaves][kBlock][HP];
  __shared__ float alpha_lds[kDecodeWaves][16];
  __shared__ float mo[kDecodeWaves][HG][kD];
  __shared__ float mm[kDecodeWaves][HG], ml[kDecodeWaves][HG];
  __shared__ int sh_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q4 = lane >> 4;   // S layout: head column, key quad
  int w = blockIdx.x;
  const int hg = w % a.n_hg;
  w /= a.n_hg;
  const int g = w % a.Hkv;
  w /= a.Hkv;

  // --- which (b, split) this workgroup takes: prefix sum of split counts ---
  int b = -1, split = 0;
  {
    int base = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int bi = b0 + lane;
      const int ns = bi < a.B ? nsplit(a, bi) : 0;
      int incl = ns;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const int excl = incl - ns;
      const unsigned long long hit = __ballot(bi < a.B && w >= base + excl && w < base + incl);
      if (hit) {
        const int src = __ffsll((long long)hit) - 1;
        b = b0 + src;
        split = w - base - __shfl(excl, src, 64);
        break;
      }
      base += __shfl(incl, 63, 64);
    }
  }
  if (b < 0) return;  // only if the device lengths disagree with the host's

  const Range R = key_range(a, b);
  const int nspl = (R.kend - R.kstart + a.chunk - 1) / a.chunk;
  const int c0 = R.kstart + split * a.chunk;
  const int c1 = min(R.kend, c0 + a.chunk);
  const int nblk = (c1 - c0 + kBlock - 1) / kBlock;
  const int h0 = g * a.G + hg * a.hg_size;
  const int nheads = min(a.hg_size, a.G - hg * a.hg_size);
  const int half = kD / 2;
  const int pos = clamp_len(R.L, 0, a.rot_rows > 0 ? a.rot_rows - 1 : 0);
  const float* cosr = a.rot ? a.cosv + int64_t(pos) * half : nullptr;
  const float* sinr = a.rot ? a.sinv + int64_t(pos) * half : nullptr;

  // --- Q^T as the MFMA B operand: lane (n, q4) holds dims 32 i + 8 q4 + e ---
  uint4 qv[4];
  {
    const uint16_t* qrow = a.q + (int64_t(b) * a.H + h0 + n) * kD + 8 * q4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qv[i] = n < nheads ? *reinterpret_cast<const uint4*>(qrow + 32 * i) : make_uint4(0, 0, 0, 0);
    if (a.rot && n < nheads) rotate_row_chunks<T>(qv, q4, cosr, sinr, a.interleaved);
  }

  const int64_t kvbase = (int64_t(b) * a.Hkv + g) * a.M * kD;
  const uint16_t* kc = a.k_cache + kvbase;
  const uint16_t* vc = a.v_cache + kvbase;

  // ---- fused append: the workgroup whose split holds row L'_b writes the new
  // token's (rotated) K row and V row there first, then reads it like any
  // other row. No other workgroup touches that row in this call. ----
  if (R.Lp >= c0 && R.Lp < c1) {
    using Bits = typename T::bits;
    const Bits* knew = reinterpret_cast<const Bits*>(a.k_new) + (int64_t(b) * a.Hkv + g) * kD;
    const Bits* vnew = reinterpret_cast<const Bits*>(a.v_new) + (int64_t(b) * a.Hkv + g) * kD;
    Bits* kdst = reinterpret_cast<Bits*>(a.k_cache + kvbase + int64_t(R.Lp) * kD);
    Bits* vdst = reinterpret_cast<Bits*>(a.v_cache + kvbase + int64_t(R.Lp) * kD);
    if (tid < half) {
      const int e1 = a.interleaved ? 2 * tid : tid;
      const int e2 = a.interleaved ? 2 * tid + 1 : tid + half;
      Bits x = knew[e1], y = knew[e2];
      if (a.rot) rotate_pair<T>(x, y, cosr[tid], sinr[tid]);
      kdst[e1] = x;
      kdst[e2] = y;
    } else if (tid < half + kD / 8) {
      const int c = tid - half;
      reinterpret_cast<uint4*>(vdst)[c] = reinterpret_cast<const uint4*>(vnew)[c];
    }
    __threadfence_block();
    __syncthreads();
  }

  float m_run = -INFINITY, l_run = 0.f;
  float o[HG][8];
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;

  const int rq = lane >> 4, dg = lane & 15;   // PV layout: key quad, dim group
  for (int blk = wave; blk < nblk; blk += kDecodeWaves) {
    const int kb = c0 + blk * kBlock;
    // ---- loads: K in MFMA A layout, V in row layout ----
    uint4 kr[kTiles][4], vr[kTiles][4];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int key = kb + 16 * t + n;
      const uint16_t* src = kc + int64_t(key < c1 ? key : c0) * kD + 8 * q4;
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[t][i] = *reinterpret_cast<const uint4*>(src + 32 * i);
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 16 * t + 4 * rq + r;
        vr[t][r] = *reinterpret_cast<const uint4*>(vc + int64_t(key < c1 ? key : c0) * kD + 8 * dg);
      }
    // ---- S^T = K Q^T on MFMA: lane gets keys 16 t + 4 q4 + r of head n ----
    float s[kTiles][4];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = Mma<T>::run(kr[t][i], qv[i], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 16 * t + 4 * q4 + r;
        s[t][r] = key < c1 ? acc[r] * a.scale_log2 : -INFINITY;
      }
    }
    // ---- online softmax (per head column; the 4 key quads share m) ----
    float bm = s[0][0];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) bm = fmaxf(bm, s[t][r]);
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float mn = fmaxf(m_run, bm);
    const float alpha = exp2f(m_run - mn);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[t][r] - mn);
        psum += p;
        if (n < HG) p_lds[wave][16 * t + 4 * q4 + r][n] = p;
      }
    l_run = l_run * alpha + psum;
    m_run = mn;
    if (q4 == 0) alpha_lds[wave][n] = alpha;
    wave_lds_sync();
    // ---- P V on the VALU: lane owns dims 8 dg..8 dg+7 of keys 16 t + 4 rq + r ----
    float al[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) al[h] = alpha_lds[wave][h];
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= al[h];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float* prow = p_lds[wave][16 * t + 4 * rq + r];
        float pv[HP];
#pragma unroll
        for (int h = 0; h < HP; h += 4) {
          const float4 x = *reinterpret_cast<const float4*>(prow + h);
          pv[h] = x.x; pv[h + 1] = x.y; pv[h + 2] = x.z; pv[h + 3] = x.w;
        }
        float v[8];
        unpack8<T>(vr[t][r], v);
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pv[h], v[e], o[h][e]);
      }
    wave_lds_sync();
  }

  // ---- wave totals: l over key quads (same head), o over key quads (same dims) ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[h][e] += __shfl_xor(o[h][e], 16, 64);
      o[h][e] += __shfl_xor(o[h][e], 32, 64);
    }
  if (rq == 0) {
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) mo[wave][h][8 * dg + e] = o[h][e];
  }
  if (q4 == 0 && n < HG) {
    mm[wave][n] = m_run;
    ml[wave][n] = l_run;
  }
  __syncthreads();

  // ---- merge the 4 waves: (o, m, l) of this split per head ----
  float res_o[(HG * kD + 255) / 256], res_m[(HG * kD + 255) / 256], res_l[(HG * kD + 255) / 256];
#pragma unroll
  for (int k = 0; k < (HG * kD + 255) / 256; ++k) {
    const int idx = tid + 256 * k;
    res_o[k] = 0.f; res_m[k] = -INFINITY; res_l[k] = 0.f;
    if (idx < HG * kD) {
      const int h = idx / kD, d = idx % kD;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kDecodeWaves; ++v) M = fmaxf(M, mm[v][h]);
      float ls = 0.f, os = 0.f;
#pragma unroll
      for (int v = 0; v < kDecodeWaves; ++v) {
        const float wgt = exp2f(mm[v][h] - M);   // 0 for a wave with no keys
        ls = fmaf(ml[v][h], wgt, ls);
        os = fmaf(mo[v][h][d], wgt, os);
      }
      res_o[k] = os; res_m[k] = M; res_l[k] = ls;
    }
  }
  if (nspl == 1) {
#pragma unroll
    for (int k = 0; k < (HG * kD + 255) / 256; ++k) {
      const int idx = tid + 256 * k;
      const int h = idx / kD, d = idx % kD;
      if (idx < HG * kD && h < nheads)
        a.out[(int64_t(b) * a.H + h0 + h) * kD + d] = T::from_float(res_o[k] / res_l[k]);
    }
    return;
  }
  const int unit = (b * a.Hkv + g) * a.n_hg + hg;
  float* slot = a.partials + (int64_t(unit) * a.max_splits + split) * kSlotFloats;
#pragma unroll
  for (int k = 0; k < (HG * kD + 255) / 256; ++k) {
    const int idx = tid + 256 * k;
    if (idx < HG * kD) {
      const int h = idx / kD, d = idx % kD;
      slot[h * kD + d] = res_o[k];
      if (d == 0) {
        slot[kDecodeMaxHG * kD + h] = res_m[k];
        slot[kDecodeMaxHG * kD + kDecodeMaxHG + h] = res_l[k];
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(a.counters + unit, 1);
    sh_last = prev == nspl - 1;
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  const float* slots = a.partials + int64_t(unit) * a.max_splits * kSlotFloats;
#pragma unroll
  for (int k = 0; k < (HG * kD + 255) / 256; ++k) {
    const int idx = tid + 256 * k;
    const int h = idx / kD, d = idx % kD;
    if (idx < HG * kD && h < nheads) {
      float M = -INFINITY;
      for (int s2 = 0; s2 < nspl; ++s2) M = fmaxf(M, slots[s2 * kSlotFloats + kDecodeMaxHG * kD + h]);
      float ls = 0.f, os = 0.f;
      for (int s2 = 0; s2 < nspl; ++s2) {
        const float* sl = slots + s2 * kSlotFloats;
        const float wgt = exp2f(sl[kDecodeMaxHG * kD + h] - M);
        ls = fmaf(sl[kDecodeMaxHG * kD + kDecodeMaxHG + h], wgt, ls);
        os = fmaf(sl[h * kD + d], wgt, os);
      }
      a.out[(int64_t(b) * a.H + h0 + h) * kD + d] = T::from_float(os / ls);
    }
  }
  if (tid == 0) a.counters[unit] = 0;  // ready for the next call
}

template <class T, int HG>
void launch(const DecodeArgs& a, int blocks, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<T, HG>), dim3(blocks), dim3(256), 0, st, a);
}

template <class T>
void launch_hg(const DecodeArgs& a, int hgt, int blocks, hipStream_t st) {
  switch (hgt) {
    case 1: launch<T, 1>(a, blocks, st); break;
    case 2: launch<T, 2>(a, blocks, st); break;
    case 4: launch<T, 4>(a, blocks, st); break;
    default: launch<T, 8>(a, blocks, st); break;
  }
}

}  // namespace

bool decode_fast_supported(const Problem& p) {
  return p.D == 128 && (p.dtype == GQA_FP16 || p.dtype == GQA_BF16) && p.S == 1;
}

hipError_t launch_decode_fast(const Problem& p, void* ws, const WorkspaceLayout& lay,
                              hipStream_t st) {
  DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k_new = static_cast<const uint16_t*>(p.k_new);
  a.v_new = static_cast<const uint16_t*>(p.v_new);
  a.k_cache = static_cast<uint16_t*>(p.k_cache);
  a.v_cache = static_cast<uint16_t*>(p.v_cache);
  a.out = static_cast<uint16_t*>(p.out);
  a.lens = p.lens_dev;
  a.cosv = p.cos; a.sinv = p.sin;
  a.rot = p.rot; a.rot_rows = p.rot_rows; a.interleaved = p.interleaved;
  a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.scratch);
  a.counters = reinterpret_cast<int*>(static_cast<char*>(ws) + lay.counters);
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.G = p.G; a.M = p.M; a.W = p.window;
  a.n_hg = ceil_div(p.G, kDecodeMaxHG);
  a.hg_size = ceil_div(p.G, a.n_hg);
  int hgt = 1;
  while (hgt < a.hg_size) hgt <<= 1;
  a.max_splits = ceil_div(p.M, kDecodeMinChunk);
  a.scale_log2 = p.scale * kLog2e;
  // split size: aim for a few workgroups per CU over the whole call
  int64_t total_keys = 0;
  for (int b = 0; b < p.B; ++b) {
    const int L = p.lens_host[b] < p.M - 1 ? p.lens_host[b] : p.M - 1;
    const int kend = L + 1;
    const int kstart = p.window > 0 ? (kend - p.window > 0 ? kend - p.window : 0) : 0;
    total_keys += kend - kstart;
  }
  const int64_t units = int64_t(p.Hkv) * a.n_hg;
  const int64_t target_wg = 1024;
  int64_t chunk = (total_keys * units + target_wg - 1) / target_wg;
  chunk = ((chunk + kDecodeMinChunk - 1) / kDecodeMinChunk) * kDecodeMinChunk;
  if (chunk < kDecodeMinChunk) chunk = kDecodeMinChunk;
  a.chunk = int(chunk);
  int64_t splits = 0;
  for (int b = 0; b < p.B; ++b) {
    const int L = p.lens_host[b] < p.M - 1 ? p.lens_host[b] : p.M - 1;
    const int kend = L + 1;
    const int kstart = p.window > 0 ? (kend - p.window > 0 ? kend - p.window : 0) : 0;
    splits += (kend - kstart + a.chunk - 1) / a.chunk;
  }
  const int blocks = int(splits * units);
  if (blocks == 0) return hipSuccess;
  if (p.dtype == GQA_FP16) launch_hg<F16>(a, hgt, blocks, st);
  else launch_hg<BF16>(a, hgt, blocks, st);
  return hipGetLastError();
}

}  // namespace gqa
