// Append: scatter the S new K/V rows of every (b, kv head) into the shared
// BNSH buffer at row L'_b + i. Source rows [B, S, Hkv*D] are read in their
// own order (fully coalesced); each destination row is one contiguous run.
// Rotary (on K only) uses the fp64 rounding rule of rotate_pair.
#include <algorithm>

#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

// Rotary position of sequence b's first new token: the absolute position of
// buffer row 0 (0 without offsets) plus the past length before any eviction.
__device__ inline int rotary_base(const int32_t* lens, const int32_t* offs, int b, int M) {
  return clamp_len(lens[b], 0, M) + (offs ? offs[b] : 0);
}

// Destination row of sequence b's first new token. With a window (cap > 0)
// the buffer was just compacted, so the append starts at the rows it kept.
__device__ inline int dest_base(const int32_t* lens, int b, int S, int M, int cap) {
  int L = clamp_len(lens[b], 0, M);
  if (cap > 0) L = kept_rows(L, S, M, cap);
  return clamp_len(L, 0, M - S);
}

// One thread per `U`-sized unit of a row; the flat source index is the unit
// index itself because [B, S, Hkv, D] flattens in the same order.
template <class U>
__global__ void __launch_bounds__(256) copy_rows_kernel(const U* __restrict__ src,
                                                        U* __restrict__ dst,
                                                        const int32_t* __restrict__ lens, int B,
                                                        int S, int Hkv, int M, int upr,
                                                        int cap) {
  const int64_t total = int64_t(B) * S * Hkv * upr;
  for (int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; idx < total;
       idx += int64_t(gridDim.x) * blockDim.x) {
    int64_t r = idx;
    const int u = int(r % upr); r /= upr;
    const int g = int(r % Hkv); r /= Hkv;
    const int i = int(r % S);
    const int b = int(r / S);
    const int row = dest_base(lens, b, S, M, cap) + i;
    dst[((int64_t(b) * Hkv + g) * M + row) * upr + u] = src[idx];
  }
}

// One thread per rotary pair of K.
template <class T>
__global__ void __launch_bounds__(256) rotary_rows_kernel(
    const typename T::bits* __restrict__ src, typename T::bits* __restrict__ dst,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ offs, int B, int S, int Hkv,
    int D, int M, const float* __restrict__ cosv, const float* __restrict__ sinv, int rot_rows,
    int interleaved, int cap) {
  const int half = D / 2;
  const int64_t total = int64_t(B) * S * Hkv * half;
  for (int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; idx < total;
       idx += int64_t(gridDim.x) * blockDim.x) {
    int64_t r = idx;
    const int j = int(r % half); r /= half;
    const int g = int(r % Hkv); r /= Hkv;
    const int i = int(r % S);
    const int b = int(r / S);
    const int pos = clamp_len(rotary_base(lens, offs, b, M) + i, 0, rot_rows - 1);
    const int e1 = interleaved ? 2 * j : j;
    const int e2 = interleaved ? 2 * j + 1 : j + half;
    const int64_t s0 = ((int64_t(b) * S + i) * Hkv + g) * D;
    typename T::bits a = src[s0 + e1], c = src[s0 + e2];
    rotate_pair<T>(a, c, cosv[int64_t(pos) * half + j], sinv[int64_t(pos) * half + j]);
    const int row = dest_base(lens, b, S, M, cap) + i;
    const int64_t d0 = ((int64_t(b) * Hkv + g) * M + row) * D;
    dst[d0 + e1] = a;
    dst[d0 + e2] = c;
  }
}

// Vector form for 2-byte types with D % 16 == 0: one thread per 8 rotary
// pairs of one row (rotate-half: 16 bytes from each half of the row;
// interleaved: two 16-byte runs of 4 pairs each), 16-byte loads and stores,
// index arithmetic once per thread.
template <class T>
__device__ inline void rot8(uint4& x, uint4& y, const float* c8, const float* s8) {
  using Bits = typename T::bits;
  uint32_t* xw = &x.x;
  uint32_t* yw = &y.x;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    Bits x0 = Bits(xw[w] & 0xFFFFu), x1 = Bits(xw[w] >> 16);
    Bits y0 = Bits(yw[w] & 0xFFFFu), y1 = Bits(yw[w] >> 16);
    rotate_pair<T>(x0, y0, c8[2 * w], s8[2 * w]);
    rotate_pair<T>(x1, y1, c8[2 * w + 1], s8[2 * w + 1]);
    xw[w] = uint32_t(x0) | (uint32_t(x1) << 16);
    yw[w] = uint32_t(y0) | (uint32_t(y1) << 16);
  }
}

template <class T>
__device__ inline void rot_inter8(uint4& x, const float* c4, const float* s4) {
  using Bits = typename T::bits;
  uint32_t* xw = &x.x;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    Bits a = Bits(xw[w] & 0xFFFFu), b = Bits(xw[w] >> 16);
    rotate_pair<T>(a, b, c4[w], s4[w]);
    xw[w] = uint32_t(a) | (uint32_t(b) << 16);
  }
}

// Fused append for 2-byte types with D % 16 == 0: K and V in one launch. A
// thread owns 16 elements of one source row, split over two 16-byte runs
// (rotate-half: the same 8 offsets in each half, so a run pairs with the
// other; interleaved: two adjacent runs of 4 pairs each). K is rotated when
// tables are given, V is copied; index arithmetic once per thread.
template <class T>
__global__ void __launch_bounds__(256) append_rows_vec_kernel(
    const uint16_t* __restrict__ k_src, uint16_t* __restrict__ k_dst,
    const uint16_t* __restrict__ v_src, uint16_t* __restrict__ v_dst,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ offs, int B, int S, int Hkv,
    int D, int M, const float* __restrict__ cosv, const float* __restrict__ sinv, int rot,
    int rot_rows, int interleaved, int cap) {
  const int half = D / 2;
  const int cpr = D / 16;                         // threads per row: 16 elements each
  const int64_t total = int64_t(B) * S * Hkv * cpr;
  for (int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; idx < total;
       idx += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = idx / cpr;                  // source row (b, i, g)
    const int ch = int(idx - r * cpr);
    const int g = int(r % Hkv);
    const int64_t bi = r / Hkv;
    const int i = int(bi % S), b = int(bi / S);
    const int row = dest_base(lens, b, S, M, cap) + i;
    const int64_t doff = ((int64_t(b) * Hkv + g) * M + row) * D;
    // the two 16-byte runs of this thread (element offsets within the row)
    const int o1 = interleaved ? 16 * ch : 8 * ch;
    const int o2 = interleaved ? 16 * ch + 8 : 8 * ch + half;
    const uint16_t* ks = k_src + r * D;
    const uint16_t* vs = v_src + r * D;
    uint4 x = *reinterpret_cast<const uint4*>(ks + o1);
    uint4 y = *reinterpret_cast<const uint4*>(ks + o2);
    const uint4 vx = *reinterpret_cast<const uint4*>(vs + o1);
    const uint4 vy = *reinterpret_cast<const uint4*>(vs + o2);
    if (rot) {
      const int pos = clamp_len(rotary_base(lens, offs, b, M) + i, 0, rot_rows - 1);
      const float* cr = cosv + int64_t(pos) * half + 8 * ch;   // pairs 8 ch .. 8 ch + 7
      const float* sr = sinv + int64_t(pos) * half + 8 * ch;
      const float4 c0 = *reinterpret_cast<const float4*>(cr);
      const float4 c1 = *reinterpret_cast<const float4*>(cr + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(sr);
      const float4 s1 = *reinterpret_cast<const float4*>(sr + 4);
      if (!interleaved) {
        const float c8[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float s8[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        rot8<T>(x, y, c8, s8);
      } else {
        const float ca[4] = {c0.x, c0.y, c0.z, c0.w}, sa[4] = {s0.x, s0.y, s0.z, s0.w};
        const float cb[4] = {c1.x, c1.y, c1.z, c1.w}, sb[4] = {s1.x, s1.y, s1.z, s1.w};
        rot_inter8<T>(x, ca, sa);
        rot_inter8<T>(y, cb, sb);
      }
    }
    *reinterpret_cast<uint4*>(k_dst + doff + o1) = x;
    *reinterpret_cast<uint4*>(k_dst + doff + o2) = y;
    *reinterpret_cast<uint4*>(v_dst + doff + o1) = vx;
    *reinterpret_cast<uint4*>(v_dst + doff + o2) = vy;
  }
}

int grid_for(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = 256 * 64;  // enough workgroups to fill the chip many times
  return int(blocks < 1 ? 1 : (blocks > cap ? cap : blocks));
}

hipError_t copy_rows(const void* src, void* dst, const Problem& p, bool evicted,
                     hipStream_t st) {
  const int row_bytes = p.D * (p.dtype == GQA_FP32 ? 4 : 2);
  const int64_t rows = int64_t(p.B) * p.S * p.Hkv;
  if (row_bytes % 16 == 0) {
    const int upr = row_bytes / 16;
    hipLaunchKernelGGL(copy_rows_kernel<uint4>, dim3(grid_for(rows * upr)), dim3(256), 0, st,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), p.lens_dev,
                       p.B, p.S, p.Hkv, p.M, upr, evicted ? p.cap : 0);
  } else if (row_bytes % 4 == 0) {
    const int upr = row_bytes / 4;
    hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, dim3(grid_for(rows * upr)), dim3(256), 0,
                       st, static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst),
                       p.lens_dev, p.B, p.S, p.Hkv, p.M, upr, evicted ? p.cap : 0);
  } else {
    const int upr = row_bytes / 2;
    hipLaunchKernelGGL(copy_rows_kernel<uint16_t>, dim3(grid_for(rows * upr)), dim3(256), 0,
                       st, static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst),
                       p.lens_dev, p.B, p.S, p.Hkv, p.M, upr, evicted ? p.cap : 0);
  }
  return hipGetLastError();
}

template <class T>
hipError_t rotary_rows(const Problem& p, bool evicted, hipStream_t st) {
  using Bits = typename T::bits;
  const int64_t total = int64_t(p.B) * p.S * p.Hkv * (p.D / 2);
  hipLaunchKernelGGL(rotary_rows_kernel<T>, dim3(grid_for(total)), dim3(256), 0, st,
                     static_cast<const Bits*>(p.k_new), static_cast<Bits*>(p.k_cache),
                     p.lens_dev, p.off_dev, p.B, p.S, p.Hkv, p.D, p.M, p.cos, p.sin, p.rot_rows,
                     p.interleaved, evicted ? p.cap : 0);
  return hipGetLastError();
}

template <class T>
hipError_t append_rows_vec(const Problem& p, bool evicted, hipStream_t st) {
  const int64_t total = int64_t(p.B) * p.S * p.Hkv * (p.D / 16);
  hipLaunchKernelGGL(append_rows_vec_kernel<T>, dim3(grid_for(total)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(p.k_new), static_cast<uint16_t*>(p.k_cache),
                     static_cast<const uint16_t*>(p.v_new), static_cast<uint16_t*>(p.v_cache),
                     p.lens_dev, p.off_dev, p.B, p.S, p.Hkv, p.D, p.M, p.cos, p.sin, p.rot, p.rot_rows,
                     p.interleaved, evicted ? p.cap : 0);
  return hipGetLastError();
}


// Prefix copy between two BNSH buffers of different row counts: y = (kv head,
// K|V), z = b; the x workgroups stride over the rows [lo_b, L_b) of that
// (b, kv head) in `U`-sized units, one unit per thread per pass.
template <class U>
__global__ void __launch_bounds__(256) copy_prefix_kernel(
    const U* __restrict__ src_k, const U* __restrict__ src_v, int src_rows, U* __restrict__ dst_k,
    U* __restrict__ dst_v, int dst_rows, const int32_t* __restrict__ lens, int Hkv, int upr,
    int window) {
  const int y = blockIdx.y, b = blockIdx.z, g = y >> 1;
  const int L = clamp_len(lens[b], 0, src_rows < dst_rows ? src_rows : dst_rows);
  int lo = 0;
  if (window > 0) {
    lo = L - window + 1 > 0 ? L - window + 1 : 0;
    lo -= lo % kStageAlignRows;
  }
  const U* src = ((y & 1) ? src_v : src_k) + (int64_t(b) * Hkv + g) * src_rows * int64_t(upr);
  U* dst = ((y & 1) ? dst_v : dst_k) + (int64_t(b) * Hkv + g) * dst_rows * int64_t(upr);
  const int64_t end = int64_t(L) * upr;
  for (int64_t u = int64_t(lo) * upr + blockIdx.x * int64_t(blockDim.x) + threadIdx.x; u < end;
       u += int64_t(gridDim.x) * blockDim.x)
    dst[u] = src[u];
}

}  // namespace

hipError_t launch_append(const Problem& p, bool evicted, hipStream_t st) {
  if (p.B == 0 || p.S == 0) return hipSuccess;
  // fp16/bf16 rows of 16-element runs: K and V in one launch (float4 rotary
  // reads need 16-byte aligned tables)
  const bool tables_aligned = !p.rot || ((reinterpret_cast<uintptr_t>(p.cos) |
                                          reinterpret_cast<uintptr_t>(p.sin)) & 15) == 0;
  if (p.dtype != GQA_FP32 && p.D % 16 == 0 && tables_aligned)
    return p.dtype == GQA_FP16 ? append_rows_vec<F16>(p, evicted, st)
                               : append_rows_vec<BF16>(p, evicted, st);
  hipError_t e;
  if (p.rot) {
    if (p.dtype == GQA_FP32) e = rotary_rows<F32>(p, evicted, st);
    else if (p.dtype == GQA_FP16) e = rotary_rows<F16>(p, evicted, st);
    else e = rotary_rows<BF16>(p, evicted, st);
  } else {
    e = copy_rows(p.k_new, p.k_cache, p, evicted, st);
  }
  if (e != hipSuccess) return e;
  return copy_rows(p.v_new, p.v_cache, p, evicted, st);
}

hipError_t launch_copy_prefix(const void* src_k, const void* src_v, int src_rows, void* dst_k,
                              void* dst_v, int dst_rows, const int32_t* lens_dev, int B, int Hkv,
                              int row_bytes, int window, int max_len, hipStream_t st) {
  if (B == 0 || max_len <= 0) return hipSuccess;
  const int unit = row_bytes % 16 == 0 ? 16 : (row_bytes % 4 == 0 ? 4 : 2);
  const int upr = row_bytes / unit;
  // enough workgroups per (b, kv head, K|V) that one pass covers the longest
  // prefix at 16 units per thread; the kernel strides over the rest
  const int64_t units = int64_t(std::min(max_len, std::min(src_rows, dst_rows))) * upr;
  const int gx = int(std::max<int64_t>(1, std::min<int64_t>(64, (units + 4095) / 4096)));
  const dim3 grid(gx, Hkv * 2, B);
  if (unit == 16)
    hipLaunchKernelGGL(copy_prefix_kernel<uint4>, grid, dim3(256), 0, st,
                       static_cast<const uint4*>(src_k), static_cast<const uint4*>(src_v), src_rows,
                       static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), dst_rows, lens_dev,
                       Hkv, upr, window);
  else if (unit == 4)
    hipLaunchKernelGGL(copy_prefix_kernel<uint32_t>, grid, dim3(256), 0, st,
                       static_cast<const uint32_t*>(src_k), static_cast<const uint32_t*>(src_v),
                       src_rows, static_cast<uint32_t*>(dst_k), static_cast<uint32_t*>(dst_v),
                       dst_rows, lens_dev, Hkv, upr, window);
  else
    hipLaunchKernelGGL(copy_prefix_kernel<uint16_t>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(src_k), static_cast<const uint16_t*>(src_v),
                       src_rows, static_cast<uint16_t*>(dst_k), static_cast<uint16_t*>(dst_v),
                       dst_rows, lens_dev, Hkv, upr, window);
  return hipGetLastError();
}

}  // namespace gqa
