// Device helpers for the gfx950 kernels: storage types, conversions, the
// rotary rounding rule and small wave utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// ----------------------------------------------------------------------------
// storage dtypes. Elements are handled as raw bits; arithmetic is fp32 (fp64
// for rotary).
// ----------------------------------------------------------------------------
struct F32 {
  using bits = uint32_t;
  static constexpr int kBytes = 4;
  __device__ static inline float to_float(bits u) { return __uint_as_float(u); }
  __device__ static inline bits from_float(float f) { return __float_as_uint(f); }
};

struct F16 {
  using bits = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static inline float to_float(bits u) {
    return static_cast<float>(__builtin_bit_cast(_Float16, u));
  }
  // v_cvt_f16_f32 rounds to nearest-even
  __device__ static inline bits from_float(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  }
};

struct BF16 {
  using bits = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static inline float to_float(bits u) { return __uint_as_float(uint32_t(u) << 16); }
  // nearest-even on the fp32 bit pattern (inputs here are finite)
  __device__ static inline bits from_float(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
};

// Rotary pair (x1, x2) by (c, s): each output is one fp64 expression whose two
// products are exact (<= 24-bit times 24-bit significands), so it carries a
// single rounding whether or not the compiler contracts it into an fma; then
// fp64 -> fp32 -> storage dtype, both nearest-even.
template <class T>
__device__ inline void rotate_pair(typename T::bits& a, typename T::bits& b, float c, float s) {
  const double x1 = static_cast<double>(T::to_float(a));
  const double x2 = static_cast<double>(T::to_float(b));
  const double dc = static_cast<double>(c), ds = static_cast<double>(s);
  const double y1 = x1 * dc - x2 * ds;
  const double y2 = x2 * dc + x1 * ds;
  float f1 = static_cast<float>(y1), f2 = static_cast<float>(y2);
  // The compiler would otherwise fold fp64->fp32->fp16 into one fp64->fp16
  // rounding, which differs from the two-step rule exactly at fp16 ties.
  asm volatile("" : "+v"(f1), "+v"(f2));
  a = T::from_float(f1);
  b = T::from_float(f2);
}

// ----------------------------------------------------------------------------
// wave (64-lane) helpers
// ----------------------------------------------------------------------------
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Lengths as the kernels see them: clamped so that every access stays inside
// the buffer even if the device copy disagrees with the validated host copy.
__device__ inline int clamp_len(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Rows a sequence of length L keeps before its S new rows (L + S <= M: all;
// otherwise the min(L, max(0, cap - S)) most recent; cap = M, or W when
// eviction is greedy).
__device__ inline int kept_rows(int L, int S, int M, int cap) {
  if (L + S <= M) return L;
  const int k = cap - S > 0 ? cap - S : 0;
  return L < k ? L : k;
}

}  // namespace gqa
