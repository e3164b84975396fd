// Plain attention over the shared buffer: one wave per (b, h, query i).
// Serves every dtype and head size up to 256 (fp32 and the shapes without a
// fused MFMA kernel). The cache must already hold this call's rows.
//
// Lanes take 64 keys at a time (key j on lane j), each lane forming its full
// dot product; an online softmax keeps (m, l) per wave; then lanes switch to
// head-dimension slices to accumulate p_j v_j. The key loop runs from the
// window start to the query's own position and stops there: nothing past
// the sequence's length is read.
#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

struct SimpleArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  const int32_t* lens;
  const int32_t* offs;   // absolute position of buffer row 0 (nullptr: 0)
  const float* cosv;
  const float* sinv;
  int B, S, H, Hkv, G, D, M, W;
  int cap;             // rows an evicting sequence keeps: min(L, max(0, cap - S))
  int rot, rot_rows, interleaved;
  float scale_log2;
  const void* bias;    // nullptr: none; element (b, h, i, col) at b bs + h hs + i T + col
  int64_t bias_bs, bias_hs;
  int bias_T;
};

constexpr float kLog2e = 1.4426950408889634f;

template <class T>
__global__ void __launch_bounds__(64) attn_simple_kernel(SimpleArgs a) {
  using Bits = typename T::bits;
  __shared__ float qs[256];
  __shared__ float ps[64];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int D = a.D, g = h / a.G;
  const int L = clamp_len(a.lens[b], 0, a.M);
  const int Lp = kept_rows(L, a.S, a.M, a.cap);   // after any eviction
  const int p = Lp + i;
  const int kstart = a.W > 0 ? (p - a.W + 1 > 0 ? p - a.W + 1 : 0) : 0;
  const int kend = p + 1;

  const Bits* qrow = static_cast<const Bits*>(a.q) + ((int64_t(b) * a.S + i) * a.H + h) * D;
  if (a.rot) {
    const int half = D / 2;
    const int pos = clamp_len(L + (a.offs ? a.offs[b] : 0) + i, 0, a.rot_rows - 1);
    for (int j = lane; j < half; j += 64) {
      const int e1 = a.interleaved ? 2 * j : j;
      const int e2 = a.interleaved ? 2 * j + 1 : j + half;
      Bits x = qrow[e1], y = qrow[e2];
      rotate_pair<T>(x, y, a.cosv[int64_t(pos) * half + j], a.sinv[int64_t(pos) * half + j]);
      qs[e1] = T::to_float(x);
      qs[e2] = T::to_float(y);
    }
  } else {
    for (int d = lane; d < D; d += 64) qs[d] = T::to_float(qrow[d]);
  }
  __syncthreads();

  const Bits* bias_row = a.bias ? static_cast<const Bits*>(a.bias) + b * a.bias_bs + h * a.bias_hs +
                                      int64_t(i) * a.bias_T
                                : nullptr;
  const Bits* K = static_cast<const Bits*>(a.k_cache) + (int64_t(b) * a.Hkv + g) * a.M * D;
  const Bits* V = static_cast<const Bits*>(a.v_cache) + (int64_t(b) * a.Hkv + g) * a.M * D;
  float m = -INFINITY, l = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kb = kstart; kb < kend; kb += 64) {
    const int j = kb + lane;
    float s = -INFINITY;
    if (j < kend) {
      const Bits* kr = K + int64_t(j) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], T::to_float(kr[d]), dot);
      s = dot * a.scale_log2;
      if (bias_row)   // the key at row j after an eviction of L - Lp rows is at position j + L - Lp
        s = fmaf(T::to_float(bias_row[j + (L - Lp)]), kLog2e, s);
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = exp2f(m - mn);
    const float pj = (j < kend) ? exp2f(s - mn) : 0.f;
    l = l * alpha + wave_sum(pj);
    m = mn;
    ps[lane] = pj;
    __syncthreads();
    const int n = kend - kb < 64 ? kend - kb : 64;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = lane + 64 * c;
      if (d < D) {
        float acc = o[c] * alpha;
        for (int jj = 0; jj < n; ++jj) acc = fmaf(ps[jj], T::to_float(V[int64_t(kb + jj) * D + d]), acc);
        o[c] = acc;
      }
    }
    __syncthreads();
  }
  Bits* orow = static_cast<Bits*>(a.out) + ((int64_t(b) * a.S + i) * a.H + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int d = lane + 64 * c;
    if (d < D) orow[d] = T::from_float(o[c] * inv);
  }
}

}  // namespace

hipError_t launch_attention_simple(const Problem& p, hipStream_t st) {
  SimpleArgs a;
  a.q = p.q; a.k_cache = p.k_cache; a.v_cache = p.v_cache; a.out = p.out;
  a.lens = p.lens_dev; a.offs = p.off_dev; a.cosv = p.cos; a.sinv = p.sin;
  a.B = p.B; a.S = p.S; a.H = p.H; a.Hkv = p.Hkv; a.G = p.G; a.D = p.D; a.M = p.M;
  a.W = p.window; a.cap = p.cap; a.rot = p.rot; a.rot_rows = p.rot_rows; a.interleaved = p.interleaved;
  a.scale_log2 = p.scale * kLog2e;
  a.bias = p.bias; a.bias_bs = p.bias_bs; a.bias_hs = p.bias_hs; a.bias_T = p.bias_T;
  const dim3 grid(p.S, p.H, p.B);
  if (p.dtype == GQA_FP32) hipLaunchKernelGGL(attn_simple_kernel<F32>, grid, dim3(64), 0, st, a);
  else if (p.dtype == GQA_FP16) hipLaunchKernelGGL(attn_simple_kernel<F16>, grid, dim3(64), 0, st, a);
  else hipLaunchKernelGGL(attn_simple_kernel<BF16>, grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace gqa
