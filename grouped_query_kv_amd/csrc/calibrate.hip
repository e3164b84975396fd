// A plain streaming read, the yardstick for the memory-bound kernels.
//
// It reads a device buffer once and does nothing with the data but fold it
// into a per-lane value that is stored only under a condition no ordinary
// input meets (which keeps the loads). Launch shape as in the split-KV
// decode: one workgroup of eight waves per CU, every wave a contiguous slice,
// 16 bytes per lane and four loads in flight per lane. Its time for a given
// byte count, on buffers that are not cache-resident, is what any kernel that
// must read those bytes once can reach on this GPU.
#include "gqa_internal.h"

namespace gqa {

// external linkage: stores to it cannot be proven dead, so the loads stay
__device__ unsigned int g_read_sink[64];

namespace {

constexpr int kReadWaves = 8;
constexpr int kReadWorkgroups = 256;

__global__ void __launch_bounds__(64 * kReadWaves) stream_read_kernel(const uint4* __restrict__ p,
                                                                        size_t n16) {
  const int lane = threadIdx.x & 63;
  const size_t waves = size_t(gridDim.x) * kReadWaves;
  const size_t w = size_t(blockIdx.x) * kReadWaves + (threadIdx.x >> 6);
  const size_t per = (n16 + waves - 1) / waves;
  const size_t s = w * per;
  const size_t e = s + per < n16 ? s + per : n16;
  unsigned int acc = 0;
  for (size_t i = s + lane; i < e; i += 4 * 64) {
    const uint4 a = p[i];
    const uint4 b = i + 64 < e ? p[i + 64] : make_uint4(0, 0, 0, 0);
    const uint4 c = i + 128 < e ? p[i + 128] : make_uint4(0, 0, 0, 0);
    const uint4 d = i + 192 < e ? p[i + 192] : make_uint4(0, 0, 0, 0);
    acc ^= (a.x + b.x + c.x + d.x) ^ (a.y + b.y + c.y + d.y) ^ (a.z + b.z + c.z + d.z) ^
           (a.w + b.w + c.w + d.w);
  }
  if (acc == 0x9E3779B9u) g_read_sink[lane] = acc;   // a per-lane (vector) store
}

}  // namespace
}  // namespace gqa

using namespace gqa;

extern "C" gqa_status gqa_stream_read(const void* src, size_t bytes, void* stream) {
  if (!src || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return set_error(GQA_ERR_INVALID_ARG,
                     "gqa_stream_read: src must be non-null and 16-byte aligned, bytes a positive "
                     "multiple of 16");
  set_error(GQA_OK, "%s", "");
  hipLaunchKernelGGL(stream_read_kernel, dim3(kReadWorkgroups), dim3(64 * kReadWaves), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     bytes / 16);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(GQA_ERR_HIP, "gqa_stream_read: %s", hipGetErrorString(e));
  return GQA_OK;
}
