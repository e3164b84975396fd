// The static device scratch behind gqa_attention_decode_noalloc, for callers
// that cannot allocate: the same op and kernels as gqa_attention_decode,
// with the workspace replaced by a static device array (`scratch`,
// GQA_NOALLOC_SCRATCH_BYTES per GPU) that the code object carries. Nothing
// here calls hipMalloc, hipFree or any allocating routine.
//
// In host code `scratch` names a host-side stand-in, not device memory:
// every host use of the array goes through the device address that
// hipGetSymbolAddress returns, fetched once per device on that device's
// first call (with the device current) and kept in a table; each GPU holds
// its own copy of the array at its own address.
#include <mutex>

#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kMaxDevices = 64;

// 256-byte aligned like a workspace allocation; its first kStaticCounterArea
// bytes are the merge counters, which must start at zero.
static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

struct DeviceEntry {
  void* ptr = nullptr;       // device address of `scratch` on this device
  bool clear = true;         // the counter area must be zeroed before the next call
};

std::mutex g_mu;
DeviceEntry g_dev[kMaxDevices];

__global__ void __launch_bounds__(256) zero_kernel(uint4* p, size_t n) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st,
                     static_cast<uint4*>(p), n);
  return hipGetLastError();
}

gqa_status static_scratch_begin(StaticScratch* sc) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(GQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(GQA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                     kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceEntry& d = g_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(GQA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                       hipGetErrorString(e));
    d.ptr = p;
    d.clear = true;
  }
  sc->device = dev;
  sc->ptr = d.ptr;
  sc->clear = d.clear;
  return GQA_OK;
}

void static_scratch_end(const StaticScratch& sc, gqa_status st) {
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceEntry& d = g_dev[sc.device];
  if (st == GQA_ERR_HIP) d.clear = true;          // counters may have been left set
  else if (sc.clear && st == GQA_OK) d.clear = false;
}

}  // namespace gqa
