// Window eviction: for every (b, kv head) with L_b + incoming > M, drop the
// oldest d_b = L_b + incoming - M rows (greedy eviction, cap = W < M:
// d_b = L_b - min(L_b, max(0, W - incoming))) and move rows [d_b, L_b) to
// [0, L_b - d_b), in place, for K and V. The buffer must stay where it is, so
// this is a memmove towards lower rows.
//
// Parallel form (d <= kEvictHaloMax): the destination range is cut into
// chunks of C rows. Chunk k reads source rows [kC + d, (k+1)C + d); the last
// d of those are the first d rows chunk k+1 overwrites. A first kernel copies
// those "halo" rows of every chunk to the workspace. In the second kernel one
// thread owns one 16-byte column of one chunk and walks it upwards, row r
// taking the value of row r + d (own rows from the cache, halo rows from the
// workspace): a thread only ever overwrites addresses it has already read
// itself, so no barrier is needed and the loads of the next rows are in
// flight while the current rows are stored. No thread reads a row another
// thread writes in the same kernel.
//
// Serial form (larger d): one workgroup per (b, kv head, K|V) walks the rows
// upwards in blocks; a block's sources lie at or above every row written so
// far, and each block's loads finish (barrier) before its stores.
#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

struct EvictArgs {
  char* k_cache;
  char* v_cache;
  char* halo;          // workspace scratch
  const int32_t* lens;
  int B, Hkv, M, incoming;
  int cap;             // an evicting sequence keeps min(L, max(0, cap - incoming)) rows
  int upr;             // units per row
  int chunk_rows;      // C
  int nchunks;         // ceil(M / C): halo slot stride
};

// (b, kv head, K|V) of this workgroup: y = g * 2 + kv, z = b.
template <class U>
__device__ inline U* cache_rows(const EvictArgs& a, int b, int y) {
  const int g = y >> 1;
  char* base = (y & 1) ? a.v_cache : a.k_cache;
  return reinterpret_cast<U*>(base) + (int64_t(b) * a.Hkv + g) * a.M * int64_t(a.upr);
}

template <class U>
__device__ inline U* halo_rows(const EvictArgs& a, int b, int y, int k) {
  return reinterpret_cast<U*>(a.halo) +
         (((int64_t(b) * a.Hkv * 2 + y) * a.nchunks + k) * kEvictHaloMax) * int64_t(a.upr);
}

__device__ inline int drop_of(const EvictArgs& a, int b, int* Lout) {
  const int L = clamp_len(a.lens[b], 0, a.M);
  *Lout = L;
  return L - kept_rows(L, a.incoming, a.M, a.cap);
}

template <class U>
__global__ void __launch_bounds__(kEvictThreads) halo_kernel(EvictArgs a) {
  const int k = blockIdx.x, y = blockIdx.y, b = blockIdx.z;
  int L;
  const int d = drop_of(a, b, &L);
  if (d == 0 || d > kEvictHaloMax) return;
  const int C = a.chunk_rows, keep = L - d;
  if ((k + 1) * C >= keep) return;  // chunk k + 1 does not exist: nobody overwrites
  const U* src = cache_rows<U>(a, b, y) + int64_t(k + 1) * C * a.upr;
  U* dst = halo_rows<U>(a, b, y, k);
  for (int u = threadIdx.x; u < d * a.upr; u += blockDim.x) dst[u] = src[u];
}

// Column chains: thread (chunk cl of the workgroup, column c) moves rows
// row0 + r <- row0 + r + d for r = 0 .. rows - 1 of column c, kEvictRowsInFlight
// rows at a time, the next group's loads issued before this group's stores
// (they touch disjoint rows: the stores end below row0 + r + P, the next
// loads start at row0 + r + P + d).
template <class U>
__device__ inline U shift_src(const EvictArgs& a, const U* rowsp, const U* halo, int row0, int src,
                              int c, bool next_exists) {
  return (next_exists && src >= row0 + a.chunk_rows)
             ? halo[int64_t(src - row0 - a.chunk_rows) * a.upr + c]
             : rowsp[int64_t(src) * a.upr + c];
}

template <class U>
__global__ void __launch_bounds__(kEvictThreads) shift_kernel(EvictArgs a) {
  constexpr int P = kEvictRowsInFlight;
  const int per_wg = kEvictThreads / a.upr;          // chunks per workgroup
  const int cl = threadIdx.x / a.upr, c = threadIdx.x - cl * a.upr;
  if (cl >= per_wg) return;
  const int k = blockIdx.x * per_wg + cl, y = blockIdx.y, b = blockIdx.z;
  if (k >= a.nchunks) return;
  int L;
  const int d = drop_of(a, b, &L);
  if (d == 0 || d > kEvictHaloMax) return;
  const int C = a.chunk_rows, keep = L - d;
  const int row0 = k * C;
  if (row0 >= keep) return;
  const int rows = (keep - row0) < C ? (keep - row0) : C;
  const bool next_exists = row0 + C < keep;
  U* rowsp = cache_rows<U>(a, b, y);
  const U* halo = halo_rows<U>(a, b, y, k);
  U cur[P], nxt[P];
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < rows) cur[p] = shift_src<U>(a, rowsp, halo, row0, row0 + p + d, c, next_exists);
  for (int r0 = 0; r0 < rows; r0 += P) {
    const bool more = r0 + P < rows;
    if (more) {
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (r0 + P + p < rows)
          nxt[p] = shift_src<U>(a, rowsp, halo, row0, row0 + r0 + P + p + d, c, next_exists);
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (r0 + p < rows) rowsp[int64_t(row0 + r0 + p) * a.upr + c] = cur[p];
#pragma unroll
    for (int p = 0; p < P; ++p) cur[p] = nxt[p];
  }
}

// A copy unit as a built-in vector (or scalar) type of the same size.
template <class U> struct RawOf { using type = U; };
template <> struct RawOf<uint4> {
  typedef uint32_t type __attribute__((ext_vector_type(4)));
};
template <class U> using Raw = typename RawOf<U>::type;

template <class U>
__global__ void __launch_bounds__(kEvictThreads) serial_kernel(EvictArgs a) {
  const int y = blockIdx.x, b = blockIdx.y;
  int L;
  const int d = drop_of(a, b, &L);
  if (d == 0) return;
  const int keep = L - d;
  U* rowsp = cache_rows<U>(a, b, y);
  const int per_block = kEvictThreads * kEvictUnitsPerThread;  // units per pass
  const int64_t total = int64_t(keep) * a.upr;
  const int64_t shift = int64_t(d) * a.upr;
  for (int64_t base = 0; base < total; base += per_block) {
    // every lane loads (past the end it rereads the last unit, which stays
    // in bounds) so the values live in registers; only the stores are guarded
    // (held as plain vector-of-int values: an array of the HIP vector
    // class is kept in scratch memory)
    Raw<U> v[kEvictUnitsPerThread];
#pragma unroll
    for (int n = 0; n < kEvictUnitsPerThread; ++n) {
      const int64_t u = base + threadIdx.x + n * kEvictThreads;
      v[n] = __builtin_bit_cast(Raw<U>, rowsp[(u < total ? u : total - 1) + shift]);
    }
    __syncthreads();  // this pass's sources are all read before any store
#pragma unroll
    for (int n = 0; n < kEvictUnitsPerThread; ++n) {
      const int64_t u = base + threadIdx.x + n * kEvictThreads;
      if (u < total) rowsp[u] = __builtin_bit_cast(U, v[n]);
    }
  }
}

template <class U>
hipError_t run(const EvictArgs& a, int max_drop, hipStream_t st) {
  if (max_drop <= kEvictHaloMax) {
    const int per_wg = kEvictThreads / a.upr;
    const dim3 grid((a.nchunks + per_wg - 1) / per_wg, a.Hkv * 2, a.B);
    if (a.nchunks > 1) {
      hipLaunchKernelGGL(halo_kernel<U>, dim3(a.nchunks - 1, a.Hkv * 2, a.B),
                         dim3(kEvictThreads), 0, st, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(shift_kernel<U>, grid, dim3(kEvictThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(serial_kernel<U>, dim3(a.Hkv * 2, a.B), dim3(kEvictThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_evict(const Problem& p, int incoming, int max_drop, void* ws,
                        const WorkspaceLayout& lay, hipStream_t st) {
  if (p.B == 0 || max_drop <= 0) return hipSuccess;
  const int row_bytes = p.D * (p.dtype == GQA_FP32 ? 4 : 2);
  const EvictGeometry eg = evict_geometry(row_bytes);
  EvictArgs a;
  a.k_cache = static_cast<char*>(p.k_cache);
  a.v_cache = static_cast<char*>(p.v_cache);
  a.halo = static_cast<char*>(ws) + lay.scratch;
  a.lens = p.lens_dev;
  a.B = p.B; a.Hkv = p.Hkv; a.M = p.M; a.incoming = incoming; a.cap = p.cap;
  a.upr = row_bytes / eg.unit;
  a.chunk_rows = eg.chunk_rows;
  a.nchunks = ceil_div(p.M, eg.chunk_rows);
  if (eg.unit == 16) return run<uint4>(a, max_drop, st);
  if (eg.unit == 4) return run<uint32_t>(a, max_drop, st);
  return run<uint16_t>(a, max_drop, st);
}

}  // namespace gqa
