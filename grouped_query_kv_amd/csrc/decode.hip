// Split-KV decode for fp16/bf16 with head_size 128 (one new token per
// sequence).
//
// The key axis of sequence b grows with every step and lives in a buffer of M
// rows ("KV Cache" discussion, notes): only rows [kstart_b, L'_b] are read.
//
// Work layout ("stream-K" at workgroup granularity). A unit is one (sequence
// b, kv head g, group hg of at most 16 of the query heads that share g). Its
// valid keys are cut into 16-key blocks; the blocks of all units, in unit
// order, form one list, and each workgroup of the launch (one per CU, all
// resident) takes an equal contiguous slice of it, so every workgroup
// streams the same number of bytes whatever the mix of lengths. Inside a
// slice the waves of the workgroup take the blocks of each unit segment in
// turn and combine their results in LDS at the segment's end. A unit the
// slice holds whole is written out directly; a unit shared with neighbouring
// slices gets one partial (unnormalised o, m, l) per workgroup, and the last
// workgroup to bump the unit's counter merges them by log-sum-exp, writes
// the output and resets the counter for the next call. Shared segments are
// processed first so those merges happen early, not at the end of the run.
//
// Per block (16 keys, 8 KiB of K and V), both products on MFMA:
//  * K and V rows are loaded fully coalesced (4 whole rows per instruction)
//    while the previous block is computed (two register sets);
//  * K goes through a per-wave LDS tile into the A layout of MFMA 16x16x32:
//    S^T = K Q^T, keys as the 16 rows, the unit's query heads as the 16
//    columns (Q^T stays in registers for the whole unit);
//  * online softmax per head column in registers; the S^T tile is already
//    the B operand P^T of the second product, so P never leaves registers;
//  * V goes through a per-wave LDS tile stored transposed (4 consecutive keys
//    per 8-byte word), giving the A operand V^T of MFMA 16x16x16:
//    O^T += V^T P^T, 8 tiles of 16 head dims.
// The block holding the new token (row L'_b) takes that row from k_new/v_new
// (K rotated under the fp64 rule when rotary is on) instead of the cache and
// writes it into the cache: the append is fused. Rows past a unit's last key
// are clamped to a valid row and their V is zeroed, so p = 0 meets 0.
#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class T> struct Mma;
template <> struct Mma<F16> {
  __device__ static inline f32x4 qk(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 pv(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
};
template <> struct Mma<BF16> {
  __device__ static inline f32x4 qk(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 pv(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
};

constexpr int kD = 128;
constexpr int kKeys = 16;                         // keys per block
constexpr int kKStride = kD + 8;                  // LDS K row stride (halves)
constexpr int kVStride = kKeys + 4;               // LDS V^T row stride (halves, 40 B)
constexpr int kSlotFloats = kDecodeMaxHG * (kD + 2);
constexpr int kThreads = 64 * kDecodeWaves;
constexpr int kMergeMax = 64;                  // partials one merge can weigh in LDS
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* out;
  const float* cosv;
  const float* sinv;
  float* partials;
  int* counters;
  int B, H, Hkv, G, M, W;
  int rot, rot_rows, interleaved;
  int n_hg, hg_size;
  int wgs;                              // workgroups in the launch
  int64_t total;                        // T: blocks over all units
  float scale_log2;
  int32_t hl[kDecodeArgBatch];          // past lengths
  int32_t pb[kDecodeArgBatch + 1];      // first global block of sequence b (all its units)
};

struct Seq {
  int L, Lp, kstart, kend, nb;          // nb: blocks per unit of this sequence
};

__device__ inline Seq seq_of(const DecodeArgs& a, int b) {
  Seq s;
  s.L = clamp_len(a.hl[b], 0, a.M);
  s.Lp = s.L < a.M - 1 ? s.L : a.M - 1;     // row of the new token (after any eviction)
  s.kend = s.Lp + 1;
  s.kstart = a.W > 0 ? (s.kend - a.W > 0 ? s.kend - a.W : 0) : 0;
  s.nb = (s.kend - s.kstart + kKeys - 1) / kKeys;
  return s;
}

// The block a wave is on. The block after `k` is found by incrementing.
struct Blk {
  const uint16_t* kc;      // this unit's K rows
  const uint16_t* vc;
  int kb, kend, Lp;        // first key, unit end, new-token row
  int b, g, ub, i, nb;
};

__device__ inline void set_unit(Blk& k, const DecodeArgs& a) {
  const Seq s = seq_of(a, k.b);
  k.g = k.ub / a.n_hg;
  const int64_t base = (int64_t(k.b) * a.Hkv + k.g) * a.M * kD;
  k.kc = a.k_cache + base;
  k.vc = a.v_cache + base;
  k.kend = s.kend;
  k.Lp = s.Lp;
  k.nb = s.nb;
  k.kb = s.kstart + kKeys * k.i;
}

__device__ inline Blk locate(const DecodeArgs& a, int64_t x) {
  Blk k;
  k.b = 0;
  for (int b = 0; b < a.B; ++b)
    if (x >= a.pb[b] && x < a.pb[b + 1]) k.b = b;
  const int nb = seq_of(a, k.b).nb;
  const int off = int(x - a.pb[k.b]);
  k.ub = off / nb;
  k.i = off - k.ub * nb;
  set_unit(k, a);
  return k;
}

__device__ inline Blk next_block(const DecodeArgs& a, const Blk& c) {
  Blk k = c;
  if (++k.i < k.nb) {
    k.kb += kKeys;
    return k;
  }
  k.i = 0;
  if (++k.ub == a.Hkv * a.n_hg) {
    k.ub = 0;
    ++k.b;
  }
  set_unit(k, a);
  return k;
}

// Rotate a query row held as 4 16-byte chunks, chunk i = dims 32 i + 8 q4 + e:
// rotate-half pairs (d, d + 64) are chunks (i, i + 2) of the same lane,
// interleaved pairs are neighbours inside a chunk.
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

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// One block's K and V rows, lane (n, q4) holding dims 8 n .. 8 n + 7 of keys
// 4 q4 + j (j = 0..3): every load instruction reads 4 whole rows. Named
// members, passed by value: an indexed array here would end up in memory.
struct Regs {
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
};

__device__ inline uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ inline Regs load_regs(const DecodeArgs& a, const Blk& k, int n, int q4) {
  const int key0 = k.kb + 4 * q4;
  const int row0 = key0 < k.kend ? key0 : k.kb;
  const int row1 = key0 + 1 < k.kend ? key0 + 1 : k.kb;
  const int row2 = key0 + 2 < k.kend ? key0 + 2 : k.kb;
  const int row3 = key0 + 3 < k.kend ? key0 + 3 : k.kb;
  const uint16_t* kc = k.kc + 8 * n;
  const uint16_t* vc = k.vc + 8 * n;
  Regs r;
  r.k0 = ld16(kc + row0 * kD);
  r.k1 = ld16(kc + row1 * kD);
  r.k2 = ld16(kc + row2 * kD);
  r.k3 = ld16(kc + row3 * kD);
  r.v0 = ld16(vc + row0 * kD);
  r.v1 = ld16(vc + row1 * kD);
  r.v2 = ld16(vc + row2 * kD);
  r.v3 = ld16(vc + row3 * kD);
  return r;
}

// 16-bit element e of a 16-byte register group
__device__ inline uint32_t h16(const uint4& u, int e) {
  const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

struct Acc {
  float m, l;          // running max (per head column) and this lane's partial sum
  f32x4 o[8];          // O^T[16 dt + 4 q4 + r][head n]
};

__device__ inline void acc_reset(Acc& s) {
  s.m = -INFINITY;
  s.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) s.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <class T>
__device__ inline uint32_t pack2(float x, float y) {
  return uint32_t(T::from_float(x)) | (uint32_t(T::from_float(y)) << 16);
}

template <class T>
__device__ inline void compute(Acc& s, Regs r, const uint4 (&qv)[4], const Blk& k,
                               const DecodeArgs& a, int lane, uint16_t* klds, uint16_t* vlds) {
  using Bits = typename T::bits;
  const int n = lane & 15, q4 = lane >> 4;
  // ---- K rows into the LDS tile (row-major), V rows transposed ----
  if (k.kb + kKeys > k.kend) {
    // last block of the unit: rows past its end are clamped copies of row kb,
    // which may be the unwritten new-token row; zero their V so that p = 0
    // meets 0, not NaN, in the product
    const int key0 = k.kb + 4 * q4;
    const uint4 z = make_uint4(0, 0, 0, 0);
    if (key0 >= k.kend) r.v0 = z;
    if (key0 + 1 >= k.kend) r.v1 = z;
    if (key0 + 2 >= k.kend) r.v2 = z;
    if (key0 + 3 >= k.kend) r.v3 = z;
  }
  {
    uint16_t* kt = klds + 4 * q4 * kKStride + 8 * n;
    *reinterpret_cast<uint4*>(kt) = r.k0;
    *reinterpret_cast<uint4*>(kt + kKStride) = r.k1;
    *reinterpret_cast<uint4*>(kt + 2 * kKStride) = r.k2;
    *reinterpret_cast<uint4*>(kt + 3 * kKStride) = r.k3;
    uint16_t* vt = vlds + 8 * n * kVStride + 4 * q4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 w;
      w.x = h16(r.v0, e) | (h16(r.v1, e) << 16);
      w.y = h16(r.v2, e) | (h16(r.v3, e) << 16);
      *reinterpret_cast<uint2*>(vt + e * kVStride) = w;
    }
  }
  if (k.Lp >= k.kb && k.Lp < k.kb + kKeys) {
    // The new token: its K row (rotated from k_new) and V row (from v_new)
    // replace the tile rows and go into the cache. Every head group of the
    // kv head writes the same bytes.
    const int t = k.Lp - k.kb;
    const int64_t kvrow = (int64_t(k.b) * a.Hkv + k.g) * kD;
    const Bits* knew = reinterpret_cast<const Bits*>(a.k_new) + kvrow;
    const Bits* vnew = reinterpret_cast<const Bits*>(a.v_new) + kvrow;
    const int64_t crow = ((int64_t(k.b) * a.Hkv + k.g) * a.M + k.Lp) * kD;
    const int e1 = a.interleaved ? 2 * lane : lane;
    const int e2 = a.interleaved ? 2 * lane + 1 : lane + kD / 2;
    Bits x = knew[e1], y = knew[e2];
    if (a.rot) {
      const int pos = clamp_len(clamp_len(a.hl[k.b], 0, a.M), 0, a.rot_rows - 1);
      rotate_pair<T>(x, y, a.cosv[int64_t(pos) * (kD / 2) + lane],
                     a.sinv[int64_t(pos) * (kD / 2) + lane]);
    }
    Bits* trow = reinterpret_cast<Bits*>(klds + t * kKStride);
    trow[e1] = x;
    trow[e2] = y;
    reinterpret_cast<Bits*>(a.k_cache)[crow + e1] = x;
    reinterpret_cast<Bits*>(a.k_cache)[crow + e2] = y;
    const Bits v1 = vnew[lane], v2 = vnew[lane + 64];
    reinterpret_cast<Bits*>(vlds)[lane * kVStride + t] = v1;
    reinterpret_cast<Bits*>(vlds)[(lane + 64) * kVStride + t] = v2;
    reinterpret_cast<Bits*>(a.v_cache)[crow + lane] = v1;
    reinterpret_cast<Bits*>(a.v_cache)[crow + lane + 64] = v2;
  }
  wave_lds_sync();
  // ---- S^T = K Q^T: lane gets keys 4 q4 + r of head column n ----
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = Mma<T>::qk(*reinterpret_cast<const uint4*>(klds + n * kKStride + 32 * i + 8 * q4),
                     qv[i], acc);
  float sv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
    sv[rr] = k.kb + 4 * q4 + rr < k.kend ? acc[rr] * a.scale_log2 : -INFINITY;
  float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  if (__any(bm > s.m)) {               // rescale only when some head's max grows
    const float mn = fmaxf(s.m, bm);
    const float alpha = exp2f(s.m - mn);
    s.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) s.o[dt] *= alpha;
    s.m = mn;
  }
  float p[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    p[rr] = exp2f(sv[rr] - s.m);
    s.l += p[rr];
  }
  uint2 pb;                            // P^T: keys 4 q4 .. 4 q4 + 3 of head n
  pb.x = pack2<T>(p[0], p[1]);
  pb.y = pack2<T>(p[2], p[3]);
  // ---- O^T += V^T P^T: A = V^T rows 16 dt + n, keys 4 q4 .. 4 q4 + 3 ----
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    s.o[dt] = Mma<T>::pv(*reinterpret_cast<const uint2*>(vlds + (16 * dt + n) * kVStride + 4 * q4),
                         pb, s.o[dt]);
  wave_lds_sync();   // the next block rewrites the tiles
}

// Q^T of one unit as the MFMA B operand: lane (n, q4) holds head n's dims
// 32 i + 8 q4 .. (zeros for padding heads), rotated at position L_b.
template <class T>
__device__ inline void load_q(uint4 (&qv)[4], const DecodeArgs& a, const Blk& k, int lane) {
  const int n = lane & 15, q4 = lane >> 4;
  const int hg = k.ub % a.n_hg;
  const int h0 = k.g * a.G + hg * a.hg_size;
  const int nheads = min(a.hg_size, a.G - hg * a.hg_size);
  const uint16_t* qrow = a.q + (int64_t(k.b) * a.H + h0 + n) * kD + 8 * q4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    qv[i] = n < nheads ? ld16(qrow + 32 * i) : make_uint4(0, 0, 0, 0);
  if (a.rot && n < nheads) {
    const int pos = clamp_len(clamp_len(a.hl[k.b], 0, a.M), 0, a.rot_rows - 1);
    rotate_row_chunks<T>(qv, q4, a.cosv + int64_t(pos) * (kD / 2),
                         a.sinv + int64_t(pos) * (kD / 2), a.interleaved);
  }
}

// The workgroup that owns global block x (slices [w T / N, (w + 1) T / N)).
__device__ inline int owner_wg(const DecodeArgs& a, int64_t x) {
  return int(((x + 1) * a.wgs - 1) / a.total);
}

// Unit index and the workgroups sharing it.
struct UnitInfo {
  int unit, h0, nheads, wg_first, wg_last;
};

__device__ inline UnitInfo unit_info(const DecodeArgs& a, int b, int ub) {
  UnitInfo u;
  const int g = ub / a.n_hg, hg = ub % a.n_hg;
  u.h0 = g * a.G + hg * a.hg_size;
  u.nheads = min(a.hg_size, a.G - hg * a.hg_size);
  u.unit = b * a.Hkv * a.n_hg + ub;
  const int nb = seq_of(a, b).nb;
  const int64_t x0 = a.pb[b] + int64_t(ub) * nb;
  u.wg_first = owner_wg(a, x0);
  u.wg_last = owner_wg(a, x0 + nb - 1);
  return u;
}

template <class T>
__device__ inline void store_out(const DecodeArgs& a, int b, int h, int d, float v) {
  reinterpret_cast<typename T::bits*>(a.out)[(int64_t(b) * a.H + h) * kD + d] = T::from_float(v);
}

// Merge the partials of a shared unit (one per workgroup wg_first..wg_last),
// write the output and reset the counter. All threads load at once.
template <class T>
__device__ inline void merge_unit(const DecodeArgs& a, int b, int ub, float* lds) {
  const int tid = threadIdx.x;
  const UnitInfo u = unit_info(a, b, ub);
  const int count = u.wg_last - u.wg_first + 1;
  auto ld = [](const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  const float* base = a.partials + int64_t(u.wg_first + u.unit) * kSlotFloats;
  float* wm = lds;                                   // [count][16] -> weights
  float* wl = lds + kMergeMax * 16;                  // [count][16]
  for (int idx = tid; idx < count * 16; idx += kThreads) {
    const int j = idx >> 4, h = idx & 15;
    const float* sl = base + int64_t(j) * kSlotFloats;
    wm[idx] = h < u.nheads ? ld(sl + kDecodeMaxHG * kD + h) : 0.f;
    wl[idx] = h < u.nheads ? ld(sl + kDecodeMaxHG * kD + kDecodeMaxHG + h) : 0.f;
  }
  __syncthreads();
  if (tid < u.nheads) {
    float M = -INFINITY;
    for (int j = 0; j < count; ++j) M = fmaxf(M, wm[j * 16 + tid]);
    float L = 0.f;
    for (int j = 0; j < count; ++j) {
      const float e = exp2f(wm[j * 16 + tid] - M);
      wm[j * 16 + tid] = e;
      L = fmaf(wl[j * 16 + tid], e, L);
    }
    const float inv = 1.f / L;
    for (int j = 0; j < count; ++j) wm[j * 16 + tid] *= inv;
  }
  __syncthreads();
  for (int idx = tid; idx < u.nheads * kD; idx += kThreads) {
    const int h = idx / kD, d = idx % kD;
    float acc = 0.f;
    for (int j0 = 0; j0 < count; j0 += 8) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x[j] = j0 + j < count ? ld(base + int64_t(j0 + j) * kSlotFloats + h * kD + d) : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j0 + j < count) acc = fmaf(x[j], wm[(j0 + j) * 16 + h], acc);
    }
    store_out<T>(a, b, u.h0 + h, d, acc);
  }
  __syncthreads();
  if (tid == 0) __hip_atomic_store(a.counters + u.unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A segment: the blocks [start, end) of one unit inside a workgroup's slice.
struct Seg {
  Blk first;                 // block `start`
  int64_t start, end;
  bool shared;               // the unit has blocks outside the slice
};

// Block `off` blocks after `k` within the same unit.
__device__ inline Blk advance_in_unit(Blk k, int off) {
  k.i += off;
  k.kb += kKeys * off;
  return k;
}

// Segments of slice [S, E), in processing order: the shared ones first (the
// unit running past the slice end, then the one starting before it), so
// every shared unit is complete early and its merge overlaps the streaming
// of the units the slice owns whole, which follow in order.
struct SegPlan {
  int64_t S, E;
  Blk fb, lb;                // first block of the slice, first block of the last segment
  int64_t f_end, l_start;
  bool single, first_shared, last_shared;
  int64_t own_s, own_e;      // owned range (whole units)
};

__device__ inline SegPlan make_plan(const DecodeArgs& a, int64_t S, int64_t E) {
  SegPlan p;
  p.S = S; p.E = E;
  p.fb = locate(a, S);
  const int64_t f_unit_end = S - p.fb.i + p.fb.nb;
  p.f_end = f_unit_end < E ? f_unit_end : E;
  p.single = p.f_end == E;
  p.first_shared = p.fb.i > 0 || f_unit_end > E;
  const Blk eb = locate(a, E - 1);
  p.l_start = (E - 1) - eb.i;
  if (p.l_start < S) p.l_start = S;
  p.lb = advance_in_unit(eb, -int((E - 1) - p.l_start));
  p.last_shared = !p.single && ((E - 1) - eb.i + eb.nb > E);
  p.own_s = p.first_shared ? p.f_end : S;
  p.own_e = (p.last_shared && !p.single) ? p.l_start : E;
  if (p.own_e < p.own_s) p.own_e = p.own_s;
  return p;
}

// One segment: this wave's blocks seg.start + wv, + 4, ... with two register
// sets in turn, then the 4 waves combine in LDS and either write the output
// (owned unit) or the workgroup's partial (shared unit).
template <class T>
__device__ inline void run_segment(const DecodeArgs& a, const Seg& sg, uint16_t* ktile,
                                   uint16_t* vtile, float* comb, int wg) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const int nseg = int(sg.end - sg.start);
  Acc s;
  acc_reset(s);
  if (wv < nseg) {
    Blk cur = advance_in_unit(sg.first, wv);
    Regs rc = load_regs(a, cur, n, q4);
    uint4 qv[4];
    load_q<T>(qv, a, sg.first, lane);
    for (int j = wv;;) {
      const int jn = j + kDecodeWaves;
      Blk nb = jn < nseg ? advance_in_unit(cur, kDecodeWaves) : cur;
      Regs rn = load_regs(a, nb, n, q4);
      compute<T>(s, rc, qv, cur, a, lane, ktile, vtile);
      if (jn >= nseg) break;
      cur = nb;
      j = jn;
      const int jn2 = j + kDecodeWaves;
      nb = jn2 < nseg ? advance_in_unit(cur, kDecodeWaves) : cur;
      rc = load_regs(a, nb, n, q4);
      compute<T>(s, rn, qv, cur, a, lane, ktile, vtile);
      if (jn2 >= nseg) break;
      cur = nb;
      j = jn2;
    }
  }
  // ---- combine the 4 waves in LDS: per wave m[16], l[16], o[16][128] ----
  float l = s.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  __syncthreads();                                  // tiles are free now
  const UnitInfo u = unit_info(a, sg.first.b, sg.first.ub);
  float* cw = comb + wv * (32 + 16 * kD);
  if (q4 == 0) { cw[n] = s.m; cw[16 + n] = l; }
  if (n < u.nheads) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(cw + 32 + n * kD + 16 * dt + 4 * q4) = s.o[dt];
  }
  __syncthreads();
  float* slot = a.partials + int64_t(wg + u.unit) * kSlotFloats;
  for (int idx = tid; idx < u.nheads * kD; idx += kThreads) {
    const int h = idx / kD, d = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w)
      if (w < nseg) M = fmaxf(M, comb[w * (32 + 16 * kD) + h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      if (w >= nseg) continue;                      // waves with no block in the segment
      const float* c = comb + w * (32 + 16 * kD);
      const float wgt = exp2f(c[h] - M);
      L = fmaf(c[16 + h], wgt, L);
      O = fmaf(c[32 + h * kD + d], wgt, O);
    }
    if (!sg.shared) {
      store_out<T>(a, sg.first.b, u.h0 + h, d, O / L);
    } else {
      __hip_atomic_store(slot + h * kD + d, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(slot + kDecodeMaxHG * kD + h, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + kDecodeMaxHG * kD + kDecodeMaxHG + h, L, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __syncthreads();                                  // the combine area is read
}

template <class T>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecodeArgs a) {
  // per-wave K and V^T tiles in one allocation, reused as the combine /
  // merge area between segments
  constexpr int kTileHalves = kKeys * kKStride + kD * kVStride;
  static_assert(kDecodeWaves * kTileHalves * 2 >= kDecodeWaves * (32 + 16 * kD) * 4, "combine area");
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kDecodeWaves * kTileHalves];
  __shared__ int sh_flag[2];
  float* comb = reinterpret_cast<float*>(tiles);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const int wg = blockIdx.x;
  const int64_t S = (int64_t(wg) * a.total) / a.wgs;
  const int64_t E = (int64_t(wg + 1) * a.total) / a.wgs;
  if (S >= E) return;
  uint16_t* ktile = tiles + wv * kTileHalves;
  uint16_t* vtile = ktile + kKeys * kKStride;
  const SegPlan plan = make_plan(a, S, E);

  // ---- phase A: the shared segments (unit past the slice end, then the
  // unit begun before it), so that the merges they feed happen early ----
  const bool do_last = plan.last_shared && !plan.single;
  Seg shs[2];
  int nsh = 0;
  if (do_last) { shs[0].first = plan.lb; shs[0].start = plan.l_start; shs[0].end = E; shs[0].shared = true; nsh = 1; }
  if (plan.first_shared) {
    Seg& f = nsh ? shs[1] : shs[0];
    f.first = plan.fb; f.start = S; f.end = plan.f_end; f.shared = true;
    ++nsh;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (k >= nsh) break;
    run_segment<T>(a, shs[k], ktile, vtile, comb, wg);
  }
  if (nsh) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // partial stores have landed
    __syncthreads();
    if (tid < nsh) {
      const Seg& sg = tid ? shs[1] : shs[0];
      const UnitInfo u = unit_info(a, sg.first.b, sg.first.ub);
      const int prev = __hip_atomic_fetch_add(a.counters + u.unit, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      sh_flag[tid] = prev == u.wg_last - u.wg_first;
    }
    __syncthreads();
    if (sh_flag[0]) merge_unit<T>(a, shs[0].first.b, shs[0].first.ub, comb);
    if (nsh > 1 && sh_flag[1]) merge_unit<T>(a, shs[1].first.b, shs[1].first.ub, comb);
  }

  // ---- phase B: the units the slice owns whole, in order ----
  if (plan.own_s >= plan.own_e) return;
  Seg cur;
  cur.first = plan.first_shared ? locate(a, plan.own_s) : plan.fb;
  cur.start = plan.own_s;
  cur.shared = false;
  for (;;) {
    const int64_t ue = cur.start - cur.first.i + cur.first.nb;
    cur.end = ue < plan.own_e ? ue : plan.own_e;
    run_segment<T>(a, cur, ktile, vtile, comb, wg);
    if (cur.end >= plan.own_e) break;
    cur.first = next_block(a, advance_in_unit(cur.first, int(cur.end - 1 - cur.start)));
    cur.start = cur.end;
  }
}

}  // namespace

bool decode_fast_supported(const Problem& p) {
  return p.D == 128 && (p.dtype == GQA_FP16 || p.dtype == GQA_BF16) && p.S == 1 &&
         p.B <= kDecodeArgBatch;
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
  a.cosv = p.cos; a.sinv = p.sin;
  a.rot = p.rot; a.rot_rows = p.rot_rows; a.interleaved = p.interleaved;
  a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.scratch);
  a.counters = reinterpret_cast<int*>(static_cast<char*>(ws) + lay.counters);
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.G = p.G; a.M = p.M; a.W = p.window;
  a.n_hg = ceil_div(p.G, kDecodeMaxHG);
  a.hg_size = ceil_div(p.G, a.n_hg);
  a.scale_log2 = p.scale * kLog2e;
  const int units_per_seq = p.Hkv * a.n_hg;
  int64_t total = 0;
  for (int b = 0; b < p.B; ++b) {
    const int L = p.lens_host[b] < p.M - 1 ? p.lens_host[b] : p.M - 1;
    const int kend = L + 1;
    const int kstart = p.window > 0 ? (kend - p.window > 0 ? kend - p.window : 0) : 0;
    a.hl[b] = p.lens_host[b];
    a.pb[b] = int32_t(total);
    total += int64_t((kend - kstart + kKeys - 1) / kKeys) * units_per_seq;
  }
  a.pb[p.B] = int32_t(total);
  a.total = total;
  if (total == 0) return hipSuccess;
  // workgroups: all resident at once, and no unit shared by more than
  // kMergeMax of them
  int64_t wgs = kDecodeMaxWorkgroups < total ? kDecodeMaxWorkgroups : total;
  int64_t max_unit = 0;
  for (int b = 0; b < p.B; ++b) {
    const int64_t nb = p.B ? (a.pb[b + 1] - a.pb[b]) / units_per_seq : 0;
    max_unit = nb > max_unit ? nb : max_unit;
  }
  while (wgs > 1 && max_unit * wgs > int64_t(kMergeMax - 1) * total) wgs /= 2;
  a.wgs = int(wgs);
  const int blocks = a.wgs;
  if (p.dtype == GQA_FP16)
    hipLaunchKernelGGL(decode_kernel<F16>, dim3(blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(decode_kernel<BF16>, dim3(blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace gqa
