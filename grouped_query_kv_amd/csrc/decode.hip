// Split-KV decode for fp16/bf16 with head_size 128 (one new token per
// sequence).
//
// The key axis of sequence b grows with every step and lives in a buffer of M
// rows ("KV Cache" discussion, notes): only rows [kstart_b, L'_b] are read.
//
// Work layout ("stream-K" at wave granularity). A unit is one (sequence b,
// kv head g, group hg of at most 16 of the query heads that share g). Its
// valid keys are cut into 16-key blocks; the blocks of all units, in unit
// order, form one list, and every wave of the launch (a "worker") takes an
// equal contiguous slice of it and streams it alone, two blocks in flight,
// with no barrier until its slice is done. So every wave moves the same
// number of bytes whatever the mix of lengths. A unit a wave holds whole is
// written out by that wave. A unit cut by a slice boundary leaves one partial
// (unnormalised o, m, l) per wave in the workgroup's LDS; at the end the
// workgroup combines the partials of each such unit, writes the output if the
// unit lies inside the workgroup, and otherwise stores one partial per
// workgroup; the last workgroup to finish a unit merges those by log-sum-exp
// and resets the unit's counter for the next call.
//
// Per block (16 keys, 8 KiB of K and V), both products on MFMA:
//  * K rows are loaded straight into the A layout of MFMA 16x16x32: lane
//    (n, q4) holds key n, dims 32 i + 8 q4 .. + 7 (i = 0..3); S^T = K Q^T with
//    the unit's query heads as the 16 columns (Q^T stays in registers);
//  * online softmax per head column in registers; the S^T tile is already
//    the B operand P^T of the second product;
//  * V rows go to a per-wave LDS tile as they were loaded (row-major, chunks
//    XOR-swizzled), and transposing LDS reads (ds_read_b64_tr_b16) hand out
//    the A operand V^T of MFMA 16x16x16: O^T += V^T P^T, 8 tiles of 16 dims.
// The block holding the new token (row L'_b) takes that row from k_new/v_new
// (K rotated under the fp64 rule when rotary is on) instead of the cache and
// writes it into the cache: the append is fused. Rows past the unit's last
// key are clamped to a valid row; their scores are masked and their V is
// zeroed, so p = 0 meets 0.
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

// Head sizes 128 and 64 (template parameter D). Partial slots and the V
// tile are laid out for the larger one: a head of D = 64 uses the first
// half of each 128-float head row of a slot and of each 256-byte tile row.
constexpr int kD = 128;                           // slot and tile row capacity
constexpr int kKeys = 16;                         // keys per block
constexpr int kVTileBytes = kKeys * kD * 2;       // per-wave V tile, 16 rows x 256 B
constexpr int kSlotFloats = kDecodeMaxHG * (kD + 2);
constexpr int kThreads = 64 * kDecodeWaves;
constexpr int kMergeMax = 64;                  // partials one merge can weigh in LDS
constexpr int kSlotBytes = kSlotFloats * 4;
// per wave in LDS: partial slot 0, then an area holding the V tile while
// streaming and partial slot 1 at the end
constexpr int kWaveLds = 2 * kSlotBytes;
static_assert(kVTileBytes <= kSlotBytes, "the V tile lives in partial slot 1 while streaming");
constexpr float kRescaleSlack = 8.f;           // binary orders the reference max may lag
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
  uint16_t* halo_k;                     // fused eviction: one row per worker, [workers, D]: the
  uint16_t* halo_v;                     //   source row after its slice that the next slice overwrites
  int shift;                            // fused eviction on: full sequences drop their oldest row
  const uint16_t* past_k;               // fused past copy: the rows [0, L_b) are read from these
  const uint16_t* past_v;               //   buffers (past_rows rows per (b, kv head)) and written
  int past_rows;                        //   to k_cache/v_cache at the same row (past_k != nullptr)
  int B, H, Hkv, G, M, W;
  int cap;                              // rows an evicting sequence keeps: M - 1, or W - 1 (greedy)
  int rot, rot_rows, interleaved;
  int n_hg, hg_size;
  int workers;                          // waves in the launch that take a slice
  int64_t total;                        // T: blocks over all units
  int fits32;                           // (T + 1) * workers < 2^32: slice bounds in 32 bits
  float scale_log2;
  const uint16_t* bias;                 // additive bias (b, h, column) at b bias_bs + h bias_hs + column
  int64_t bias_bs, bias_hs;
  int32_t hl[kDecodeArgBatch];          // past lengths
  int32_t ro[kDecodeArgBatch];          // absolute position of buffer row 0 (rotary only)
  int32_t pb[kDecodeArgBatch + 1];      // first global block of sequence b (all its units)
};

struct Seq {
  int L, Lp, kstart, kend, nb;          // nb: blocks per unit of this sequence
  int d;                                // rows dropped by the fused eviction (0 or 1)
};

// The per-sequence plan values in registers: lane j holds sequence j's past
// length and first global block (B <= 64, one lane each), loaded once per
// wave with two vector loads; an entry is then one scalar lane read.
// Reading the argument block at a runtime index instead costs a memory
// round trip each time (about 0.8 us), at the start of a wave's slice, at
// every unit it enters and in the end phase.
struct SeqRegs {
  int hl, pb, pb1;          // L_j, pb[j], pb[j + 1]
};

__device__ inline SeqRegs load_seq_regs(const DecodeArgs& a, int lane) {
  const int j = lane < a.B ? lane : 0;          // every lane reads in bounds (B >= 1)
  SeqRegs r;
  r.hl = a.hl[j];
  r.pb = a.pb[j];
  r.pb1 = a.pb[j + 1];                          // pb holds B + 1 entries
  return r;
}

__device__ inline int lane_of(int v, int b) { return __builtin_amdgcn_readlane(v, b); }

__device__ inline Seq seq_of(const DecodeArgs& a, int b, const SeqRegs& sr) {
  Seq s;
  s.L = clamp_len(lane_of(sr.hl, b), 0, a.M);
  s.Lp = kept_rows(s.L, 1, a.M, a.cap);     // row of the new token (after any eviction)
  s.kend = s.Lp + 1;
  s.kstart = a.W > 0 ? (s.kend - a.W > 0 ? s.kend - a.W : 0) : 0;
  s.nb = (s.kend - s.kstart + kKeys - 1) / kKeys;
  s.d = a.shift && s.L >= a.M ? 1 : 0;
  return s;
}

// The block a wave is on. The block after `k` is found by incrementing.
struct Blk {
  const uint16_t* kc;      // this unit's K rows
  const uint16_t* vc;
  int kb, kend, Lp;        // first key, unit end, new-token row
  int b, g, ub, i, nb;
  int d;                   // fused eviction: key r is read from buffer row r + d
  int coff;                // bias column of key r: r + coff (its position before any eviction)
  int L;                   // past length (with the sequence's position offset: the rotary position)
};

template <int D>
__device__ inline void set_unit(Blk& k, const DecodeArgs& a, const SeqRegs& sr) {
  const Seq s = seq_of(a, k.b, sr);
  k.g = k.ub / a.n_hg;
  const int64_t base = (int64_t(k.b) * a.Hkv + k.g) * a.M * D;
  k.kc = a.k_cache + base;
  k.vc = a.v_cache + base;
  k.kend = s.kend;
  k.Lp = s.Lp;
  k.nb = s.nb;
  k.kb = s.kstart + kKeys * k.i;
  k.d = s.d;
  k.coff = s.L - s.Lp;
  k.L = s.L;
}

template <int D>
__device__ inline Blk locate(const DecodeArgs& a, int64_t x, const SeqRegs& sr, int lane) {
  Blk k;
  // the lane whose sequence holds block x (none past the end: sequence 0)
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < a.B && x >= sr.pb && x < sr.pb1);
  k.b = hit ? int(__builtin_ctzll(hit)) : 0;
  const int nb = seq_of(a, k.b, sr).nb;
  const int off = int(x - lane_of(sr.pb, k.b));
  // callers pass x < total; the clamps keep every derived address inside the
  // caches even if one did not
  const int units = a.Hkv * a.n_hg;
  k.ub = nb > 0 ? off / nb : 0;
  k.ub = k.ub < units ? (k.ub > 0 ? k.ub : 0) : units - 1;
  k.i = off - k.ub * nb;
  k.i = k.i < nb ? (k.i > 0 ? k.i : 0) : (nb > 0 ? nb - 1 : 0);
  set_unit<D>(k, a, sr);
  return k;
}

template <int D>
__device__ inline Blk next_block(const DecodeArgs& a, const Blk& c, const SeqRegs& sr) {
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
  set_unit<D>(k, a, sr);
  return k;
}

// Rotation of one lane's four 16-byte chunks of a row (chunk i = dims
// 32 i + 8 q4 .. + 7), on named values so that no array is formed:
// rotate-half pairs (d, d + 64) are chunks (0, 2) and (1, 3), element by
// element; interleaved pairs are neighbours inside a chunk.
template <class T>
__device__ inline void rot_word_pair(uint32_t& x, uint32_t& y, int j, const float* cosr,
                                     const float* sinr) {
  using Bits = typename T::bits;
  Bits x0 = Bits(x & 0xFFFFu), x1 = Bits(x >> 16), y0 = Bits(y & 0xFFFFu), y1 = Bits(y >> 16);
  rotate_pair<T>(x0, y0, cosr[j], sinr[j]);
  rotate_pair<T>(x1, y1, cosr[j + 1], sinr[j + 1]);
  x = uint32_t(x0) | (uint32_t(x1) << 16);
  y = uint32_t(y0) | (uint32_t(y1) << 16);
}

template <class T>
__device__ inline void rot_half_chunks(uint4& a, uint4& b, int j0, const float* cosr,
                                       const float* sinr) {
  rot_word_pair<T>(a.x, b.x, j0, cosr, sinr);
  rot_word_pair<T>(a.y, b.y, j0 + 2, cosr, sinr);
  rot_word_pair<T>(a.z, b.z, j0 + 4, cosr, sinr);
  rot_word_pair<T>(a.w, b.w, j0 + 6, cosr, sinr);
}

template <class T>
__device__ inline void rot_inter_word(uint32_t& w, int j, const float* cosr, const float* sinr) {
  using Bits = typename T::bits;
  Bits x = Bits(w & 0xFFFFu), y = Bits(w >> 16);
  rotate_pair<T>(x, y, cosr[j], sinr[j]);
  w = uint32_t(x) | (uint32_t(y) << 16);
}

template <class T>
__device__ inline void rot_inter_chunk(uint4& c, int j0, const float* cosr, const float* sinr) {
  rot_inter_word<T>(c.x, j0, cosr, sinr);
  rot_inter_word<T>(c.y, j0 + 1, cosr, sinr);
  rot_inter_word<T>(c.z, j0 + 2, cosr, sinr);
  rot_inter_word<T>(c.w, j0 + 3, cosr, sinr);
}

// The lane's D / 32 chunks (c2, c3 only for D = 128); `cosr`/`sinr` point
// at the position's D / 2 table entries.
template <class T, int D>
__device__ inline void rotate4(uint4& c0, uint4& c1, uint4& c2, uint4& c3, int q4,
                               const float* cosr, const float* sinr, int interleaved) {
  if (D == 128) {
    if (!interleaved) {
      rot_half_chunks<T>(c0, c2, 8 * q4, cosr, sinr);          // dims 8 q4 + e with + 64
      rot_half_chunks<T>(c1, c3, 32 + 8 * q4, cosr, sinr);
    } else {
      rot_inter_chunk<T>(c0, 4 * q4, cosr, sinr);               // pair index (32 i + 8 q4 + e) / 2
      rot_inter_chunk<T>(c1, 16 + 4 * q4, cosr, sinr);
      rot_inter_chunk<T>(c2, 32 + 4 * q4, cosr, sinr);
      rot_inter_chunk<T>(c3, 48 + 4 * q4, cosr, sinr);
    }
  } else {
    if (!interleaved) {
      rot_half_chunks<T>(c0, c1, 8 * q4, cosr, sinr);          // dims 8 q4 + e with + 32
    } else {
      rot_inter_chunk<T>(c0, 4 * q4, cosr, sinr);
      rot_inter_chunk<T>(c1, 16 + 4 * q4, cosr, sinr);
    }
  }
}

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// One block's K and V rows for lane (n, q4): key kb + n (clamped to kb past
// the unit end), dims 32 i + 8 q4 .. + 7 in member i. Named members passed by
// value: an indexed array here would end up in memory.
struct KV {
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
  uint32_t b01, b23;       // with a bias: the lane's four bias values (keys 4 q4 .. + 3 of head n)
};

// Q^T of a unit for lane (n, q4): head n, dims 32 i + 8 q4 .. + 7 in member i.
struct Q4 {
  uint4 c0, c1, c2, c3;
};

__device__ inline uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <bool kBias, int D>
__device__ inline KV load_kv(const DecodeArgs& a, const Blk& k, int n, int q4, bool slice_end,
                             bool spare = false) {
  const int row = k.kb + n < k.kend ? k.kb + n : k.kb;
  // fused eviction: key `row` is buffer row row + d. The first row of the
  // next block's sources is overwritten by that block's shifted stores. When
  // this wave also takes the next block, it loads this block well before it
  // stores the next one; when the next block starts another wave's slice,
  // the last key comes from the copy taken before the kernel. The new-token
  // key has no buffer row (past the end: any valid row, replaced).
  int src = row + k.d;
  const bool halo = k.d && slice_end && n == kKeys - 1 && k.i + 1 < k.nb;
  src = src < a.M ? src : row;
  // the slice's halo row, at its wave's index in the launch (recomputed
  // here rather than kept live through the stream)
  const int worker = int(blockIdx.x) * kDecodeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t hrow = int64_t(worker) * D + 8 * q4;
  const uint16_t* kb = k.kc;
  const uint16_t* vb = k.vc;
  if (a.past_k) {
    // fused past copy: the unit's rows come from the past buffers
    const int64_t pbase = (int64_t(k.b) * a.Hkv + k.g) * a.past_rows * D;
    kb = a.past_k + pbase;
    vb = a.past_v + pbase;
  }
  const uint16_t* kp = halo ? a.halo_k + hrow : kb + int64_t(src) * D + 8 * q4;
  const uint16_t* vp = halo ? a.halo_v + hrow : vb + int64_t(src) * D + 8 * q4;
  if (k.Lp < k.kb + kKeys) {
    // the block of the new token: that key's K and V rows come from k_new
    // and v_new (the cache row is written when the block is computed), in
    // flight with the rest of the block
    if (row == k.Lp) {
      const int64_t kvrow = (int64_t(k.b) * a.Hkv + k.g) * D + 8 * q4;
      kp = a.k_new + kvrow;
      vp = a.v_new + kvrow;
    }
  }
  // a spare load (the pipeline's refill past the slice's last block) reads
  // the first 128 Q elements instead: one cache line for the wave, not a
  // second copy of the last block, and the wait counts stay those of a full
  // pipeline (a skipped load makes the compiler wait one block earlier).
  // The bias kernel, at its register limit, measured slower with it.
  if (!kBias && spare) { kp = a.q + 8 * q4; vp = kp; }
  KV r;
  r.k0 = ld16(kp); r.k1 = ld16(kp + 32);
  r.v0 = ld16(vp); r.v1 = ld16(vp + 32);
  if (D == 128) {
    r.k2 = ld16(kp + 64); r.k3 = ld16(kp + 96);
    r.v2 = ld16(vp + 64); r.v3 = ld16(vp + 96);
  } else {
    r.k2 = r.k3 = r.v2 = r.v3 = make_uint4(0, 0, 0, 0);   // no such dims
  }
  if (kBias) {
    // head column n of the unit (padding columns reuse head h0; their
    // scores are never written out), keys kb + 4 q4 + e clamped to the
    // unit's last key: columns stay below L_b + 1 <= bias_total
    const int hg = k.ub % a.n_hg;
    const int h0 = k.g * a.G + hg * a.hg_size;
    const int nheads = min(a.hg_size, a.G - hg * a.hg_size);
    const uint16_t* brow = a.bias + k.b * a.bias_bs + int64_t(h0 + (n < nheads ? n : 0)) * a.bias_hs;
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k.kb + 4 * q4 + j < k.kend ? k.kb + 4 * q4 + j : k.kend - 1;
      e[j] = brow[key + k.coff];
    }
    r.b01 = e[0] | (e[1] << 16);
    r.b23 = e[2] | (e[3] << 16);
  }
  return r;
}

// V tile: row r holds key kb + r; its 16-byte chunk c sits at chunk
// c ^ 2 (r & 7), so that the 32 lanes of a transposing read (8 rows x 2
// chunks) hit distinct banks.
__device__ inline int vchunk(int row, int c) { return c ^ ((row & 7) << 1); }

struct Acc {
  float m_run, m_use;  // running max of the head column (log2 units) and the reference in the exponent
  float l;             // this lane's partial sum of the packed weights
  f32x4 o[8];          // O^T[16 dt + 4 q4 + r][head n]
};

__device__ inline void acc_reset(Acc& s) {
  s.m_run = -INFINITY;
  s.m_use = 0.f;
  s.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) s.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <class T>
__device__ inline uint32_t pack2(float x, float y) {
  return uint32_t(T::from_float(x)) | (uint32_t(T::from_float(y)) << 16);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <class T, bool kBias, bool kRot, int D>
__device__ inline void compute(Acc& s, KV r, const Q4& qv, const Blk& k,
                               const DecodeArgs& a, int lane, unsigned char* vt) {
  const int n = lane & 15, q4 = lane >> 4;
  if (k.kb + kKeys > k.kend && k.kb + n >= k.kend) {
    // past the unit end: the clamped row may be the unwritten new-token row
    const uint4 z = make_uint4(0, 0, 0, 0);
    r.v0 = z; r.v1 = z; r.v2 = z; r.v3 = z;
  }
  if (k.Lp >= k.kb && k.Lp < k.kb + kKeys && n == k.Lp - k.kb) {
    // the new token: its K row (loaded from k_new, rotated here) and V row
    // (from v_new) go into the cache; the head group 0 unit of the kv head
    // writes them
    if (kRot && a.rot) {
      const int pos = clamp_len(k.L + a.ro[k.b], 0, a.rot_rows - 1);
      rotate4<T, D>(r.k0, r.k1, r.k2, r.k3, q4, a.cosv + int64_t(pos) * (D / 2),
                    a.sinv + int64_t(pos) * (D / 2), a.interleaved);
    }
    if (k.ub % a.n_hg == 0) {
      const int64_t crow = ((int64_t(k.b) * a.Hkv + k.g) * a.M + k.Lp) * D + 8 * q4;
      uint4* kc = reinterpret_cast<uint4*>(a.k_cache + crow);
      uint4* vc = reinterpret_cast<uint4*>(a.v_cache + crow);
      kc[0] = r.k0; kc[4] = r.k1;
      vc[0] = r.v0; vc[4] = r.v1;
      if (D == 128) {
        kc[8] = r.k2; kc[12] = r.k3;
        vc[8] = r.v2; vc[12] = r.v3;
      }
    }
  }
  if ((k.d || a.past_k) && k.ub % a.n_hg == 0 && k.kb + n < k.kend) {
    // fused eviction: key kb + n now lives in buffer row kb + n (its source
    // rows of this block are already in registers; the row this overwrites
    // for the previous block was read from the halo copy). Fused past copy
    // (d = 0): the row read from the past buffer goes to the same row of
    // the cache.
    const int64_t crow = int64_t(k.kb + n) * D + 8 * q4;
    uint4* kc = reinterpret_cast<uint4*>(const_cast<uint16_t*>(k.kc) + crow);
    uint4* vc = reinterpret_cast<uint4*>(const_cast<uint16_t*>(k.vc) + crow);
    kc[0] = r.k0; kc[4] = r.k1;
    vc[0] = r.v0; vc[4] = r.v1;
    if (D == 128) {
      kc[8] = r.k2; kc[12] = r.k3;
      vc[8] = r.v2; vc[12] = r.v3;
    }
  }
  // ---- V rows into the tile ----
  {
    unsigned char* row = vt + n * 256;
    *reinterpret_cast<uint4*>(row + 16 * vchunk(n, q4)) = r.v0;
    *reinterpret_cast<uint4*>(row + 16 * vchunk(n, 4 + q4)) = r.v1;
    if (D == 128) {
      *reinterpret_cast<uint4*>(row + 16 * vchunk(n, 8 + q4)) = r.v2;
      *reinterpret_cast<uint4*>(row + 16 * vchunk(n, 12 + q4)) = r.v3;
    }
  }
  // ---- S^T = K Q^T: lane gets keys 4 q4 + rr of head column n ----
  f32x4 acc = Mma<T>::qk(r.k0, qv.c0, f32x4{0.f, 0.f, 0.f, 0.f});
  acc = Mma<T>::qk(r.k1, qv.c1, acc);
  if (D == 128) {
    acc = Mma<T>::qk(r.k2, qv.c2, acc);
    acc = Mma<T>::qk(r.k3, qv.c3, acc);
  }
  float sv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    float x = acc[rr] * a.scale_log2;
    if (kBias) {
      const uint32_t w = rr < 2 ? r.b01 : r.b23;
      x = fmaf(T::to_float(typename T::bits((w >> (16 * (rr & 1))) & 0xFFFFu)), kLog2e, x);
    }
    sv[rr] = k.kb + 4 * q4 + rr < k.kend ? x : -INFINITY;
  }
  float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  if (__any(bm > s.m_run + kRescaleSlack)) {
    const float mn = fmaxf(s.m_run, bm);
    const float use = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2f(s.m_use - use);
    s.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) s.o[dt] *= alpha;
    s.m_run = mn;
    s.m_use = use;
  }
  float p[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) p[rr] = exp2f(sv[rr] - s.m_use);
  uint2 pb;                            // P^T: keys 4 q4 .. 4 q4 + 3 of head n
  pb.x = pack2<T>(p[0], p[1]);
  pb.y = pack2<T>(p[2], p[3]);
  // the row sum uses the weights as rounded for the product
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
    s.l += T::to_float(typename T::bits(((rr < 2 ? pb.x : pb.y) >> (16 * (rr & 1))) & 0xFFFFu));
  wave_lds_sync();
  // ---- O^T += V^T P^T: transposing reads give lane (n, q4) dim 16 dt + n of
  // keys 4 q4 .. 4 q4 + 3 (in each 16-lane group, lane j points at key
  // 4 q4 + j / 4, dims 16 dt + 4 (j % 4) .. + 3) ----
  const int trow = 4 * q4 + (n >> 2);
  const unsigned char* tbase = vt + trow * 256 + 8 * ((n & 3) & 1);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int c = 2 * dt + ((n & 3) >> 1);
    const s16x4 x =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tbase + 16 * vchunk(trow, c)));
    s.o[dt] = Mma<T>::pv(__builtin_bit_cast(uint2, x), pb, s.o[dt]);
  }
  wave_lds_sync();   // the next block rewrites the tile
}

// The worker (wave of the launch) that owns global block x: worker w takes
// the slice [w T / N, (w + 1) T / N).
__device__ inline int owner_worker(const DecodeArgs& a, int64_t x) {
  if (a.fits32)   // the usual case: a 32-bit division (the 64-bit one is a long sequence)
    return int((uint32_t(x + 1) * uint32_t(a.workers) - 1u) / uint32_t(a.total));
  return int(((x + 1) * a.workers - 1) / a.total);
}

// Unit index, its heads and the workers sharing it.
struct UnitInfo {
  int unit, h0, nheads, w_first, w_last;
};

__device__ inline UnitInfo unit_info(const DecodeArgs& a, int b, int ub, const SeqRegs& sr) {
  UnitInfo u;
  const int g = ub / a.n_hg, hg = ub % a.n_hg;
  u.h0 = g * a.G + hg * a.hg_size;
  u.nheads = min(a.hg_size, a.G - hg * a.hg_size);
  u.unit = b * a.Hkv * a.n_hg + ub;
  const int nb = seq_of(a, b, sr).nb;
  const int64_t x0 = lane_of(sr.pb, b) + int64_t(ub) * nb;
  u.w_first = owner_worker(a, x0);
  u.w_last = owner_worker(a, x0 + nb - 1);
  return u;
}

template <class T, int D>
__device__ inline void store_out(const DecodeArgs& a, int b, int h, int d, float v) {
  reinterpret_cast<typename T::bits*>(a.out)[(int64_t(b) * a.H + h) * D + d] = T::from_float(v);
}

__device__ inline float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// End of one unit segment of this wave: normalise and write the output (the
// wave saw the whole unit) or put the unnormalised partial (o, m, l) into the
// wave's LDS slot. Lane (n, q4) holds head column n, dims 16 dt + 4 q4 + r.
template <class T, int D>
__device__ inline void finish_segment(const DecodeArgs& a, const Acc& s, const Blk& k, bool shared,
                                      float* slot, int lane) {
  const int n = lane & 15, q4 = lane >> 4;
  float l = s.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const int hg = k.ub % a.n_hg;
  const int h0 = k.g * a.G + hg * a.hg_size;
  const int nheads = min(a.hg_size, a.G - hg * a.hg_size);
  if (n >= nheads) return;
  if (!shared) {
    const float inv = 1.f / l;
    using Bits = typename T::bits;
    Bits* orow = reinterpret_cast<Bits*>(a.out) + (int64_t(k.b) * a.H + h0 + n) * D + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      uint2 w;
      w.x = pack2<T>(s.o[dt][0] * inv, s.o[dt][1] * inv);
      w.y = pack2<T>(s.o[dt][2] * inv, s.o[dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * dt) = w;
    }
    return;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<f32x4*>(slot + n * kD + 16 * dt + 4 * q4) = s.o[dt];
  if (q4 == 0) {
    slot[kDecodeMaxHG * kD + n] = s.m_use;
    slot[kDecodeMaxHG * kD + kDecodeMaxHG + n] = l;
  }
}

// Raw Q rows of block k's unit: lane (n, q4) holds head n's dims 32 i + 8 q4.
template <int D>
__device__ inline Q4 load_q_raw(const DecodeArgs& a, const Blk& k, int lane) {
  const int n = lane & 15, q4 = lane >> 4;
  const int hg = k.ub % a.n_hg;
  const int h0 = k.g * a.G + hg * a.hg_size;
  const int nheads = min(a.hg_size, a.G - hg * a.hg_size);
  const uint16_t* qrow = a.q + (int64_t(k.b) * a.H + h0 + (n < nheads ? n : 0)) * D + 8 * q4;
  Q4 q;
  q.c0 = ld16(qrow); q.c1 = ld16(qrow + 32);
  if (D == 128) {
    q.c2 = ld16(qrow + 64); q.c3 = ld16(qrow + 96);
  } else {
    q.c2 = q.c3 = make_uint4(0, 0, 0, 0);
  }
  return q;
}

__device__ inline uint4 mask4(uint4 c, uint32_t m) {
  return make_uint4(c.x & m, c.y & m, c.z & m, c.w & m);
}

// Rotate Q at position L_b and zero the padding heads (a mask, no select of
// aggregates: the rows stay in registers).
template <class T, bool kRot, int D>
__device__ __forceinline__ Q4 finish_q(Q4 q, const DecodeArgs& a, const Blk& k, int lane) {
  const int n = lane & 15, q4 = lane >> 4;
  const int hg = k.ub % a.n_hg;
  const int nheads = min(a.hg_size, a.G - hg * a.hg_size);
  if (kRot && a.rot) {
    const int pos = clamp_len(k.L + a.ro[k.b], 0, a.rot_rows - 1);
    rotate4<T, D>(q.c0, q.c1, q.c2, q.c3, q4, a.cosv + int64_t(pos) * (D / 2),
                  a.sinv + int64_t(pos) * (D / 2), a.interleaved);
  }
  const uint32_t keep = n < nheads ? 0xFFFFFFFFu : 0u;
  q.c0 = mask4(q.c0, keep); q.c1 = mask4(q.c1, keep);
  q.c2 = mask4(q.c2, keep); q.c3 = mask4(q.c3, keep);
  return q;
}

// A workgroup's table entry: a unit one of its waves holds only in part
// (from the start of its slice, or to its end), with what its combine and
// merge need. Written at the start of the slice, read after it.
enum { kEntUnit, kEntB, kEntH0, kEntHeads, kEntWFirst, kEntWLast, kEntInts = 8 };

struct EntInfo {
  int unit, b, h0, nheads, w_first, w_last;
};

// One LDS round trip; every lane reads the same words (wave-uniform values).
__device__ inline EntInfo read_entry(const int* ent) {
  const int4 x = *reinterpret_cast<const int4*>(ent);
  const int2 y = *reinterpret_cast<const int2*>(ent + 4);
  EntInfo u;
  u.unit = __builtin_amdgcn_readfirstlane(x.x);
  u.b = __builtin_amdgcn_readfirstlane(x.y);
  u.h0 = __builtin_amdgcn_readfirstlane(x.z);
  u.nheads = __builtin_amdgcn_readfirstlane(x.w);
  u.w_first = __builtin_amdgcn_readfirstlane(y.x);
  u.w_last = __builtin_amdgcn_readfirstlane(y.y);
  return u;
}

// Merge the workgroup partials of a unit (slots wg_first + unit .. wg_last +
// unit) by log-sum-exp, write the output and reset the unit's counter. All
// threads of the workgroup; `lds` holds 2 kMergeMax x 16 floats.
template <class T, int D>
__device__ inline void merge_unit(const DecodeArgs& a, const EntInfo& u, float* lds) {
  const int tid = threadIdx.x;
  const int b = u.b;
  const int wg_first = u.w_first / kDecodeWaves, wg_last = u.w_last / kDecodeWaves;
  const int count = wg_last - wg_first + 1;
  const float* base = a.partials + int64_t(wg_first + u.unit) * kSlotFloats;
  if (count <= 4) {
    // usual case: every thread loads m, l and o of all partials for its
    // output at once (one memory round trip), no LDS pass
    for (int idx = tid; idx < u.nheads * D; idx += kThreads) {
      const int h = idx / D, d = idx % D;
      float m[4], l[4], o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* sl = base + int64_t(j < count ? j : 0) * kSlotFloats;
        m[j] = ld_agent(sl + kDecodeMaxHG * kD + h);
        l[j] = ld_agent(sl + kDecodeMaxHG * kD + kDecodeMaxHG + h);
        o[j] = ld_agent(sl + h * kD + d);
      }
      float M = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) M = j < count ? fmaxf(M, m[j]) : M;
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float w = j < count ? __builtin_amdgcn_exp2f(m[j] - M) : 0.f;
        L = fmaf(l[j], w, L);
        O = fmaf(o[j], w, O);
      }
      store_out<T, D>(a, b, u.h0 + h, d, O / L);
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.counters + u.unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  float* wm = lds;                                   // [count][16] -> weights
  float* wl = lds + kMergeMax * 16;                  // [count][16]
  for (int idx = tid; idx < count * 16; idx += kThreads) {
    const int j = idx >> 4, h = idx & 15;
    const float* sl = base + int64_t(j) * kSlotFloats;
    wm[idx] = h < u.nheads ? ld_agent(sl + kDecodeMaxHG * kD + h) : 0.f;
    wl[idx] = h < u.nheads ? ld_agent(sl + kDecodeMaxHG * kD + kDecodeMaxHG + h) : 0.f;
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
  for (int idx = tid; idx < u.nheads * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float acc = 0.f;
    for (int j0 = 0; j0 < count; j0 += 8) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x[j] = j0 + j < count ? ld_agent(base + int64_t(j0 + j) * kSlotFloats + h * kD + d) : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j0 + j < count) acc = fmaf(x[j], wm[(j0 + j) * 16 + h], acc);
    }
    store_out<T, D>(a, b, u.h0 + h, d, acc);
  }
  __syncthreads();
  if (tid == 0) __hip_atomic_store(a.counters + u.unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Entry `ent` of this wave: unit of block k when `on`, else empty.
__device__ inline void set_entry(const DecodeArgs& a, int* ent, bool on, const Blk& k,
                                 const SeqRegs& sr, int lane) {
  if (on) {
    const UnitInfo u = unit_info(a, k.b, k.ub, sr);
    if (lane == 0) {
      ent[kEntUnit] = u.unit; ent[kEntB] = k.b; ent[kEntH0] = u.h0; ent[kEntHeads] = u.nheads;
      ent[kEntWFirst] = u.w_first; ent[kEntWLast] = u.w_last;
    }
  } else if (lane == 0) {
    ent[kEntUnit] = -1;
  }
}

// One launch: workgroups of kDecodeWaves waves; every wave of the grid
// streams its own slice (see the top of the file), then the workgroup
// combines the partials its waves left.
template <class T, bool kBias, bool kRot, int D>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kDecodeWaves * kWaveLds];
  // per wave, entries 2 wv (its first unit, partial in slot 0) and 2 wv + 1
  // (its last unit, partial in slot 1)
  __shared__ __attribute__((aligned(16))) int sh_ent[2 * kDecodeWaves][kEntInts];
  __shared__ int sh_flag[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q4 = lane >> 4;
  const int wg = blockIdx.x;
  const int worker = wg * kDecodeWaves + wv;
  float* slot0 = reinterpret_cast<float*>(lds + wv * kWaveLds);
  float* slot1 = reinterpret_cast<float*>(lds + wv * kWaveLds + kSlotBytes);
  unsigned char* vt = lds + wv * kWaveLds + kSlotBytes;     // the V tile while streaming
  const SeqRegs sr = load_seq_regs(a, lane);

  int64_t S = 0, E = 0;
  if (worker < a.workers) {
    if (a.fits32) {
      S = uint32_t(worker) * uint32_t(a.total) / uint32_t(a.workers);
      E = uint32_t(worker + 1) * uint32_t(a.total) / uint32_t(a.workers);
    } else {
      S = (int64_t(worker) * a.total) / a.workers;
      E = (int64_t(worker + 1) * a.total) / a.workers;
    }
  }
  if (S >= E) {
    set_entry(a, sh_ent[2 * wv], false, Blk{}, sr, lane);
    set_entry(a, sh_ent[2 * wv + 1], false, Blk{}, sr, lane);
  } else {
    Blk cur = locate<D>(a, S, sr, lane);
    const Q4 qraw = load_q_raw<D>(a, cur, lane);
    KV rc = load_kv<kBias, D>(a, cur, n, q4, S + 1 >= E);
    Acc s;
    acc_reset(s);
    bool seg_shared = cur.i > 0;          // the unit began in an earlier slice

    // Blocks move through three register sets: while block x is computed,
    // x + 1 and x + 2 are in flight. `ahead` is the block whose loads go out
    // next (x + 2), clamped to the slice's last block; past it the loads are
    // spare ones. Q rows are loaded when their unit starts (a small,
    // cache-resident read).
    Blk nxt = S + 1 < E ? next_block<D>(a, cur, sr) : cur;        // block x + 1
    KV r1 = load_kv<kBias, D>(a, nxt, n, q4, S + 2 >= E);
    Blk ahead = S + 2 < E ? next_block<D>(a, nxt, sr) : nxt;       // block x + 2

    // While the first loads are in flight: this wave's table entries. Its
    // first unit leaves a partial (slot 0) if it began in an earlier slice
    // and ends inside this one; its last unit (slot 1) if it goes on past
    // the slice, or if it is also the first and began earlier. The
    // segment-closing code below writes exactly these slots.
    {
      const Blk lb = S + 1 < E ? locate<D>(a, E - 1, sr, lane) : cur;
      const bool same = lb.b == cur.b && lb.ub == cur.ub;
      const bool open_end = lb.i + 1 < lb.nb;
      set_entry(a, sh_ent[2 * wv], cur.i > 0 && !same, cur, sr, lane);
      set_entry(a, sh_ent[2 * wv + 1], same ? (cur.i > 0 || open_end) : open_end, lb, sr, lane);
    }
    Q4 qv = finish_q<T, kRot, D>(qraw, a, cur, lane);

    // one block: issue the loads of x + 2, compute x, close the segment at a
    // unit end or at the slice end. Returns false after the slice's last block.
    auto step = [&](int64_t x, KV& r_cur, KV& r_fill) -> bool {
      const bool last = x + 1 >= E;
      const bool unit_end = cur.i + 1 >= cur.nb;
      r_fill = load_kv<kBias, D>(a, ahead, n, q4, x + 3 >= E, x + 2 >= E);   // ahead = min(x + 2, E - 1)
      compute<T, kBias, kRot, D>(s, r_cur, qv, cur, a, lane, vt);
      if (unit_end || last) {
        const bool shared = seg_shared || !unit_end;
        if (shared) {
          // the slice's last segment goes to slot 1 (over the V tile, free now)
          finish_segment<T, D>(a, s, cur, true, last ? slot1 : slot0, lane);
        } else {
          finish_segment<T, D>(a, s, cur, false, slot0, lane);
        }
        if (last) return false;
        acc_reset(s);
        seg_shared = false;
        qv = finish_q<T, kRot, D>(load_q_raw<D>(a, nxt, lane), a, nxt, lane);
      }
      cur = nxt;
      nxt = ahead;
      ahead = x + 3 < E ? next_block<D>(a, ahead, sr) : ahead;
      return true;
    };
    KV r2;
    for (int64_t x = S;; x += 3) {
      if (!step(x, rc, r2)) break;
      if (!step(x + 1, r1, rc)) break;
      if (!step(x + 2, r2, r1)) break;
    }
  }
  __syncthreads();

  // ---- combine the partials of each cut unit. Entries of a unit are
  // consecutive in slice order (empty entries between them are skipped).
  // This runs once per workgroup after its slowest wave, so it is kept to
  // scalar masks and the reads each unit needs: the entries were filled in
  // at the start of the slices. ----
  int key[2 * kDecodeWaves];                  // unit of each entry, -1 if empty
#pragma unroll
  for (int f = 0; f < 2 * kDecodeWaves; ++f) key[f] = __builtin_amdgcn_readfirstlane(sh_ent[f][kEntUnit]);
  uint32_t firsts = 0;                        // first entry of each unit
  {
    int lastk = -1;
#pragma unroll
    for (int f = 0; f < 2 * kDecodeWaves; ++f) {
      if (key[f] >= 0 && key[f] != lastk) firsts |= 1u << f;
      lastk = key[f] >= 0 ? key[f] : lastk;
    }
  }
  int nglob = 0, gent0 = 0, gent1 = 0;        // entries of the units counted in (at most two)
  while (firsts) {
    const int e = __builtin_ctz(firsts);
    firsts &= firsts - 1;
    const EntInfo u = read_entry(sh_ent[e]);
    uint32_t um = 0;                          // this unit's entries
#pragma unroll
    for (int f = 0; f < 2 * kDecodeWaves; ++f) um |= (key[f] == u.unit ? 1u : 0u) << f;
    const bool inside = u.w_first >= wg * kDecodeWaves && u.w_last < (wg + 1) * kDecodeWaves;
    float* gslot = a.partials + int64_t(wg + u.unit) * kSlotFloats;
    for (int idx = tid; idx < u.nheads * D; idx += kThreads) {
      const int h = idx / D, d = idx % D;
      float m[2 * kDecodeWaves], l[2 * kDecodeWaves], o[2 * kDecodeWaves];
#pragma unroll
      for (int f = 0; f < 2 * kDecodeWaves; ++f) {
        m[f] = -INFINITY;
        l[f] = 0.f;
        o[f] = 0.f;
        if (um & (1u << f)) {                 // wave-uniform
          const float* sl = reinterpret_cast<const float*>(lds + (f >> 1) * kWaveLds + (f & 1) * kSlotBytes);
          m[f] = sl[kDecodeMaxHG * kD + h];
          l[f] = sl[kDecodeMaxHG * kD + kDecodeMaxHG + h];
          o[f] = sl[h * kD + d];
        }
      }
      float M = -INFINITY;
#pragma unroll
      for (int f = 0; f < 2 * kDecodeWaves; ++f) M = __builtin_elementwise_maximum(M, m[f]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int f = 0; f < 2 * kDecodeWaves; ++f) {
        const float wgt = __builtin_amdgcn_exp2f(m[f] - M);     // 0 for the others
        L = fmaf(l[f], wgt, L);
        O = fmaf(o[f], wgt, O);
      }
      if (inside) {
        store_out<T, D>(a, u.b, u.h0 + h, d, O / L);
      } else {
        __hip_atomic_store(gslot + h * kD + d, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
          __hip_atomic_store(gslot + kDecodeMaxHG * kD + h, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(gslot + kDecodeMaxHG * kD + kDecodeMaxHG + h, L, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (!inside) {
      if (nglob == 0) gent0 = e;
      else gent1 = e;
      ++nglob;
    }
  }
  if (nglob == 0) return;
  // release/acquire handoff: the workgroup barrier orders every thread's
  // partial stores before the count; the counting thread's increment
  // releases them at agent scope (every increment of a counter continues
  // the release sequence of the earlier ones), and the thread whose
  // increment completes the count acquires at agent scope before the
  // barrier that carries it to the whole workgroup. Only that workgroup pays
  // for the acquire (an L2 invalidate, which would otherwise also drop lines
  // the other workgroups on its XCD still read).
  __syncthreads();
  if (tid < nglob) {
    // counted in; the workgroup that completes the count merges
    const int* ent = sh_ent[tid ? gent1 : gent0];
    const int need = ent[kEntWLast] / kDecodeWaves - ent[kEntWFirst] / kDecodeWaves;
    const int prev = __hip_atomic_fetch_add(a.counters + ent[kEntUnit], 1, __ATOMIC_RELEASE,
                                            __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == need;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sh_flag[tid] = last;
  }
  __syncthreads();
  float* mlds = reinterpret_cast<float*>(lds);       // the slots are read: reuse
#pragma unroll 1
  for (int j = 0; j < nglob; ++j)                     // one copy of the merge code
    if (sh_flag[j]) merge_unit<T, D>(a, read_entry(sh_ent[j ? gent1 : gent0]), mlds);
}

// Fused eviction, before the decode kernel: for the last block i of every
// worker's slice whose unit goes on into the next worker's slice, copy the
// first source row of block i + 1 (key 16 i + 15's source), which block
// i + 1's shifted stores, made by another wave, may overwrite first.
template <int D>
__global__ void __launch_bounds__(64) shift_halo_kernel(DecodeArgs a) {
  // one wave per worker (its plan values stay scalar): lanes 0-15 copy the K
  // row, lanes 16-31 the V row, 16 bytes each
  const int w = blockIdx.x, lane = threadIdx.x;
  int64_t S, E;
  if (a.fits32) {
    S = uint32_t(w) * uint32_t(a.total) / uint32_t(a.workers);
    E = uint32_t(w + 1) * uint32_t(a.total) / uint32_t(a.workers);
  } else {
    S = (int64_t(w) * a.total) / a.workers;
    E = (int64_t(w + 1) * a.total) / a.workers;
  }
  if (S >= E) return;
  // all 64 lanes take part in the lookup (one lane per sequence)
  const SeqRegs sr = load_seq_regs(a, lane);
  const Blk k = locate<D>(a, E - 1, sr, lane);
  const int part = lane & 15;
  if (lane >= 32 || !k.d || k.i + 1 >= k.nb || 8 * part >= D) return;
  const bool vside = lane >= 16;
  const uint16_t* src = (vside ? k.vc : k.kc) + int64_t(k.kb + kKeys - 1 + k.d) * D;
  uint16_t* dst = (vside ? a.halo_v : a.halo_k) + int64_t(w) * D;
  *reinterpret_cast<uint4*>(dst + 8 * part) = *reinterpret_cast<const uint4*>(src + 8 * part);
}

}  // namespace

bool decode_fused_evict_supported(const Problem& p) {
  // the window must cover the whole buffer (every kept row is read, so every
  // kept row can be moved by its reader), and one unit per kv head (a single
  // head group reads, and so may rewrite, each row)
  return p.window >= p.M && ceil_div(p.G, kDecodeMaxHG) == 1;
}

bool decode_fast_supported(const Problem& p) {
  return (p.D == 128 || p.D == 64) && (p.dtype == GQA_FP16 || p.dtype == GQA_BF16) && p.S == 1;
}

namespace {

// One instantiation per dtype, bias, rotary and head size.
template <int D>
hipError_t launch_decode_kernel(const Problem& p, const DecodeArgs& a, dim3 grid, dim3 wg,
                                hipStream_t st) {
  if (a.shift) {
    hipLaunchKernelGGL(shift_halo_kernel<D>, dim3(a.workers), dim3(64), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // rotary gets kernels of its own: without the rotation code the streaming
  // loop needs fewer registers
  const bool fp16 = p.dtype == GQA_FP16;
  if (a.rot) {
    if (p.bias && fp16) hipLaunchKernelGGL((decode_kernel<F16, true, true, D>), grid, wg, 0, st, a);
    else if (p.bias) hipLaunchKernelGGL((decode_kernel<BF16, true, true, D>), grid, wg, 0, st, a);
    else if (fp16) hipLaunchKernelGGL((decode_kernel<F16, false, true, D>), grid, wg, 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<BF16, false, true, D>), grid, wg, 0, st, a);
  } else {
    if (p.bias && fp16) hipLaunchKernelGGL((decode_kernel<F16, true, false, D>), grid, wg, 0, st, a);
    else if (p.bias) hipLaunchKernelGGL((decode_kernel<BF16, true, false, D>), grid, wg, 0, st, a);
    else if (fp16) hipLaunchKernelGGL((decode_kernel<F16, false, false, D>), grid, wg, 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<BF16, false, false, D>), grid, wg, 0, st, a);
  }
  return hipGetLastError();
}

// One launch over at most kDecodeArgBatch sequences (their plan travels in
// the kernel arguments).
hipError_t launch_decode_batch(const Problem& p, void* ws, const WorkspaceLayout& lay,
                               hipStream_t st, bool fuse_evict) {
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
  a.shift = fuse_evict ? 1 : 0;
  a.past_k = static_cast<const uint16_t*>(p.past_k);
  a.past_v = static_cast<const uint16_t*>(p.past_v);
  a.past_rows = p.past_rows;
  a.halo_k = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + lay.decode_halo);
  a.halo_v = a.halo_k + int64_t(kDecodeMaxWorkers) * p.D;
  a.B = p.B; a.H = p.H; a.Hkv = p.Hkv; a.G = p.G; a.M = p.M; a.W = p.window; a.cap = p.cap;
  a.n_hg = ceil_div(p.G, kDecodeMaxHG);
  a.hg_size = ceil_div(p.G, a.n_hg);
  a.scale_log2 = p.scale * kLog2e;
  a.bias = static_cast<const uint16_t*>(p.bias);
  a.bias_bs = p.bias_bs; a.bias_hs = p.bias_hs;
  const int units_per_seq = p.Hkv * a.n_hg;
  int64_t total = 0;
  for (int b = 0; b < p.B; ++b) {
    const int L = kept_rows_host(p.lens_host[b], 1, p.M, p.cap);
    const int kend = L + 1;
    const int kstart = p.window > 0 ? (kend - p.window > 0 ? kend - p.window : 0) : 0;
    a.hl[b] = p.lens_host[b];
    a.ro[b] = p.off_host ? p.off_host[b] : 0;
    a.pb[b] = int32_t(total);
    total += int64_t((kend - kstart + kKeys - 1) / kKeys) * units_per_seq;
  }
  a.pb[p.B] = int32_t(total);
  a.total = total;
  if (total == 0) return hipSuccess;
  // workers (waves): at most one workgroup per CU, and no unit shared by
  // more than kMergeMax of them
  int64_t workers = kDecodeMaxWorkers < total ? kDecodeMaxWorkers : total;
  int64_t max_unit = 0;
  for (int b = 0; b < p.B; ++b) {
    const int64_t nb = p.B ? (a.pb[b + 1] - a.pb[b]) / units_per_seq : 0;
    max_unit = nb > max_unit ? nb : max_unit;
  }
  while (workers > 1 && max_unit * workers > int64_t(kMergeMax - 1) * total) workers /= 2;
  a.workers = int(workers);
  a.fits32 = (total + 1) * workers < (int64_t(1) << 32) ? 1 : 0;
  const int blocks = int((workers + kDecodeWaves - 1) / kDecodeWaves);
  const dim3 grid(blocks), wg(kThreads);
  return p.D == 128 ? launch_decode_kernel<128>(p, a, grid, wg, st)
                    : launch_decode_kernel<64>(p, a, grid, wg, st);
}

}  // namespace

// Batches of more than kDecodeArgBatch sequences run as consecutive launches
// over groups of kDecodeArgBatch sequences (sequences are independent; the
// launches share the workspace in stream order, and each leaves the merge
// counters at zero for the next).
hipError_t launch_decode_fast(const Problem& p, void* ws, const WorkspaceLayout& lay,
                              hipStream_t st, bool fuse_evict) {
  if (p.B <= kDecodeArgBatch) return launch_decode_batch(p, ws, lay, st, fuse_evict);
  for (int b0 = 0; b0 < p.B; b0 += kDecodeArgBatch) {
    Problem c = p;
    c.B = p.B - b0 < kDecodeArgBatch ? p.B - b0 : kDecodeArgBatch;
    const int64_t qrow = int64_t(b0) * p.H * p.D;             // [B, 1, H, D] (S == 1)
    const int64_t kvrow = int64_t(b0) * p.Hkv * p.D;          // [B, 1, Hkv, D]
    const int64_t crow = int64_t(b0) * p.Hkv * p.M * p.D;     // [B, Hkv, M, D]
    c.q = static_cast<const uint16_t*>(p.q) + qrow;
    c.out = static_cast<uint16_t*>(p.out) + qrow;
    c.k_new = static_cast<const uint16_t*>(p.k_new) + kvrow;
    c.v_new = static_cast<const uint16_t*>(p.v_new) + kvrow;
    c.k_cache = static_cast<uint16_t*>(p.k_cache) + crow;
    c.v_cache = static_cast<uint16_t*>(p.v_cache) + crow;
    if (p.past_k) {
      const int64_t prow = int64_t(b0) * p.Hkv * p.past_rows * p.D;
      c.past_k = static_cast<const uint16_t*>(p.past_k) + prow;
      c.past_v = static_cast<const uint16_t*>(p.past_v) + prow;
    }
    c.lens_host = p.lens_host + b0;
    c.lens_dev = p.lens_dev ? p.lens_dev + b0 : nullptr;
    c.off_host = p.off_host ? p.off_host + b0 : nullptr;
    c.off_dev = p.off_dev ? p.off_dev + b0 : nullptr;
    if (p.bias) c.bias = static_cast<const uint16_t*>(p.bias) + b0 * p.bias_bs;
    const hipError_t e = launch_decode_batch(c, ws, lay, st, fuse_evict);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gqa
