// Device-side helpers shared by the FlashHead kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cfloat>

#include "fh_internal.hpp"

namespace fh {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- numerics --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// a.x*b.x + a.y*b.y + acc over packed bfloat16 pairs, float32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Dot product of one 16-byte chunk: 8 bfloat16 or 4 float32 elements.
template <typename T>
struct Chunk;

template <>
struct Chunk<uint16_t> {  // bfloat16 bit patterns
  static constexpr int kElems = 8;
  __device__ __forceinline__ static float dot(const uint4& a, const uint4& b, float acc) {
    acc = dot2_bf16(a.x, b.x, acc);
    acc = dot2_bf16(a.y, b.y, acc);
    acc = dot2_bf16(a.z, b.z, acc);
    acc = dot2_bf16(a.w, b.w, acc);
    return acc;
  }
};

template <>
struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static float dot(const uint4& a, const uint4& b, float acc) {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
    return acc;
  }
};

// ------------------------------------------------------------ wave helpers --
// Cross-lane work uses DPP: four row-local steps (quad swaps, half-row and
// row mirrors) combine the 16 lanes of each row with VALU latency, and the
// four row results are read back as scalars.  The combination order is
// fixed, so results are deterministic.

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <typename Op>
__device__ __forceinline__ float row_allreduce(float v, Op op) {
  v = op(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_f<0x141>(v));  // row_half_mirror
  v = op(v, dpp_f<0x140>(v));  // row_mirror
  return v;
}

__device__ __forceinline__ float wave_sum(float x) {
  x = row_allreduce(x, [](float a, float b) { return a + b; });
  return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}

__device__ __forceinline__ float wave_max(float x) {
  x = row_allreduce(x, [](float a, float b) { return fmaxf(a, b); });
  return fmaxf(fmaxf(readlane_f(x, 0), readlane_f(x, 16)), fmaxf(readlane_f(x, 32), readlane_f(x, 48)));
}

__device__ __forceinline__ float wave_min(float x) {
  x = row_allreduce(x, [](float a, float b) { return fminf(a, b); });
  return fminf(fminf(readlane_f(x, 0), readlane_f(x, 16)), fminf(readlane_f(x, 32), readlane_f(x, 48)));
}

// Inclusive prefix sum across the wave (lane order): a Hillis-Steele scan
// inside each row (row_shr 1, 2, 4, 8 with zero fill), then the totals of
// earlier rows added from scalar reads.
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
  x += dpp_i<0x111>(x);
  x += dpp_i<0x112>(x);
  x += dpp_i<0x114>(x);
  x += dpp_i<0x118>(x);
  const int t0 = __builtin_amdgcn_readlane(x, 15);
  const int t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// ------------------------------------------------------------------ Philox --
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds over a
// 128-bit counter with a 64-bit key; counter words 0 and 2 are multiplied by
// two fixed odd constants, the product halves are mixed with the other
// words and the key, and the key advances by two Weyl increments per round.

struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox4x32_10(U4 ctr, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t a = 0xD2511F53u * ctr.x;
    const uint32_t ah = __umulhi(0xD2511F53u, ctr.x);
    const uint32_t c = 0xCD9E8D57u * ctr.z;
    const uint32_t ch = __umulhi(0xCD9E8D57u, ctr.z);
    ctr = U4{ch ^ ctr.y ^ k0, c, ah ^ ctr.w ^ k1, a};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return ctr;
}

// The four Philox words of block `blk` (= index / 4) for (seed, row, stage).
__device__ __forceinline__ U4 philox_block(uint64_t seed, uint32_t row, uint32_t blk,
                                           uint32_t stage) {
  return philox4x32_10(U4{blk, row, stage, 0u}, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t u4_word(const U4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// Standard Gumbel variate from one 32-bit word: u = ((w >> 9) + 1/2) 2^-23
// lies in (0, 1) and is exact in float32; G = -ln(-ln u).
__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
  const float u = ((float)(w >> 9) + 0.5f) * 1.1920928955078125e-07f;
  return -logf(-logf(u));
}

__device__ __forceinline__ float gumbel_at(uint64_t seed, uint32_t row, uint32_t index,
                                           uint32_t stage) {
  const U4 blk = philox_block(seed, row, index >> 2, stage);
  return gumbel_from_word(u4_word(blk, index & 3));
}

// The stage-1 value of query q and cluster k: the score, or the selection
// key s / T + G(seed, q, k, 0) (the same float operations as k_select's).
__device__ __forceinline__ float stage1_value(float s, int sample, float temperature,
                                              uint64_t seed, uint32_t q, uint32_t k) {
  return sample ? s / temperature + gumbel_at(seed, q, k, 0u) : s;
}

// -------------------------------------------- device-coherent accesses ----
// Agent-scope relaxed atomics compile to sc1 loads/stores on gfx950: they
// reach the device coherence point, so workgroups on other XCDs see them
// without an L2-wide writeback or invalidate.

__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------ epilogue partials --
// A partial result over a set of candidate tokens: the best (key, id) pair
// with the logit of that token, and (m, s) with m = max x, s = sum exp(x - m)
// for x = z / T'.


__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ Part part_empty() {
  return Part{-INFINITY, 0.f, -INFINITY, 0.f, 0x7FFFFFFF};
}

__device__ __forceinline__ Part part_merge(const Part& a, const Part& b) {
  Part r;
  if (better(b.key, b.id, a.key, a.id)) {
    r.key = b.key; r.id = b.id; r.z = b.z;
  } else {
    r.key = a.key; r.id = a.id; r.z = a.z;
  }
  // (m, s): the larger max keeps its sum, the other's sum is rescaled by
  // one exponential (commutative: equal maxima add the sums either way)
  const bool ab = a.m >= b.m;
  const float hm = ab ? a.m : b.m, lm = ab ? b.m : a.m;
  const float hs = ab ? a.s : b.s, ls = ab ? b.s : a.s;
  r.m = hm;
  r.s = hm == -INFINITY ? 0.f : fmaf(ls, __expf(lm - hm), hs);
  return r;
}

template <int CTRL>
__device__ __forceinline__ Part dpp_part(const Part& p) {
  return Part{dpp_f<CTRL>(p.key), dpp_f<CTRL>(p.z), dpp_f<CTRL>(p.m), dpp_f<CTRL>(p.s),
              dpp_i<CTRL>(p.id)};
}

__device__ __forceinline__ Part readlane_part(const Part& p, int l) {
  return Part{readlane_f(p.key, l), readlane_f(p.z, l), readlane_f(p.m, l), readlane_f(p.s, l),
              __builtin_amdgcn_readlane(p.id, l)};
}

// Merge the Parts of all 64 lanes; every lane gets the result.
__device__ __forceinline__ Part wave_merge_part(Part p) {
  p = part_merge(p, dpp_part<0xB1>(p));
  p = part_merge(p, dpp_part<0x4E>(p));
  p = part_merge(p, dpp_part<0x141>(p));
  p = part_merge(p, dpp_part<0x140>(p));
  return part_merge(part_merge(readlane_part(p, 0), readlane_part(p, 16)),
                    part_merge(readlane_part(p, 32), readlane_part(p, 48)));
}

__device__ __forceinline__ void st_coherent_part(Part* p, const Part& v) {
  st_coherent(&p->key, v.key);
  st_coherent(&p->z, v.z);
  st_coherent(&p->m, v.m);
  st_coherent(&p->s, v.s);
  __hip_atomic_store(&p->id, v.id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ Part ld_coherent_part(const Part* p) {
  Part v;
  v.key = ld_coherent(&p->key);
  v.z = ld_coherent(&p->z);
  v.m = ld_coherent(&p->m);
  v.s = ld_coherent(&p->s);
  v.id = __hip_atomic_load(const_cast<int32_t*>(&p->id), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

}  // namespace fh
