// Device building blocks shared by the FlashHead kernels for gfx950: row
// GEMVs over bf16 / fp32 / INT4 rows with a fused max / log-sum-exp / Gumbel
// epilogue, the block-wide probe selection and the partial-result merge.
//
// Sources (page title and section): FlashHead technical explainer
// (framerc.cn) §1.1, §1.2.1-§1.2.4, §2.2.2, §2.3; "FlashHead: Efficient
// Drop-In Replacement for the Classification Head in Language Model
// Inference" (arXiv 2603.14591), abstract.
#pragma once

#include <cfloat>
#include <cstdint>

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "fh_device.hpp"
#include "fh_internal.hpp"

namespace fh {

// Optional per-workgroup phase timestamps for performance probes (off in
// the library build): slot s, workgroup w -> wall clock at phase s.
#ifdef FH_PHASE_TRACE
__device__ unsigned long long g_fh_trace[24][4096];
#define FH_TRACE(slot) \
  if (threadIdx.x == 0 && blockIdx.x < 4096) g_fh_trace[slot][blockIdx.x] = wall_clock64();
__device__ __forceinline__ void g_fh_trace_cnt(int n) { g_fh_trace[15][blockIdx.x] = (unsigned long long)n; }
#else
#define FH_TRACE(slot)
#define g_fh_trace_cnt(n)
#endif

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// ======================================================================
// Wave-level row GEMV.
//
// A wavefront computes z = M[src(r)] . h_q for rows r = r_begin, r_begin +
// stride, ... < r_end and NQ queries.  Lane l owns the 16-byte chunks l,
// l+64, ... of a row (MAXM of them at most), so a row is read as fully
// coalesced 16-byte loads and the lane's slice of each h stays in registers
// (hv) for all rows.  RPI rows' loads are issued before any math; AUX is the
// loads' cache policy (kLoadStream for rows read once).  `sink` is called by
// every lane with the wave-uniform result of each (row, query) and the token
// id tok_of(src(r)).
// ======================================================================
template <typename T, int MAXM>
__device__ __forceinline__ void load_hslice(const T* h, int nch, int lane, uint4 (&hv)[MAXM]) {
  const uint4* hq = reinterpret_cast<const uint4*>(h);
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    const int ch = lane + 64 * m;
    hv[m] = ch < nch ? hq[ch] : uint4{0u, 0u, 0u, 0u};
  }
}

// A 16-byte load of chunk ch of a row through a buffer resource whose range
// is the row's nch chunks: chunks past the row read as zero, so no lane needs
// an exec mask around the load, and the compiler can count the loads in
// flight exactly (waiting for one row while later rows are still loading).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, int nch) {
  // word 3: raw (untyped) 32-bit dword access, as CDNA buffer loads take it
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, nch * 16, 0x00020000);
}
// Cache-policy argument of a buffer load: the non-temporal (nt) hint, for
// rows streamed once per call.
constexpr int kLoadStream = 2;
template <int AUX = 0>
__device__ __forceinline__ uint4 row_chunk(__amdgpu_buffer_rsrc_t rs, int ch) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, ch * 16, 0, AUX);
  return uint4{v[0], v[1], v[2], v[3]};
}

template <typename T, int MAXM, int NQ, int RPI = 2, int AUX = 0, typename SrcOf,
          typename TokOf, typename Sink>
__device__ __forceinline__ void wave_rows(const T* __restrict__ M, int d, int lane,
                                          const uint4 (&hv)[NQ][MAXM], int nq, int64_t r_begin,
                                          int64_t r_end, int64_t stride, SrcOf src_of,
                                          TokOf tok_of, Sink sink) {
  const int nch = d / Chunk<T>::kElems;
#pragma unroll 1
  for (int64_t r = r_begin; r < r_end; r += RPI * stride) {
    // RPI rows' loads are issued before any math
    bool ok[RPI];
    int64_t src[RPI], tk[RPI];
    uint4 mr[RPI][MAXM];
#pragma unroll
    for (int i = 0; i < RPI; ++i) {
      ok[i] = i == 0 || r + i * stride < r_end;
      // a row past the end stands in as row r (read twice, from cache), so
      // that no index or load is conditional on another row's loaded value
      src[i] = src_of(ok[i] ? r + i * stride : r);
      tk[i] = tok_of(src[i]);
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(M + src[i] * d, nch);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) mr[i][m] = row_chunk<AUX>(rs, lane + 64 * m);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q >= nq) break;
      // each row's dot product as soon as its own loads are in
#pragma unroll
      for (int i = 0; i < RPI; ++i) {
        if (!ok[i]) break;
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc = Chunk<T>::dot(mr[i][m], hv[q][m], acc);
        sink(q, r + i * stride, tk[i], wave_sum(acc));
      }
    }
  }
}

// ======================================================================
// Wave-level stage-1 GEMV on g32 codes: s[k] = sum_g sigma[k, g] sum_{i in g}
// q h (INT4 or INT8).  Lane l owns groups l, l+64, ...; the query's groups
// and their sums stay in registers (HGroups).  INT4: one 16-byte load is one
// group's 32 nibbles; nibbles become unsigned bytes u = q + 8 (xor
// 0x88888888, two masks), cvt_f32_ubyte converts them, and sum q h =
// sum u h - 8 sum_g h removes the offset with the group sums of h.
// ======================================================================
template <int MAXG>
struct HGroups {
  float h[MAXG][32];
  float hsum[MAXG];
};

template <typename T, int MAXG>
__device__ __forceinline__ void load_hgroups(const T* h, int G, int lane, HGroups<MAXG>& hg) {
  constexpr int kPer = 16 / (int)sizeof(T);  // elements per 16-byte load
#pragma unroll
  for (int m = 0; m < MAXG; ++m) {
    const int g = lane + 64 * m;
    const uint4* src = reinterpret_cast<const uint4*>(h + (int64_t)min(g, G - 1) * 32);
#pragma unroll
    for (int c = 0; c < 32 / kPer; ++c) {
      const uint4 v = g < G ? src[c] : uint4{0u, 0u, 0u, 0u};
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        float x;
        if (sizeof(T) == 2)
          x = __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
        else
          x = __uint_as_float(w[e]);
        hg.h[m][kPer * c + e] = x;
      }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += hg.h[m][i];
    hg.hsum[m] = s;
  }
}

template <int MAXG>
__device__ __forceinline__ float int4_group_dot(const uint4& qv, float sg,
                                                const HGroups<MAXG>& hg, int m, float acc) {
  const uint32_t w4[4] = {qv.x ^ 0x88888888u, qv.y ^ 0x88888888u, qv.z ^ 0x88888888u,
                          qv.w ^ 0x88888888u};
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = w4[j] & 0x0F0F0F0Fu;         // elements 8j+0, +2, +4, +6
    const uint32_t hi = (w4[j] >> 4) & 0x0F0F0F0Fu;  // elements 8j+1, +3, +5, +7
    t = fmaf((float)(lo & 0xFFu), hg.h[m][8 * j + 0], t);
    t = fmaf((float)(hi & 0xFFu), hg.h[m][8 * j + 1], t);
    t = fmaf((float)((lo >> 8) & 0xFFu), hg.h[m][8 * j + 2], t);
    t = fmaf((float)((hi >> 8) & 0xFFu), hg.h[m][8 * j + 3], t);
    t = fmaf((float)((lo >> 16) & 0xFFu), hg.h[m][8 * j + 4], t);
    t = fmaf((float)((hi >> 16) & 0xFFu), hg.h[m][8 * j + 5], t);
    t = fmaf((float)(lo >> 24), hg.h[m][8 * j + 6], t);
    t = fmaf((float)(hi >> 24), hg.h[m][8 * j + 7], t);
  }
  return fmaf(sg, fmaf(-8.f, hg.hsum[m], t), acc);
}

// INT8 (the W8A16 configuration): one group is 32 bytes, two 16-byte loads;
// bytes become u = q + 128 (xor 0x80 each), converted as unsigned bytes, and
// sum q h = sum u h - 128 sum_g h.
template <int MAXG>
__device__ __forceinline__ float int8_group_dot(const uint4& q0, const uint4& q1, float sg,
                                                const HGroups<MAXG>& hg, int m, float acc) {
  const uint32_t w8[8] = {q0.x ^ 0x80808080u, q0.y ^ 0x80808080u, q0.z ^ 0x80808080u,
                          q0.w ^ 0x80808080u, q1.x ^ 0x80808080u, q1.y ^ 0x80808080u,
                          q1.z ^ 0x80808080u, q1.w ^ 0x80808080u};
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // dword j holds elements 4j .. 4j + 3
    t = fmaf((float)(w8[j] & 0xFFu), hg.h[m][4 * j + 0], t);
    t = fmaf((float)((w8[j] >> 8) & 0xFFu), hg.h[m][4 * j + 1], t);
    t = fmaf((float)((w8[j] >> 16) & 0xFFu), hg.h[m][4 * j + 2], t);
    t = fmaf((float)(w8[j] >> 24), hg.h[m][4 * j + 3], t);
  }
  return fmaf(sg, fmaf(-128.f, hg.hsum[m], t), acc);
}

// Stage-1 scores of g32-quantised centroid rows (BITS = 4: packed nibbles,
// d/2 bytes per row; BITS = 8: int8, d bytes per row) against NQ queries'
// register-resident groups.  Lane l owns groups l, l + 64, ...; two rows'
// loads are issued before any math.
template <int BITS, int MAXG, int NQ, typename Sink>
__device__ __forceinline__ void wave_rows_q(const uint8_t* __restrict__ Q,
                                            const uint16_t* __restrict__ SG, int d, int lane,
                                            const HGroups<MAXG> (&hg)[NQ], int nq,
                                            int64_t r_begin, int64_t r_end, int64_t stride,
                                            Sink sink) {
  static_assert(BITS == 4 || BITS == 8, "INT4 or INT8 codes");
  constexpr int L = BITS / 4;  // 16-byte loads per group
  constexpr uint32_t kZero = BITS == 4 ? 0x88888888u : 0x80808080u;  // q = 0 after the offset
  const int G = d / 32;
  const int64_t row_bytes = (int64_t)d * BITS / 8;
#pragma unroll 1
  for (int64_t r = r_begin; r < r_end; r += 2 * stride) {
    const int64_t rb = r + stride;
    const bool okb = rb < r_end;
    const uint4* qa = reinterpret_cast<const uint4*>(Q + r * row_bytes);
    const uint4* qb = reinterpret_cast<const uint4*>(Q + (okb ? rb : r) * row_bytes);
    uint4 va[MAXG][L], vb[MAXG][L];
    float sa[MAXG], sb[MAXG];
#pragma unroll
    for (int m = 0; m < MAXG; ++m) {
      const int g = lane + 64 * m;
      const bool ok = g < G;
#pragma unroll
      for (int j = 0; j < L; ++j) {
        va[m][j] = ok ? qa[g * L + j] : uint4{kZero, kZero, kZero, kZero};
        vb[m][j] = (ok && okb) ? qb[g * L + j] : uint4{kZero, kZero, kZero, kZero};
      }
      sa[m] = ok ? __half2float(__ushort_as_half(SG[r * G + g])) : 0.f;
      sb[m] = (ok && okb) ? __half2float(__ushort_as_half(SG[rb * G + g])) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q >= nq) break;
      float acc_a = 0.f, acc_b = 0.f;
#pragma unroll
      for (int m = 0; m < MAXG; ++m) {
        if constexpr (BITS == 4) {
          acc_a = int4_group_dot<MAXG>(va[m][0], sa[m], hg[q], m, acc_a);
          acc_b = int4_group_dot<MAXG>(vb[m][0], sb[m], hg[q], m, acc_b);
        } else {
          acc_a = int8_group_dot<MAXG>(va[m][0], va[m][L - 1], sa[m], hg[q], m, acc_a);
          acc_b = int8_group_dot<MAXG>(vb[m][0], vb[m][L - 1], sb[m], hg[q], m, acc_b);
        }
      }
      acc_a = wave_sum(acc_a);
      acc_b = wave_sum(acc_b);
      sink(q, r, r, acc_a);
      if (okb) sink(q, rb, rb, acc_b);
    }
  }
}

// ======================================================================
// Epilogue helpers: fold one (row, z) into a running Part; merge Parts
// across the waves of a workgroup.
// ======================================================================
__device__ __forceinline__ Part part_of(float z, int32_t t, int token_sample, float tprime,
                                        uint64_t seed, uint32_t row) {
  float key = z;
  if (token_sample) key = z / tprime + gumbel_at(seed, row, (uint32_t)t, 1u);
  return Part{key, z, z / tprime, 1.f, t};
}

// A wave's running partial over rows whose (z, token) arrive one at a time,
// uniform across the wave.  A sampled token's key needs its Gumbel noise (a
// Philox block and two logarithms): drawn by the whole wave for each row it
// costs as much as 64 draws.  So with token sampling row i is parked in lane
// i % 64, and every 64 rows (and at the end) each lane draws for its own row
// and merges it into its own running partial; the lanes are merged at the
// end.  The token and its logit do not depend on the merge order; the LSE's
// rounding does.  Without token sampling a row's partial is merged at once.
struct LaneParts {
  Part acc;  // this lane's running partial (sampling) or the wave's (greedy)
  float z;   // the row parked in this lane
  int32_t t;
  int n;     // rows parked since the last draw (uniform)
};

__device__ __forceinline__ LaneParts lane_parts_empty() {
  return LaneParts{part_empty(), 0.f, 0, 0};
}

__device__ __forceinline__ void lane_parts_add(LaneParts& lp, float z, int32_t t, int token_sample,
                                               float tprime, uint64_t seed, uint32_t row) {
  if (!token_sample) {
    lp.acc = part_merge(lp.acc, part_of(z, t, 0, tprime, seed, row));
    return;
  }
  if ((int)(threadIdx.x & 63) == lp.n) {
    lp.z = z;
    lp.t = t;
  }
  if (++lp.n == 64) {
    lp.acc = part_merge(lp.acc, part_of(lp.z, lp.t, 1, tprime, seed, row));
    lp.n = 0;
  }
}

// The wave's partial (uniform).
__device__ __forceinline__ Part lane_parts_finish(LaneParts& lp, int token_sample, float tprime,
                                                  uint64_t seed, uint32_t row) {
  if (!token_sample) return lp.acc;
  if ((int)(threadIdx.x & 63) < lp.n) lp.acc = part_merge(lp.acc, part_of(lp.z, lp.t, 1, tprime, seed, row));
  lp.n = 0;
  return wave_merge_part(lp.acc);
}

// Merge the NWAVES per-wave Parts of each of nq queries held by lane 0s;
// thread q (< nq) returns the workgroup Part of query q.
template <int NWAVES, int NQ>
__device__ __forceinline__ Part block_merge_parts(const Part (&part)[NQ], int nq, Part* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) sh[wave * NQ + q] = part[q];
  }
  __syncthreads();
  Part acc = part_empty();
  if constexpr (NQ == 1 && NWAVES <= 16) {
    // one query: lanes 0..15 of wave 0 merge the wave partials as a DPP tree
    // within their row (4 levels, fixed pattern); thread 0 returns it
    if (wave == 0) {
      acc = lane < NWAVES ? sh[lane] : part_empty();
      acc = part_merge(acc, dpp_part<0xB1>(acc));   // quad_perm [1,0,3,2]
      acc = part_merge(acc, dpp_part<0x4E>(acc));   // quad_perm [2,3,0,1]
      acc = part_merge(acc, dpp_part<0x141>(acc));  // row_half_mirror
      acc = part_merge(acc, dpp_part<0x140>(acc));  // row_mirror
    }
    return acc;
  }
  if ((int)threadIdx.x < nq) {
    const int q = threadIdx.x;
    acc = sh[q];
    for (int w = 1; w < NWAVES; ++w) acc = part_merge(acc, sh[w * NQ + q]);
  }
  return acc;
}

// ======================================================================
// Probe selection (explainer §1.2.2 top-p, §1.2.3 multinomial probes), one
// 1024-thread workgroup per query.  Thread t holds the keys of clusters
// k = t + 1024 i (i < KP), so consecutive threads read consecutive scores.
// The result is a bitset of the p chosen clusters in LDS (the p largest keys,
// ties to the smaller id).
//
// Fast path: a threshold tau is placed from the keys' mean and standard
// deviation (a normal-tail quantile for a little more than p keys) and the
// keys above it are compacted into per-wave candidate lists.  If there are at
// least p of them and no list overflowed, the exact selection runs over the
// candidates only; otherwise over all keys.  Either way the selection is an
// exact radix select on order-preserving 32-bit images of the keys, taken
// relative to the smallest image in play: a histogram of the top 11 bits of
// the range and a suffix scan locate the digit holding the p-th key, keys
// with a larger digit are taken, smaller ones dropped, and the keys sharing
// the boundary digit go on to the next 11 bits.  A round stops as soon as
// the whole boundary digit is taken; keys still tied after the last bits are
// bit-identical, and the smallest ids among them are taken.
// ======================================================================
constexpr int kSelThreads = 1024;  // workgroup size of a selection
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelBins = 2048;
constexpr int kSelMaxC = 16384;
constexpr int kCandPerWave = 128;
constexpr int kCandMax = kCandPerWave * kSelWaves;

struct SelShared {
  int hist[kSelBins];
  uint32_t selbits[kSelMaxC / 32];
  uint32_t tiebits[kSelMaxC / 32];
  uint32_t cand_v[kCandMax];
  int cand_id[kCandMax];
  float red[3][kSelWaves];
  int wcnt[kSelWaves];
  int red_scan[kSelWaves];
  int red_out[kSelWaves];
  int beta, above, cnt;
  float tau, kmax;
};

// Keys per thread for c clusters over 1024 threads (1, 2, 8 or 16).
inline int sel_keys_per_thread(int64_t c) {
  const int64_t k = (c + kSelThreads - 1) / kSelThreads;
  return k <= 1 ? 1 : k <= 2 ? 2 : k <= 8 ? 8 : k <= 16 ? 16 : -1;
}

// Selection keys saturate: NaN is taken as -FLT_MAX and +-inf as +-FLT_MAX.
__device__ __forceinline__ float saturate_key(float x) {
  return isnan(x) ? -FLT_MAX : fminf(fmaxf(x, -FLT_MAX), FLT_MAX);
}

// Order-preserving image of a (saturated) key: a larger float gives a larger
// integer, and -0 maps like +0 so that equal floats give equal images.
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t b = x == 0.f ? 0u : __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum over each row of 16 lanes (row_shr 1, 2, 4, 8 with
// zero fill).
__device__ __forceinline__ int row_inclusive_scan(int x) {
  x += dpp_i<0x111>(x);
  x += dpp_i<0x112>(x);
  x += dpp_i<0x114>(x);
  x += dpp_i<0x118>(x);
  return x;
}

// Exclusive prefix sum of x over the 1024 threads (index order) through one
// LDS exchange in `red` (one barrier); *total gets the sum.  The 16 wave
// totals are combined lane-parallel (lanes 0..15 of every wave).
__device__ __forceinline__ int block_exclusive_scan(int x, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(x, lane);
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  const int t = row_inclusive_scan(lane < kSelWaves ? red[lane] : 0);
  *total = __builtin_amdgcn_readlane(t, kSelWaves - 1);
  const int before = wave > 0 ? __builtin_amdgcn_readlane(t, wave - 1) : 0;
  return before + inc - x;
}

// OR the bits of key slot i (clusters k = tid + 1024 i) into a bitset with
// one ballot per wave: a wave's 64 lanes own 64 consecutive clusters.
template <int KP>
__device__ __forceinline__ void ballot_bits(uint32_t mask, uint32_t* bits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const unsigned long long b = __ballot((mask >> i) & 1u);
    if (lane == 0 && b) {
      const int word = (kSelThreads * i + 64 * wave) >> 5;
      if ((uint32_t)b) atomicOr(&bits[word], (uint32_t)b);
      if ((uint32_t)(b >> 32)) atomicOr(&bits[word + 1], (uint32_t)(b >> 32));
    }
  }
}

// Clear the selection's LDS state; a barrier must follow before the
// selection proper.
__device__ __forceinline__ void select_clear(SelShared& sh) {
  const int tid = threadIdx.x;
  sh.hist[2 * tid] = 0;
  sh.hist[2 * tid + 1] = 0;
  if (tid < kSelMaxC / 32) {
    sh.selbits[tid] = 0u;
    sh.tiebits[tid] = 0u;
  }
}

// One radix round over the entries flagged in `cand`: histogram of the digit
// (v >> shift) & 2047, suffix scan, and the digit beta holding the need-th
// largest entry, with the count above it and its own count.  Leaves the
// histogram cleared.
template <int N>
__device__ __forceinline__ void radix_round(const uint32_t (&v)[N], uint32_t cand, int shift,
                                            int need, SelShared& sh, int* beta, int* above,
                                            int* cnt) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (cand & (1u << i)) atomicAdd(&sh.hist[(v[i] >> shift) & (kSelBins - 1)], 1);
  __syncthreads();
  // thread t owns digits 2047 - 2t and 2046 - 2t (suffix order)
  const int j0 = kSelBins - 1 - 2 * tid;
  const int h0 = sh.hist[j0], h1 = sh.hist[j0 - 1];
  sh.hist[j0] = 0;
  sh.hist[j0 - 1] = 0;
  int tot;
  const int before = block_exclusive_scan(h0 + h1, sh.red_scan, &tot);
  if (before < need && before + h0 >= need) {
    sh.beta = j0;
    sh.above = before;
    sh.cnt = h0;
  } else if (before + h0 < need && before + h0 + h1 >= need) {
    sh.beta = j0 - 1;
    sh.above = before + h0;
    sh.cnt = h1;
  }
  __syncthreads();
  *beta = sh.beta;
  *above = sh.above;
  *cnt = sh.cnt;
}

// Radix rounds over entries v (images relative to the smallest in play,
// span = the largest such value): narrows `cand` to the boundary entries and
// sets bits in `sel` for entries taken.  Returns how many of the boundary
// entries are still to be taken (> 0 only when they are all equal).
template <int N>
__device__ __forceinline__ int radix_rounds(const uint32_t (&v)[N], uint32_t span, int need,
                                            uint32_t& cand, uint32_t& sel, SelShared& sh) {
  const int bits = span ? 32 - __clz((int)span) : 0;
  int shift = bits > 11 ? bits - 11 : 0;
  for (int round = 0; round < 3 && need > 0; ++round) {
    int beta, above, cnt;
    radix_round<N>(v, cand, shift, need, sh, &beta, &above, &cnt);
    FH_TRACE(10 + round);
    if (round == 0 && threadIdx.x == 0 && blockIdx.x < 4096) g_fh_trace_cnt(cnt);
    need -= above;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t bit = cand & (1u << i);
      const int dig = (int)((v[i] >> shift) & (kSelBins - 1));
      if (bit && dig > beta) sel |= bit;
      if (bit && dig != beta) cand &= ~bit;
    }
    if (cnt == need) {  // the whole boundary digit is taken
      sel |= cand;
      cand = 0u;
      need = 0;
    }
    if (shift == 0) break;
    shift = shift > 11 ? shift - 11 : 0;
  }
  return need;
}

// Add the `need` smallest ids flagged in sh.tiebits to sh.selbits.  Thread t
// scans clusters [t*KP, t*KP + KP).  Call after a barrier; ends with one.
template <int KP>
__device__ __forceinline__ void take_ties(int c, int need, SelShared& sh) {
  const int b0 = threadIdx.x * KP;
  uint32_t tie_mine = 0u;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int k = b0 + i;
    if (k < c && (sh.tiebits[k >> 5] & (1u << (k & 31)))) tie_mine |= 1u << i;
  }
  int tot;
  int rank = block_exclusive_scan(__popc(tie_mine), sh.red_scan, &tot);
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if (tie_mine & (1u << i)) {
      const int k = b0 + i;
      if (rank < need) atomicOr(&sh.selbits[k >> 5], 1u << (k & 31));
      ++rank;
    }
  }
  __syncthreads();
}

// Exact selection over all keys (thread t holds clusters t + 1024 i).
template <int KP>
__device__ __forceinline__ void select_all(const float (&x)[KP], int c, int p, float xmin,
                                           float xmax, SelShared& sh) {
  const int tid = threadIdx.x;
  uint32_t cand = 0u, sel = 0u;
  uint32_t v[KP];
  const uint32_t lo = ordered_bits(xmin);
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if (tid + kSelThreads * i < c) cand |= 1u << i;
    v[i] = ordered_bits(x[i]) - lo;
  }
  const int need = radix_rounds<KP>(v, ordered_bits(xmax) - lo, p, cand, sel, sh);
  ballot_bits<KP>(sel, sh.selbits);
  if (need > 0) ballot_bits<KP>(cand, sh.tiebits);
  __syncthreads();
  if (need > 0) take_ties<KP>(c, need, sh);
}

// Candidate target for the fast path: a few more than p keys above tau.
__host__ __device__ inline int select_target(int p) { return p + p / 4 + 64; }
__host__ __device__ inline bool select_fast_ok(int c, int p) {
  return p < c && 2 * select_target(p) <= c && select_target(p) <= kCandMax * 3 / 4;
}

// The p largest of the c keys x (thread t holds clusters t + 1024 i; keys
// saturated; slots past c hold -FLT_MAX) into sh.selbits.  `zq` is the standard-normal quantile with
// P(Z > zq) = select_target(p) / c (used when select_fast_ok(c, p)).  Run by
// the whole workgroup after select_clear and a barrier; ends with a barrier.
template <int KP>
__device__ __forceinline__ void select_bits(const float (&x)[KP], int c, int p, float zq,
                                            SelShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  FH_TRACE(9);
  if (p >= c) {
    uint32_t all = 0u;
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if (tid + kSelThreads * i < c) all |= 1u << i;
    ballot_bits<KP>(all, sh.selbits);
    __syncthreads();
    return;
  }
  if (select_fast_ok(c, p)) {
    // largest key over all (padding is -FLT_MAX); mean and spread from the
    // first 1024 keys
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < KP; ++i) mx = x[i] > mx ? x[i] : mx;
    const bool s0 = tid < c;
    float sum = s0 ? x[0] : 0.f, sq = s0 ? x[0] * x[0] : 0.f;
    mx = wave_max(mx);
    sum = wave_sum(sum);
    sq = wave_sum(sq);
    if (lane == 0) {
      sh.red[0][wave] = mx;
      sh.red[1][wave] = sum;
      sh.red[2][wave] = sq;
    }
    __syncthreads();
    const bool rl = lane < kSelWaves;
    if (wave == 0) {
      // one wave combines the wave partials and places tau
      const float m0 = readlane_f(row_allreduce(rl ? sh.red[0][lane] : -FLT_MAX,
                                                [](float a, float b) { return fmaxf(a, b); }), 0);
      const float s0 = readlane_f(row_allreduce(rl ? sh.red[1][lane] : 0.f,
                                                [](float a, float b) { return a + b; }), 0);
      const float q0 = readlane_f(row_allreduce(rl ? sh.red[2][lane] : 0.f,
                                                [](float a, float b) { return a + b; }), 0);
      const float inv = 1.f / (float)min(c, kSelThreads);
      const float mean = s0 * inv;
      const float sd = sqrtf(fmaxf(q0 * inv - mean * mean, 0.f));
      // at least -FLT_MAX (also for a NaN or -inf estimate), so that padding
      // slots are never above it
      if (lane == 0) {
        sh.tau = fmaxf(mean + sd * zq, -FLT_MAX);
        sh.kmax = m0;
      }
    }
    __syncthreads();
    const float tau = sh.tau;
    mx = sh.kmax;
    const uint32_t lo = ordered_bits(tau);
    // compact the keys above tau into this wave's candidate list
    int wcount = 0;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int k = tid + kSelThreads * i;
      const bool take = x[i] > tau;
      const unsigned long long b = __ballot(take);
      if (b) {
        const int off = wcount + __builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        if (take && off < kCandPerWave) {
          sh.cand_v[wave * kCandPerWave + off] = ordered_bits(x[i]) - lo;
          sh.cand_id[wave * kCandPerWave + off] = k;
        }
        wcount += __popcll(b);
      }
    }
    if (lane == 0) sh.wcnt[wave] = wcount;
    __syncthreads();
    const int wc = rl ? sh.wcnt[lane] : 0;
    const int total = __builtin_amdgcn_readlane(row_inclusive_scan(wc), kSelWaves - 1);
    const bool overflow = __ballot(wc > kCandPerWave) != 0ull;
    if (!overflow && total >= p) {
      FH_TRACE(8);
      // this wave's list: entries lane and lane + 64
      const int n = __builtin_amdgcn_readlane(wc, wave);
      uint32_t v[2];
      int id[2];
      uint32_t cand = 0u, sel = 0u;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int slot = lane + 64 * e;
        v[e] = slot < n ? sh.cand_v[wave * kCandPerWave + slot] : 0u;
        id[e] = slot < n ? sh.cand_id[wave * kCandPerWave + slot] : 0;
        if (slot < n) cand |= 1u << e;
      }
      const int need = radix_rounds<2>(v, ordered_bits(mx) - lo, p, cand, sel, sh);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (sel & (1u << e)) atomicOr(&sh.selbits[id[e] >> 5], 1u << (id[e] & 31));
        if (need > 0 && (cand & (1u << e))) atomicOr(&sh.tiebits[id[e] >> 5], 1u << (id[e] & 31));
      }
      __syncthreads();
      if (need > 0) take_ties<KP>(c, need, sh);
      return;
    }
  }
  // exact selection over all keys, relative to the smallest
  float mn = FLT_MAX, mx = -FLT_MAX;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if (tid + kSelThreads * i < c) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  __syncthreads();  // sh.red may still be read above
  if (lane == 0) {
    sh.red[0][wave] = mn;
    sh.red[1][wave] = mx;
  }
  __syncthreads();
  const bool rl = lane < kSelWaves;
  mn = readlane_f(row_allreduce(rl ? sh.red[0][lane] : FLT_MAX,
                                [](float a, float b) { return fminf(a, b); }), 0);
  mx = readlane_f(row_allreduce(rl ? sh.red[1][lane] : -FLT_MAX,
                                [](float a, float b) { return fmaxf(a, b); }), 0);
  select_all<KP>(x, c, p, mn, mx, sh);
}

// Write the clusters flagged in sh.selbits in ascending id:
// emit(position, cluster).  Thread t reads clusters [t*KP, t*KP + KP).
template <int KP, typename Emit>
__device__ __forceinline__ void emit_selected(int c, Emit emit, SelShared& sh) {
  const int b0 = threadIdx.x * KP;
  uint32_t mine = 0u;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int k = b0 + i;
    if (k < c && (sh.selbits[k >> 5] & (1u << (k & 31)))) mine |= 1u << i;
  }
  int tot;
  int off = block_exclusive_scan(__popc(mine), sh.red_out, &tot);
#pragma unroll
  for (int i = 0; i < KP; ++i)
    if (mine & (1u << i)) emit(off++, b0 + i);
  FH_TRACE(13);
}

// ======================================================================
// Adaptive probe count (FlashHead explainer §1.2.2: the number of probes
// follows the distribution of h; §4.2: fewer probes for confident queries).
// Of the top pmax probes by selection key, keep the first n in key order
// (descending, ties to the smaller id) whose softmax(s/T) mass reaches tau of
// the total over all c clusters, n clamped to [pmin, pmax].  Every step has
// a fixed order (block trees, a bitonic network, a fixed scan), so the count
// is deterministic.  All helpers are called by all 1024 threads.
// ======================================================================
struct MassTotal {
  float M;  // max_k s_k / T
  float W;  // sum_k exp(s_k / T - M)
};

// Max (or sum) over the 1024 threads: waves first, then the 16 wave values
// in one row; the result is uniform.  `red` (16 floats) is free on return.
template <bool MAX>
__device__ __forceinline__ float block_reduce_f(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = MAX ? wave_max(x) : wave_sum(x);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float t = lane < kSelWaves ? red[lane] : (MAX ? -INFINITY : 0.f);
  t = MAX ? row_allreduce(t, [](float a, float b) { return fmaxf(a, b); })
          : row_allreduce(t, [](float a, float b) { return a + b; });
  const float r = readlane_f(t, 0);
  __syncthreads();
  return r;
}

// M and W of the scores s[k] of clusters k = tid + 1024 i (entries past c
// ignored).
template <int KP>
__device__ __forceinline__ MassTotal mass_total(const float (&s)[KP], int c, float temperature,
                                                float* red) {
  float xs[KP];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const bool live = (int)threadIdx.x + kSelThreads * i < c;
    xs[i] = live ? s[i] / temperature : -INFINITY;
    mx = fmaxf(mx, xs[i]);
  }
  MassTotal mt;
  mt.M = block_reduce_f<true>(mx, red);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < KP; ++i)
    acc += (int)threadIdx.x + kSelThreads * i < c ? __expf(xs[i] - mt.M) : 0.f;
  mt.W = block_reduce_f<false>(acc, red);
  return mt;
}

// The selection key of cluster k with score s: s, or s/T + G(seed, row, k, 0)
// for sampled probes, saturated (the key k_select and the batch-1 stage 1
// form).
__device__ __forceinline__ float probe_key(float s, int sample, float temperature, uint64_t seed,
                                           uint32_t row, int k) {
  if (sample) s = s / temperature + gumbel_at(seed, row, (uint32_t)k, 0u);
  return saturate_key(s);
}

// 64-bit sort image of (key, k): larger key first, then the smaller id.  Every
// image is above 0, which pads a sort.
__device__ __forceinline__ unsigned long long probe_sort_key(float key, int k) {
  return ((unsigned long long)ordered_bits(key) << 32) |
         (unsigned long long)(0xFFFFFFFFu - (uint32_t)k);
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p2 = 1;
  while (p2 < n) p2 <<= 1;
  return p2;
}

// Bitonic sort into descending order of P2 elements (P2 a power of two,
// <= 1024), one per thread: thread i holds element i in (key, val) and
// returns holding the i-th largest key with its val.  A compare-exchange at
// distance j < 64 stays inside the wave (lane shuffles, no barrier); only the
// steps with j >= 64 exchange through lds_key / lds_val ([P2] each), with a
// barrier on each side.  Called by all 1024 threads.
__device__ __forceinline__ void bitonic_sort_desc(unsigned long long& key, float& val, int P2,
                                                  unsigned long long* lds_key, float* lds_val) {
  const int i = threadIdx.x;
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      unsigned long long okey;
      float oval;
      if (j < 64) {
        const uint32_t lo = __shfl_xor((uint32_t)key, j);
        const uint32_t hi = __shfl_xor((uint32_t)(key >> 32), j);
        okey = ((unsigned long long)hi << 32) | lo;
        oval = __shfl_xor(val, j);
      } else {
        __syncthreads();  // the previous exchange's reads are done
        if (i < P2) {
          lds_key[i] = key;
          lds_val[i] = val;
        }
        __syncthreads();
        okey = i < P2 ? lds_key[i ^ j] : 0ull;
        oval = i < P2 ? lds_val[i ^ j] : 0.f;
      }
      // in a descending block (i & k) == 0 the lower index keeps the larger
      // element; in an ascending one, the smaller
      const bool lower = (i & j) == 0;
      const bool want_larger = ((i & k) == 0) == lower;
      const bool take = want_larger ? okey > key : okey < key;
      if (i < P2 && take) {
        key = okey;
        val = oval;
      }
    }
  }
}

// Inclusive prefix sum of x over the 1024 threads in index order (float; the
// same fixed pattern as block_exclusive_scan).
__device__ __forceinline__ float block_inclusive_scan_f(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x += dpp_f<0x111>(x);
  x += dpp_f<0x112>(x);
  x += dpp_f<0x114>(x);
  x += dpp_f<0x118>(x);
  const float t0 = readlane_f(x, 15), t1 = readlane_f(x, 31), t2 = readlane_f(x, 47);
  const int row = lane >> 4;
  x = x + (row >= 1 ? t0 : 0.f) + (row >= 2 ? t1 : 0.f) + (row >= 3 ? t2 : 0.f);
  if (lane == 63) red[wave] = x;
  __syncthreads();
  float t = lane < kSelWaves ? red[lane] : 0.f;
  t += dpp_f<0x111>(t);
  t += dpp_f<0x112>(t);
  t += dpp_f<0x114>(t);
  t += dpp_f<0x118>(t);
  const float before = wave > 0 ? readlane_f(t, wave - 1) : 0.f;
  __syncthreads();
  return before + x;
}

// Two cases settle the count without the sort, as the sorted scan would: if
// all p probes together hold less than tau W, every prefix falls short and
// n = p (the scan's last prefix is the same sum in another order, so the two
// can differ only where the total lies within rounding of tau W); if the top
// probe alone holds tau W (and pmin <= 1), the first prefix -- that same
// weight -- reaches it and n = 1.
// Each thread passes the weight sum of its own selected probes and the
// largest sort image among them with that probe's score.  Returns n (0: no
// fast case) and, for n = 1, the top probe's image in *top.
__device__ __forceinline__ int adaptive_fast(float wsel, unsigned long long best, float best_s,
                                             int p, int pmin, float tau, const MassTotal& mt,
                                             float temperature, float* redf,
                                             unsigned long long* redk, unsigned long long* top) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float Wsel = block_reduce_f<false>(wsel, redf);
  if (Wsel < tau * mt.W) return p;
  unsigned long long b = best;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)b, m);
    const uint32_t hi = __shfl_xor((uint32_t)(b >> 32), m);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    b = o > b ? o : b;
  }
  // the images are distinct: one lane holds the wave's largest
  if (best == b && b != 0ull) {
    redk[wave] = b;
    redf[wave] = best_s;
  } else if (lane == 0 && b == 0ull) {
    redk[wave] = 0ull;
  }
  __syncthreads();
  unsigned long long tb = 0ull;
  float ts = 0.f;
  for (int v = 0; v < kSelWaves; ++v)
    if (redk[v] > tb) {
      tb = redk[v];
      ts = redf[v];
    }
  __syncthreads();
  *top = tb;
  if (pmin <= 1 && tb != 0ull && __expf(ts / temperature - mt.M) >= tau * mt.W) return 1;
  return 0;
}

// The count n from the pmax probes sorted by bitonic_sort_desc (thread t
// holding the t-th: its sort image skey and score s): thread t's id goes to
// *id (else -1), the weights exp(s/T - M) are scanned in key order, and
// n - 1 is the number of prefixes short of tau W.
__device__ __forceinline__ int adaptive_count(unsigned long long skey, float s, int pmax,
                                              int pmin, float tau, const MassTotal& mt,
                                              float temperature, float* redf, int* red_cnt,
                                              int* id) {
  const int t = threadIdx.x;
  float w = 0.f;
  *id = -1;
  if (t < pmax) {
    *id = (int)(0xFFFFFFFFu - (uint32_t)(skey & 0xFFFFFFFFull));
    w = __expf(s / temperature - mt.M);
  }
  const float cum = block_inclusive_scan_f(w, redf);
  int below;
  (void)block_exclusive_scan(t < pmax && cum < tau * mt.W ? 1 : 0, red_cnt, &below);
  return min(max(below + 1, pmin), pmax);
}

// ======================================================================
// Finisher: merge n Parts in a fixed order (threads stride, then a tree).
// ======================================================================
// Merge n Parts: each thread folds a strided subset in index order (eight
// loads in flight, then eight merges: one memory round trip per eight
// partials, not per partial; past n the slots hold part_empty(), which
// part_merge leaves the running partial unchanged by, bit for bit), the waves
// merge their lanes, and thread 0 merges the waves in order.
template <int NT>
__device__ __forceinline__ Part merge_parts_block(const Part* __restrict__ pq, int n, Part* sh) {
  Part acc = part_empty();
  for (int i = threadIdx.x; i < n; i += 8 * NT) {
    Part x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = i + u * NT < n ? pq[i + u * NT] : part_empty();
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = part_merge(acc, x[u]);
  }
  acc = wave_merge_part(acc);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  Part r = sh[0];
  for (int w = 1; w < NT / 64; ++w) r = part_merge(r, sh[w]);
  return r;
}

__device__ __forceinline__ void write_outputs(const Part& r, int q, int32_t* out_token,
                                              float* out_logit, float* out_lse) {
  if (out_token) out_token[q] = r.id;
  if (out_logit) out_logit[q] = r.z;
  if (out_lse) out_lse[q] = r.m + logf(r.s);
}

}  // namespace fh
