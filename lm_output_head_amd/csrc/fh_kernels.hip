// FlashHead kernels for gfx950 (MI355X): INT4 centroid quantisation, row
// GEMV (stage-1 scores, stage-2 gather-score, dense head) with a fused
// max / log-sum-exp / Gumbel epilogue, probe selection, the finisher, and a
// single-launch fused kernel for batch-1 decode.
//
// Sources (page title and section): FlashHead technical explainer
// (framerc.cn) §1.1, §1.2.1-§1.2.4, §2.2.2, §2.3; "FlashHead: Efficient
// Drop-In Replacement for the Classification Head in Language Model
// Inference" (arXiv 2603.14591), abstract.

#include <algorithm>

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "fh_device.hpp"
#include "fh_internal.hpp"

namespace fh {

// Optional per-workgroup phase timestamps for performance probes (off in
// the library build): slot s, workgroup w -> wall clock at phase s.
#ifdef FH_PHASE_TRACE
__device__ unsigned long long g_fh_trace[16][4096];
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
// INT4 g32 quantisation of the centroids (explainer §1.2.4, §2.3).
// One thread per (row, group of 32 consecutive elements).  sigma is
// fp16(amax / 7) with an IEEE float32 division and round-to-nearest-even to
// fp16; q = clamp(rint(x / sigma), -7, 7) with float32 division (rint ties
// to even); q = 0 where sigma = 0.  Nibbles are packed two's-complement,
// element 2m in the low nibble of byte m.  *bad is set if a scale overflows.
// ======================================================================
template <typename T>
__global__ __launch_bounds__(256) void k_quant_int4(const T* __restrict__ C, int64_t c, int d,
                                                    uint8_t* __restrict__ qout,
                                                    uint16_t* __restrict__ sout,
                                                    int* __restrict__ bad) {
  const int G = d / 32;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= c * G) return;
  const int64_t row = gid / G;
  const int g = (int)(gid % G);
  const int64_t base = row * d + (int64_t)g * 32;
  float x[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    x[i] = load_elem<T>(C, base + i);
    amax = fmaxf(amax, fabsf(x[i]));
  }
  const __half hs = __float2half_rn(amax / 7.0f);
  const float s = __half2float(hs);
  if (!isfinite(s)) atomicOr(bad, 1);
  uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int qi = 0;
    if (s > 0.f) qi = (int)fminf(fmaxf(rintf(x[i] / s), -7.f), 7.f);
    words[i >> 3] |= ((uint32_t)qi & 0xFu) << (4 * (i & 7));
  }
  uint4* dst = reinterpret_cast<uint4*>(qout + row * (d / 2) + (int64_t)g * 16);
  *dst = uint4{words[0], words[1], words[2], words[3]};
  sout[row * G + g] = __half_as_ushort(hs);
}

// ======================================================================
// Wave-level row GEMV.
//
// A wavefront computes z = M[src(r)] . h_q for rows r = r_begin, r_begin +
// stride, ... < r_end and NQ queries.  Lane l owns the 16-byte chunks l,
// l+64, ... of a row (MAXM of them at most), so a row is read as fully
// coalesced 16-byte loads and the lane's slice of each h stays in registers
// (hv) for all rows.  Two rows' loads are issued before any math.  `sink` is
// called by every lane with the wave-uniform result of each (row, query).
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

template <typename T, int MAXM, int NQ, typename SrcOf, typename Sink>
__device__ __forceinline__ void wave_rows(const T* __restrict__ M, int d, int lane,
                                          const uint4 (&hv)[NQ][MAXM], int nq, int64_t r_begin,
                                          int64_t r_end, int64_t stride, SrcOf src_of,
                                          Sink sink) {
  const int nch = d / Chunk<T>::kElems;
#pragma unroll 1
  for (int64_t r = r_begin; r < r_end; r += 2 * stride) {
    const int64_t rb = r + stride;
    const bool okb = rb < r_end;
    const int64_t sa = src_of(r);
    const int64_t sb = okb ? src_of(rb) : sa;
    const uint4* ra_p = reinterpret_cast<const uint4*>(M + sa * d);
    const uint4* rb_p = reinterpret_cast<const uint4*>(M + sb * d);
    uint4 ma[MAXM], mb[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      const int ch = lane + 64 * m;
      ma[m] = ch < nch ? ra_p[ch] : uint4{0u, 0u, 0u, 0u};
      mb[m] = (okb && ch < nch) ? rb_p[ch] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q >= nq) break;
      float acc_a = 0.f, acc_b = 0.f;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        acc_a = Chunk<T>::dot(ma[m], hv[q][m], acc_a);
        acc_b = Chunk<T>::dot(mb[m], hv[q][m], acc_b);
      }
      acc_a = wave_sum(acc_a);
      acc_b = wave_sum(acc_b);
      sink(q, r, sa, acc_a);
      if (okb) sink(q, rb, sb, acc_b);
    }
  }
}

// ======================================================================
// Wave-level INT4 stage-1 GEMV: s[k] = sum_g sigma[k, g] sum_{i in g} q h.
// Lane l owns groups l, l+64, ...: one 16-byte load is one group's 32
// nibbles.  Nibbles become unsigned bytes u = q + 8 (xor 0x88888888, two
// masks), cvt_f32_ubyte converts them, and sum q h = sum u h - 8 sum_g h
// removes the offset with the group sums of h.
// ======================================================================
template <int MAXG>
struct HGroups {
  float h[MAXG][32];
  float hsum[MAXG];
};

template <typename T, int MAXG>
__device__ __forceinline__ void load_hgroups(const T* h, int G, int lane, HGroups<MAXG>& hg) {
#pragma unroll
  for (int m = 0; m < MAXG; ++m) {
    const int g = lane + 64 * m;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      hg.h[m][i] = g < G ? load_elem<T>(h, (int64_t)g * 32 + i) : 0.f;
      s += hg.h[m][i];
    }
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

template <int MAXG, int NQ, typename Sink>
__device__ __forceinline__ void wave_rows_int4(const uint8_t* __restrict__ Q,
                                               const uint16_t* __restrict__ SG, int d, int lane,
                                               const HGroups<MAXG> (&hg)[NQ], int nq,
                                               int64_t r_begin, int64_t r_end, int64_t stride,
                                               Sink sink) {
  const int G = d / 32;
#pragma unroll 1
  for (int64_t r = r_begin; r < r_end; r += 2 * stride) {
    const int64_t rb = r + stride;
    const bool okb = rb < r_end;
    const uint4* qa = reinterpret_cast<const uint4*>(Q + r * (d / 2));
    const uint4* qb = reinterpret_cast<const uint4*>(Q + (okb ? rb : r) * (d / 2));
    uint4 va[MAXG], vb[MAXG];
    float sa[MAXG], sb[MAXG];
#pragma unroll
    for (int m = 0; m < MAXG; ++m) {
      const int g = lane + 64 * m;
      const bool ok = g < G;
      va[m] = ok ? qa[g] : uint4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
      vb[m] = (ok && okb) ? qb[g] : uint4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
      sa[m] = ok ? __half2float(__ushort_as_half(SG[r * G + g])) : 0.f;
      sb[m] = (ok && okb) ? __half2float(__ushort_as_half(SG[rb * G + g])) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q >= nq) break;
      float acc_a = 0.f, acc_b = 0.f;
#pragma unroll
      for (int m = 0; m < MAXG; ++m) {
        acc_a = int4_group_dot<MAXG>(va[m], sa[m], hg[q], m, acc_a);
        acc_b = int4_group_dot<MAXG>(vb[m], sb[m], hg[q], m, acc_b);
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
  if ((int)threadIdx.x < nq) {
    const int q = threadIdx.x;
    acc = sh[q];
    for (int w = 1; w < NWAVES; ++w) acc = part_merge(acc, sh[w * NQ + q]);
  }
  return acc;
}

// ======================================================================
// Multi-launch path: row GEMV kernel (any B).
//   GATHER = false: row r is M's row r (stage 1 over C; the dense head over E).
//   GATHER = true : row r of query q is token t = C2T[S[q, r / b], r % b]
//                   of E (stage 2, explainer §1.2.4); one query per grid row.
//   EPI: fold each (z, t) into per-query Parts; one Part per workgroup and
//        query goes to parts[q * gridDim.x + blockIdx.x].
// ======================================================================
struct RowsArgs {
  const void* M;
  int64_t nrows;  // rows per query (c, v, or p*b)
  int d;
  const int32_t* c2t;
  int bsz;
  const int32_t* S;
  int ldS;
  const void* H;
  int B;
  float* out_vals;  // [B x ld_vals] or null
  int64_t ld_vals;
  int32_t* out_ids;  // [B x ld_vals] or null (GATHER only)
  int token_sample;
  float tprime;  // T' (1 unless tokens are sampled)
  uint64_t seed;
  Part* parts;  // [B x gridDim.x] (EPI)
};

template <typename T, int MAXM, int NQ, int RPW, bool GATHER, bool EPI>
__global__ __launch_bounds__(256) void k_rows(RowsArgs a) {
  __shared__ Part sh[4 * NQ];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nch = a.d / Chunk<T>::kElems;
  const int q0 = blockIdx.y * NQ;
  const int nq = min(NQ, a.B - q0);
  const T* Hp = static_cast<const T*>(a.H);
  uint4 hv[NQ][MAXM];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    load_hslice<T, MAXM>(Hp + (int64_t)(q0 + min(q, nq - 1)) * a.d, nch, lane, hv[q]);
  Part part[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) part[q] = part_empty();

  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
  const int64_t r1 = min(r0 + RPW, a.nrows);
  const int32_t* Sq = GATHER ? a.S + (int64_t)q0 * a.ldS : nullptr;
  auto src_of = [&](int64_t r) -> int64_t {
    if (GATHER) return a.c2t[(int64_t)Sq[r / a.bsz] * a.bsz + r % a.bsz];
    return r;
  };
  auto sink = [&](int q, int64_t r, int64_t src, float z) {
    const int64_t oq = q0 + q;
    if (lane == 0) {
      if (a.out_vals) a.out_vals[oq * a.ld_vals + r] = z;
      if (GATHER && a.out_ids) a.out_ids[oq * a.ld_vals + r] = (int32_t)src;
    }
    if (EPI)
      part[q] = part_merge(part[q], part_of(z, (int32_t)src, a.token_sample, a.tprime, a.seed,
                                            (uint32_t)oq));
  };
  wave_rows<T, MAXM, NQ>(static_cast<const T*>(a.M), a.d, lane, hv, nq, r0, r1, 1, src_of, sink);
  if (EPI) {
    const Part wg = block_merge_parts<4, NQ>(part, nq, sh);
    if ((int)threadIdx.x < nq) a.parts[(int64_t)(q0 + threadIdx.x) * gridDim.x + blockIdx.x] = wg;
  }
}

template <typename T, int MAXG, int NQ, int RPW>
__global__ __launch_bounds__(256) void k_score_int4(const uint8_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ SG, int64_t c,
                                                    int d, const T* __restrict__ H, int B,
                                                    float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q0 = blockIdx.y * NQ;
  const int nq = min(NQ, B - q0);
  HGroups<MAXG> hg[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    load_hgroups<T, MAXG>(H + (int64_t)(q0 + min(q, nq - 1)) * d, d / 32, lane, hg[q]);
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
  const int64_t r1 = min(r0 + RPW, c);
  auto sink = [&](int q, int64_t r, int64_t, float s) {
    if (lane == 0) out[(int64_t)(q0 + q) * c + r] = s;
  };
  wave_rows_int4<MAXG, NQ>(Q, SG, d, lane, hg, nq, r0, r1, 1, sink);
}

// ======================================================================
// Probe selection (explainer §1.2.2 top-p, §1.2.3 multinomial probes), one
// 1024-thread workgroup per query.
//
// Thread t holds the keys of clusters [t*KPT, t*KPT + KPT) in registers:
// key = s (TOPK), or s/T + G(seed, row, k, 0) (SAMPLE: the top p of
// Gumbel-perturbed keys are p draws without replacement from softmax(s/T)).
// The p-th largest key is located by bucketing: the active key range
// [lo, hi] is cut into 2048 equal buckets (a monotone map sending lo to
// bucket 0 and hi to bucket 2047), a histogram and a suffix scan find the
// bucket holding the boundary, keys above it are taken and keys below it
// dropped.  A small boundary bucket (<= 1024 keys) is resolved exactly by
// ranking its keys against each other (key desc, id asc); a large one
// becomes the next range.  When all remaining keys are equal the smallest
// ids are taken.  The chosen ids are written ascending with a block prefix
// sum.  Non-finite keys are saturated to +-FLT_MAX (NaN to -FLT_MAX).
// ======================================================================
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelBins = 2048;
constexpr int kRankMax = 1024;

struct SelShared {
  int hist[kSelBins];
  float cand_key[kRankMax];
  int cand_id[kRankMax];
  uint32_t selbits[16384 / 32];
  uint32_t tiebits[16384 / 32];
  float red[4][kSelWaves];
  int red_scan[kSelWaves];
  int red_out[kSelWaves];
  int beta, above, cnt, ncand;
};

struct KeyStats {
  float lo, hi, mean, sd;
};

// Block-wide min, max, mean and standard deviation of the active keys
// through one LDS exchange (one barrier).
__device__ __forceinline__ KeyStats block_stats(float mn, float mx, float sum, float sq, int n,
                                                SelShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  mn = wave_min(mn);
  mx = wave_max(mx);
  sum = wave_sum(sum);
  sq = wave_sum(sq);
  if (lane == 0) {
    sh.red[0][wave] = mn;
    sh.red[1][wave] = mx;
    sh.red[2][wave] = sum;
    sh.red[3][wave] = sq;
  }
  __syncthreads();
  KeyStats r{sh.red[0][0], sh.red[1][0], sh.red[2][0], sh.red[3][0]};
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) {
    r.lo = fminf(r.lo, sh.red[0][w]);
    r.hi = fmaxf(r.hi, sh.red[1][w]);
    r.mean += sh.red[2][w];
    r.sd += sh.red[3][w];
  }
  const float inv = n > 0 ? 1.f / (float)n : 0.f;
  r.mean *= inv;
  r.sd = sqrtf(fmaxf(r.sd * inv - r.mean * r.mean, 0.f));
  return r;
}

// Exclusive prefix sum over threads in index order through one LDS
// exchange in `red` (one barrier); *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int x, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(x, lane);
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int v = red[w];
    before += w < wave ? v : 0;
    tot += v;
  }
  *total = tot;
  return before + inc - x;
}

// OR the bits of key slot i (clusters k = tid + 1024 i) into a bitset with
// one ballot per wave: the wave's 64 lanes own 64 consecutive clusters.
template <int KPT>
__device__ __forceinline__ void ballot_bits(uint32_t mask, uint32_t* bits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const unsigned long long b = __ballot((mask >> i) & 1u);
    if (lane == 0 && b) {
      const int word = (kSelThreads * i + 64 * wave) >> 5;
      if ((uint32_t)b) atomicOr(&bits[word], (uint32_t)b);
      if ((uint32_t)(b >> 32)) atomicOr(&bits[word + 1], (uint32_t)(b >> 32));
    }
  }
}

template <int KPT, typename ScoreOf, typename Emit>
__device__ __forceinline__ void select_block(ScoreOf score_of, int c, int p, int sample,
                                             float temperature, uint64_t seed, uint32_t row,
                                             Emit emit, SelShared& sh) {
  // Thread t holds clusters k = t + 1024 i (i < KPT): consecutive threads
  // read consecutive scores.  Order-dependent steps (equal-key ties, the
  // ascending output) go through bitsets in LDS.
  const int tid = threadIdx.x;
  float raw[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) raw[i] = score_of(i, min(tid + kSelThreads * i, c - 1));
  if (sample) {
    // one Philox body in a rolled loop (not one copy per key)
#pragma unroll 1
    for (int i = 0; i < KPT; ++i) {
      const float g = gumbel_at(seed, row, (uint32_t)(tid + kSelThreads * i), 0u);
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (j == i) raw[j] = raw[j] / temperature + g;
    }
  }
  float (&key)[KPT] = raw;
  uint32_t act = 0u, sel = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int k = tid + kSelThreads * i;
    const float x = key[i];
    key[i] = isnan(x) ? -FLT_MAX : fminf(fmaxf(x, -FLT_MAX), FLT_MAX);
    if (k < c) act |= 1u << i;
  }
  FH_TRACE(8);
  sh.hist[2 * tid] = 0;
  sh.hist[2 * tid + 1] = 0;
  if (tid < 16384 / 32) {
    sh.selbits[tid] = 0u;
    sh.tiebits[tid] = 0u;
  }
  if (tid == 0) sh.ncand = 0;

  int need = p;
  if (need >= c) {
    sel = act;
    need = 0;
  }
  int nact = c;
  KeyStats st;
  {
    float mn = FLT_MAX, mx = -FLT_MAX, sum = 0.f, sq = 0.f;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (act & (1u << i)) {
        mn = fminf(mn, key[i]);
        mx = fmaxf(mx, key[i]);
        sum += key[i];
        sq += key[i] * key[i];
      }
    st = block_stats(mn, mx, sum, sq, nact, sh);  // its barrier also orders the zeroing above
  }
  FH_TRACE(9);

  bool ties = false;  // take the `need` smallest ids among the active keys
  while (need > 0) {
    if (!(st.lo < st.hi)) {
      ties = true;
      break;
    }
    // Buckets cover [a, b]: the keys' mean +- 4 standard deviations clipped
    // to [lo, hi], so that a few outlying keys do not squeeze the bulk into
    // a handful of buckets; keys outside fall into the end buckets.  The map
    // is monotone, lo lands in bucket 0 and hi in bucket 2047, so the
    // boundary bucket always holds fewer distinct keys than the range did.
    double a = fmax((double)st.lo, (double)st.mean - 4.0 * (double)st.sd);
    double b = fmin((double)st.hi, (double)st.mean + 4.0 * (double)st.sd);
    if (!(a < b)) {
      a = st.lo;
      b = st.hi;
    }
    const double scale = (double)kSelBins / (b - a);
    auto bucket = [&](float x) {
      const double t = ((double)x - a) * scale;
      return t <= 0.0 ? 0 : (int)fmin(t, (double)(kSelBins - 1));
    };
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (act & (1u << i)) atomicAdd(&sh.hist[bucket(key[i])], 1);
    __syncthreads();
    // suffix counts: thread t covers buckets j0 = 2047-2t and j1 = j0-1
    const int j0 = kSelBins - 1 - 2 * tid, j1 = j0 - 1;
    const int h0 = sh.hist[j0], h1 = sh.hist[j1];
    sh.hist[j0] = 0;  // ready for a next round
    sh.hist[j1] = 0;
    int tot;
    const int before = block_exclusive_scan(h0 + h1, sh.red_scan, &tot);
    if (before < need && before + h0 >= need) {
      sh.beta = j0; sh.above = before; sh.cnt = h0;
    } else if (before + h0 < need && before + h0 + h1 >= need) {
      sh.beta = j1; sh.above = before + h0; sh.cnt = h1;
    }
    __syncthreads();
    const int beta = sh.beta, cntb = sh.cnt;
    FH_TRACE(10);
    if (tid == 0 && blockIdx.x < 4096) g_fh_trace_cnt(cntb);
    need -= sh.above;
    float mn = FLT_MAX, mx = -FLT_MAX, sum = 0.f, sq = 0.f;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (!(act & (1u << i))) continue;
      const int bi = bucket(key[i]);
      if (bi > beta) {
        sel |= 1u << i;
        act &= ~(1u << i);
      } else if (bi < beta) {
        act &= ~(1u << i);
      } else {
        mn = fminf(mn, key[i]);
        mx = fmaxf(mx, key[i]);
        sum += key[i];
        sq += key[i] * key[i];
      }
    }
    if (cntb == need) {
      sel |= act;
      break;
    }
    if (cntb <= kRankMax) {
      // exact rank of each boundary key among the boundary keys
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (act & (1u << i)) {
          const int slot = atomicAdd(&sh.ncand, 1);
          sh.cand_key[slot] = key[i];
          sh.cand_id[slot] = tid + kSelThreads * i;
        }
      }
      __syncthreads();
      const int n = sh.ncand;
      if (tid < n) {
        const float mk = sh.cand_key[tid];
        const int mi = sh.cand_id[tid];
        int rank = 0;
        for (int j = 0; j < n; ++j) rank += better(sh.cand_key[j], sh.cand_id[j], mk, mi) ? 1 : 0;
        if (rank < need) atomicOr(&sh.selbits[mi >> 5], 1u << (mi & 31));
      }
      FH_TRACE(11);
      break;
    }
    // a large boundary bucket becomes the next range (red[] was last read
    // before this round's first barrier)
    nact = cntb;
    st = block_stats(mn, mx, sum, sq, nact, sh);
  }

  ballot_bits<KPT>(sel, sh.selbits);
  if (ties) ballot_bits<KPT>(act, sh.tiebits);
  __syncthreads();
  FH_TRACE(12);
  // ascending compaction: thread t reads the bits of clusters [t*KPT, t*KPT+KPT)
  const int b0 = tid * KPT;
  uint32_t mine = 0u, tie_mine = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int k = b0 + i;
    if (k < c && (sh.selbits[k >> 5] & (1u << (k & 31)))) mine |= 1u << i;
    if (ties && k < c && (sh.tiebits[k >> 5] & (1u << (k & 31)))) tie_mine |= 1u << i;
  }
  if (ties) {
    // keep the first `need` of the equal keys in id order
    int tie_tot;
    int rank = block_exclusive_scan(__popc(tie_mine), sh.red_scan, &tie_tot);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (tie_mine & (1u << i)) {
        if (rank < need) mine |= 1u << i;
        ++rank;
      }
    }
  }
  int tot;
  int off = block_exclusive_scan(__popc(mine), sh.red_out, &tot);
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (mine & (1u << i)) emit(off++, b0 + i);
  FH_TRACE(13);
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ scores, int c,
                                                        int p, int sample, float temperature,
                                                        uint64_t seed, int32_t* __restrict__ S,
                                                        int ldS) {
  __shared__ SelShared sh;
  FH_TRACE(14);
  const int q = blockIdx.x;
  const float* sq = scores + (int64_t)q * c;
  int32_t* Sq = S + (int64_t)q * ldS;
  select_block<KPT>([&](int, int k) { return sq[k]; }, c, p, sample, temperature, seed, (uint32_t)q,
                    [&](int pos, int k) { Sq[pos] = k; }, sh);
}

// ======================================================================
// Finisher: merge n Parts in a fixed order (threads stride, then a tree).
// ======================================================================
// Merge n Parts: each thread folds a strided subset in index order, the
// waves merge their lanes, and thread 0 merges the waves in order.
template <int NT>
__device__ __forceinline__ Part merge_parts_block(const Part* __restrict__ pq, int n, Part* sh) {
  Part acc = part_empty();
  for (int i = threadIdx.x; i < n; i += NT) acc = part_merge(acc, pq[i]);
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

__global__ __launch_bounds__(256) void k_finish(const Part* __restrict__ parts, int nparts,
                                                int32_t* __restrict__ out_token,
                                                float* __restrict__ out_logit,
                                                float* __restrict__ out_lse) {
  __shared__ Part sh[256];
  const int q = blockIdx.x;
  const Part r = merge_parts_block<256>(parts + (int64_t)q * nparts, nparts, sh);
  if (threadIdx.x == 0) write_outputs(r, q, out_token, out_logit, out_lse);
}

// ======================================================================
// Batch-1 path: the whole call in one launch.
//
// The grid's workgroups (1024 threads) take roles by index, in the order
// they are dispatched:
//   [0, G1)        stage 1: rows1 centroid rows each (16 waves x 2 rows at a
//                  time);
//   [G1, G1+G2)    stage 2: rows2 of the p*b retrieved tokens each, with the
//                  fused epilogue.  The first of them (G1) is also the
//                  selector: before its own rows it waits for the c scores
//                  and selects the probes.  The last (G1+G2-1) is also the
//                  finisher: after its own rows it waits for the G2 partials
//                  and merges them.
// Results pass between workgroups as 64-bit words tagged with the call's
// epoch (epoch << 32 | payload), written and polled with agent-scope (sc1)
// accesses.  A workgroup only ever waits for words written by workgroups
// with smaller or equal indices.  Like a decoupled look-back scan, this
// relies on workgroups being dispatched in index order, so every awaited
// workgroup is already running and never waits for its waiter; the grid
// need not be co-resident.  Sizes keep G1 < CUs and G2 <= CUs so that at
// one workgroup per CU the selector starts at once and every stage-2
// workgroup is resident when stage 1 retires.  Every wait is bounded: past
// kSpinLimit polls the waiter sets *err and goes on with what it has, so the
// grid always drains.
// ======================================================================
struct FusedArgs {
  const void* E;
  const void* C;
  const uint8_t* cq;
  const uint16_t* csig;
  const int32_t* c2t;
  int c;
  int bsz;
  int d;
  const void* h;
  int p;
  int probe_sample;
  int token_sample;
  float temperature;
  float tprime;
  uint64_t seed;
  int g1, g2;                   // stage-1 and stage-2 workgroup counts
  int rows1, rows2;             // rows per stage-1 / stage-2 workgroup
  unsigned epoch;               // never 0
  unsigned long long* tscores;  // [c] tagged scores
  unsigned long long* tsel;     // [p] tagged probe ids (ascending)
  unsigned long long* tparts;   // [5 x g2] tagged Parts
  int32_t* out_clusters;        // [p] or null
  int32_t* out_ids;
  float* out_logits;
  int32_t* out_token;
  float* out_logit;
  float* out_lse;
  unsigned* err;  // sticky: a poll gave up
};

constexpr int kRowsUnit = 32;  // 16 waves x 2 rows
constexpr unsigned kSpinLimit = 1u << 20;

__device__ __forceinline__ unsigned long long tag(unsigned epoch, uint32_t bits) {
  return ((unsigned long long)epoch << 32) | bits;
}

__device__ __forceinline__ void st_tagged(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll N tagged words until each carries `epoch`, keeping every load of a
// round in flight together; out[i] gets word i's low 32 bits.  Words with
// live[i] false are skipped.
template <int N>
__device__ __forceinline__ void poll_tagged(unsigned long long* const (&p)[N],
                                            const bool (&live)[N], unsigned epoch,
                                            unsigned* err, uint32_t (&out)[N]) {
  unsigned long long v[N];
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = live[i] ? __hip_atomic_load(p[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : tag(epoch, 0u);
  for (unsigned n = 0;; ++n) {
    bool done = true;
#pragma unroll
    for (int i = 0; i < N; ++i) done = done && (unsigned)(v[i] >> 32) == epoch;
    if (done) break;
    if (n >= kSpinLimit) {
      __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((unsigned)(v[i] >> 32) != epoch)
        v[i] = __hip_atomic_load(p[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = (uint32_t)v[i];
}

union Batch1Shared {
  SelShared sel;
  Part parts[1024];
  int probes[1024];
};

template <typename T, int MAXM, int KPT, bool INT4, int MAXG>
__global__ __launch_bounds__(1024) void k_batch1(FusedArgs a) {
  __shared__ Batch1Shared sh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int w = blockIdx.x;
  const T* hp = static_cast<const T*>(a.h);

  if (w < a.g1) {  // ---- stage 1
    FH_TRACE(0);
    const int64_t r_lo = (int64_t)w * a.rows1;
    const int64_t r_hi = min((int64_t)a.c, r_lo + a.rows1);
    auto sink = [&](int, int64_t r, int64_t, float s) {
      if (lane == 0) st_tagged(a.tscores + r, tag(a.epoch, __float_as_uint(s)));
    };
    if (INT4) {
      HGroups<MAXG> hg[1];
      load_hgroups<T, MAXG>(hp, a.d / 32, lane, hg[0]);
      wave_rows_int4<MAXG, 1>(a.cq, a.csig, a.d, lane, hg, 1, r_lo + wave, r_hi, 16, sink);
    } else {
      uint4 hv[1][MAXM];
      load_hslice<T, MAXM>(hp, a.d / Chunk<T>::kElems, lane, hv[0]);
      wave_rows<T, MAXM, 1>(static_cast<const T*>(a.C), a.d, lane, hv, 1, r_lo + wave, r_hi, 16,
                            [](int64_t r) { return r; }, sink);
    }
    FH_TRACE(1);
#ifdef FH_PHASE_TRACE
    __syncthreads();
    FH_TRACE(7);  // every wave of this workgroup is done
#endif
    return;
  }

  const int j = w - a.g1;  // stage-2 workgroup index
  if (j == 0) {            // ---- selector
    FH_TRACE(2);
    // the keys this thread holds in select_block: k = tid + 1024 i
    unsigned long long* ptr[KPT];
    bool live[KPT];
    uint32_t raw[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int k = (int)threadIdx.x + kSelThreads * i;
      live[i] = k < a.c;
      ptr[i] = a.tscores + (live[i] ? k : 0);
    }
    poll_tagged<KPT>(ptr, live, a.epoch, a.err, raw);
    select_block<KPT>(
        [&](int i, int) { return __uint_as_float(raw[i]); }, a.c, a.p, a.probe_sample,
        a.temperature, a.seed, 0u,
        [&](int pos, int k) {
          st_tagged(a.tsel + pos, tag(a.epoch, (uint32_t)k));
          if (a.out_clusters) a.out_clusters[pos] = k;
        },
        sh.sel);
    FH_TRACE(3);
    __syncthreads();  // sh.sel is reused below
  }

  // ---- stage 2
  FH_TRACE(4);
  const int64_t n2 = (int64_t)a.p * a.bsz;
  const int64_t r_lo = (int64_t)j * a.rows2;
  const int64_t r_hi = min(n2, r_lo + a.rows2);
  uint4 hv[1][MAXM];
  load_hslice<T, MAXM>(hp, a.d / Chunk<T>::kElems, lane, hv[0]);
  // the probes this workgroup's rows come from, published by the selector
  const int pos0 = (int)(r_lo / a.bsz);
  const int npos = r_hi > r_lo ? (int)((r_hi - 1) / a.bsz) - pos0 + 1 : 0;
  for (int t = threadIdx.x; t < npos; t += 1024) {
    unsigned long long* const ptr[1] = {a.tsel + pos0 + t};
    const bool live[1] = {true};
    uint32_t k[1];
    poll_tagged<1>(ptr, live, a.epoch, a.err, k);
    sh.probes[t] = (int)k[0];
  }
  __syncthreads();
  FH_TRACE(5);
  Part part[1] = {part_empty()};
  auto src_of = [&](int64_t r) -> int64_t {
    return a.c2t[(int64_t)sh.probes[r / a.bsz - pos0] * a.bsz + r % a.bsz];
  };
  auto sink = [&](int, int64_t r, int64_t src, float z) {
    if (lane == 0) {
      if (a.out_logits) a.out_logits[r] = z;
      if (a.out_ids) a.out_ids[r] = (int32_t)src;
    }
    part[0] = part_merge(part[0], part_of(z, (int32_t)src, a.token_sample, a.tprime, a.seed, 0u));
  };
  wave_rows<T, MAXM, 1>(static_cast<const T*>(a.E), a.d, lane, hv, 1, r_lo + wave, r_hi, 16,
                        src_of, sink);
  __syncthreads();  // sh.probes is read above; sh.parts aliases it
  const Part wg = block_merge_parts<16, 1>(part, 1, sh.parts);
  if (threadIdx.x == 0) {
    unsigned long long* tp = a.tparts + 5 * (int64_t)j;
    st_tagged(tp + 0, tag(a.epoch, __float_as_uint(wg.key)));
    st_tagged(tp + 1, tag(a.epoch, __float_as_uint(wg.z)));
    st_tagged(tp + 2, tag(a.epoch, __float_as_uint(wg.m)));
    st_tagged(tp + 3, tag(a.epoch, __float_as_uint(wg.s)));
    st_tagged(tp + 4, tag(a.epoch, (uint32_t)wg.id));
  }
  FH_TRACE(6);
  if (j != a.g2 - 1) return;

  // ---- finisher: every stage-2 partial, merged in a fixed order
  __syncthreads();  // sh.parts is reused
  Part acc = part_empty();
  for (int i = threadIdx.x; i < a.g2; i += 1024) {
    unsigned long long* tp = a.tparts + 5 * (int64_t)i;
    unsigned long long* const ptr[5] = {tp, tp + 1, tp + 2, tp + 3, tp + 4};
    const bool live[5] = {true, true, true, true, true};
    uint32_t wv[5];
    poll_tagged<5>(ptr, live, a.epoch, a.err, wv);
    acc = part_merge(acc, Part{__uint_as_float(wv[0]), __uint_as_float(wv[1]),
                               __uint_as_float(wv[2]), __uint_as_float(wv[3]), (int32_t)wv[4]});
  }
  acc = wave_merge_part(acc);
  if (lane == 0) sh.parts[wave] = acc;
  __syncthreads();
  Part r = sh.parts[0];
  for (int w2 = 1; w2 < 16; ++w2) r = part_merge(r, sh.parts[w2]);
  if (threadIdx.x == 0) write_outputs(r, 0, a.out_token, a.out_logit, a.out_lse);
  FH_TRACE(14);
}

// ======================================================================
// Host-side launchers
// ======================================================================

int64_t rows_blocks(int64_t nrows, int rpw) { return (nrows + 4 * rpw - 1) / (4 * rpw); }

template <typename T, int NQ, int RPW, bool GATHER, bool EPI>
static hipError_t launch_rows(const RowsArgs& a, hipStream_t st, int64_t* nblocks) {
  const int nch = a.d / Chunk<T>::kElems;
  const int maxm = (nch + 63) / 64;
  const int64_t gx = rows_blocks(a.nrows, RPW);
  const int gy = GATHER ? a.B : (a.B + NQ - 1) / NQ;
  if (nblocks) *nblocks = gx;
  if (gx <= 0 || gy <= 0) return hipSuccess;
  const dim3 grid((unsigned)gx, (unsigned)gy);
  switch (maxm) {
#define FH_CASE(MM) \
  case MM: hipLaunchKernelGGL((k_rows<T, MM, NQ, RPW, GATHER, EPI>), grid, dim3(256), 0, st, a); break;
    FH_CASE(1) FH_CASE(2) FH_CASE(3) FH_CASE(4) FH_CASE(5) FH_CASE(6) FH_CASE(7) FH_CASE(8)
#undef FH_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t score_dispatch(const KernelCtx& k, const void* h, int B, float* out) {
  RowsArgs a{};
  a.M = k.C; a.nrows = k.c; a.d = k.d; a.H = h; a.B = B; a.out_vals = out; a.ld_vals = k.c;
  a.tprime = 1.f;
  if (B == 1) return launch_rows<T, 1, kScoreRPW, false, false>(a, k.stream, nullptr);
  if (B == 2) return launch_rows<T, 2, kScoreRPW, false, false>(a, k.stream, nullptr);
  return launch_rows<T, 4, kScoreRPW, false, false>(a, k.stream, nullptr);
}

hipError_t launch_score(const KernelCtx& k, const void* h, int B, float* out) {
  return k.bf16 ? score_dispatch<uint16_t>(k, h, B, out) : score_dispatch<float>(k, h, B, out);
}

template <typename T, int NQ>
static hipError_t int4_launch(const KernelCtx& k, const void* h, int B, float* out) {
  const int G = k.d / 32;
  const int maxg = (G + 63) / 64;
  const int64_t gx = (k.c + 4 * kInt4RPW - 1) / (4 * kInt4RPW);
  const dim3 grid((unsigned)gx, (unsigned)((B + NQ - 1) / NQ));
  const T* hp = static_cast<const T*>(h);
  switch (maxg) {
#define FH_CASE(MG) \
  case MG: hipLaunchKernelGGL((k_score_int4<T, MG, NQ, kInt4RPW>), grid, dim3(256), 0, k.stream, k.cq, k.csig, k.c, k.d, hp, B, out); break;
    FH_CASE(1) FH_CASE(2) FH_CASE(3) FH_CASE(4)
#undef FH_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_int4(const KernelCtx& k, const void* h, int B, float* out) {
  if (k.bf16) return B == 1 ? int4_launch<uint16_t, 1>(k, h, B, out) : int4_launch<uint16_t, 2>(k, h, B, out);
  return B == 1 ? int4_launch<float, 1>(k, h, B, out) : int4_launch<float, 2>(k, h, B, out);
}

hipError_t launch_quant_int4(const KernelCtx& k, int* bad) {
  const int64_t n = k.c * (k.d / 32);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (k.bf16)
    hipLaunchKernelGGL((k_quant_int4<uint16_t>), grid, dim3(256), 0, k.stream,
                       static_cast<const uint16_t*>(k.C), k.c, k.d, const_cast<uint8_t*>(k.cq),
                       const_cast<uint16_t*>(k.csig), bad);
  else
    hipLaunchKernelGGL((k_quant_int4<float>), grid, dim3(256), 0, k.stream,
                       static_cast<const float*>(k.C), k.c, k.d, const_cast<uint8_t*>(k.cq),
                       const_cast<uint16_t*>(k.csig), bad);
  return hipGetLastError();
}

static int select_kpt(int64_t c) {
  const int64_t k = (c + kSelThreads - 1) / kSelThreads;
  return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : k <= 16 ? 16 : -1;
}

hipError_t launch_select(const KernelCtx& k, const float* scores, int B, int p, int sample,
                         float temperature, uint64_t seed, int32_t* S, int ldS) {
  const dim3 grid((unsigned)B), block(kSelThreads);
  const int c = (int)k.c;
  switch (select_kpt(k.c)) {
#define FH_CASE(KK) \
  case KK: hipLaunchKernelGGL((k_select<KK>), grid, block, 0, k.stream, scores, c, p, sample, temperature, seed, S, ldS); break;
    FH_CASE(1) FH_CASE(2) FH_CASE(4) FH_CASE(8) FH_CASE(16)
#undef FH_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t gather_t(const KernelCtx& k, const void* h, int B, const int32_t* S, int p,
                           int token_sample, float tprime, uint64_t seed, int32_t* out_ids,
                           float* out_logits, Part* parts, int64_t* nparts) {
  RowsArgs a{};
  a.M = k.E; a.nrows = (int64_t)p * k.b; a.d = k.d; a.c2t = k.c2t; a.bsz = (int)k.b;
  a.S = S; a.ldS = p; a.H = h; a.B = B; a.out_vals = out_logits; a.ld_vals = a.nrows;
  a.out_ids = out_ids; a.token_sample = token_sample; a.tprime = tprime; a.seed = seed;
  a.parts = parts;
  return launch_rows<T, 1, kGatherRPW, true, true>(a, k.stream, nparts);
}

hipError_t launch_gather(const KernelCtx& k, const void* h, int B, const int32_t* S, int p,
                         int token_sample, float tprime, uint64_t seed, int32_t* out_ids,
                         float* out_logits, Part* parts, int64_t* nparts) {
  return k.bf16 ? gather_t<uint16_t>(k, h, B, S, p, token_sample, tprime, seed, out_ids, out_logits, parts, nparts)
                : gather_t<float>(k, h, B, S, p, token_sample, tprime, seed, out_ids, out_logits, parts, nparts);
}

template <typename T>
static hipError_t dense_t(const KernelCtx& k, const void* h, int B, int token_sample, float tprime,
                          uint64_t seed, float* out_logits, Part* parts, int64_t* nparts) {
  RowsArgs a{};
  a.M = k.E; a.nrows = k.v; a.d = k.d; a.H = h; a.B = B; a.out_vals = out_logits; a.ld_vals = k.v;
  a.token_sample = token_sample; a.tprime = tprime; a.seed = seed; a.parts = parts;
  if (B == 1) return launch_rows<T, 1, kDenseRPW, false, true>(a, k.stream, nparts);
  if (B == 2) return launch_rows<T, 2, kDenseRPW, false, true>(a, k.stream, nparts);
  return launch_rows<T, 4, kDenseRPW, false, true>(a, k.stream, nparts);
}

hipError_t launch_dense(const KernelCtx& k, const void* h, int B, int token_sample, float tprime,
                        uint64_t seed, float* out_logits, Part* parts, int64_t* nparts) {
  return k.bf16 ? dense_t<uint16_t>(k, h, B, token_sample, tprime, seed, out_logits, parts, nparts)
                : dense_t<float>(k, h, B, token_sample, tprime, seed, out_logits, parts, nparts);
}

hipError_t launch_finish(const KernelCtx& k, const Part* parts, int B, int64_t nparts,
                         int32_t* out_token, float* out_logit, float* out_lse) {
  hipLaunchKernelGGL(k_finish, dim3((unsigned)B), dim3(256), 0, k.stream, parts, (int)nparts,
                     out_token, out_logit, out_lse);
  return hipGetLastError();
}

// ---- batch-1 path: one launch

// Rows per workgroup: a multiple of 32 (16 waves x 2 rows) large enough that
// a stage needs at most `slots` workgroups: cus - 4 for stage 1 (so the
// selector and a few stage-2 workgroups start at once), cus for stage 2.
static int64_t batch1_rows(int64_t n, int64_t slots) {
  slots = std::max<int64_t>(slots, 1);
  const int64_t units = (n + kRowsUnit - 1) / kRowsUnit;
  return kRowsUnit * std::max<int64_t>(1, (units + slots - 1) / slots);
}
static int64_t slots1(int cus) { return cus > 8 ? cus - 4 : 4; }
int batch1_stage1_blocks(int64_t c, int cus) {
  const int64_t r = batch1_rows(c, slots1(cus));
  return (int)((c + r - 1) / r);
}
int batch1_stage2_blocks(int64_t p, int64_t b, int cus) {
  const int64_t r = batch1_rows(p * b, cus);
  return (int)std::max<int64_t>(1, (p * b + r - 1) / r);
}

static FusedArgs fused_args(const FusedLaunch& f) {
  const KernelCtx& k = *f.ctx;
  FusedArgs a{};
  a.E = k.E; a.C = k.C; a.cq = k.cq; a.csig = k.csig; a.c2t = k.c2t;
  a.c = (int)k.c; a.bsz = (int)k.b; a.d = k.d; a.h = f.h; a.p = f.p;
  a.probe_sample = f.probe_sample; a.token_sample = f.token_sample;
  a.temperature = f.temperature; a.tprime = f.tprime; a.seed = f.seed;
  a.rows1 = (int)batch1_rows(k.c, slots1(f.cus));
  a.rows2 = (int)batch1_rows((int64_t)f.p * k.b, f.cus);
  a.g1 = batch1_stage1_blocks(k.c, f.cus);
  a.g2 = batch1_stage2_blocks(f.p, k.b, f.cus);
  a.epoch = f.epoch; a.tscores = f.tscores; a.tsel = f.tsel; a.tparts = f.tparts;
  a.out_clusters = f.out_clusters; a.out_ids = f.out_ids; a.out_logits = f.out_logits;
  a.out_token = f.out_token; a.out_logit = f.out_logit; a.out_lse = f.out_lse;
  a.err = f.err;
  return a;
}

template <typename T, int MAXM, int KPT, bool INT4, int MAXG>
static hipError_t b1_go(const FusedLaunch& f, const FusedArgs& a) {
  const unsigned grid = (unsigned)(a.g1 + a.g2);
  hipLaunchKernelGGL((k_batch1<T, MAXM, KPT, INT4, MAXG>), dim3(grid), dim3(1024), 0,
                     f.ctx->stream, a);
  return hipGetLastError();
}

template <typename T, int KPT, bool INT4, int MAXG>
static hipError_t b1_m(const FusedLaunch& f, const FusedArgs& a) {
  const int nch = f.ctx->d / Chunk<T>::kElems;
  switch ((nch + 63) / 64) {
#define FH_CASE(MM) case MM: return b1_go<T, MM, KPT, INT4, MAXG>(f, a);
    FH_CASE(1) FH_CASE(2) FH_CASE(3) FH_CASE(4) FH_CASE(5) FH_CASE(6) FH_CASE(7) FH_CASE(8)
#undef FH_CASE
    default: return hipErrorInvalidValue;
  }
}

template <typename T, bool INT4, int MAXG>
static hipError_t b1_k(const FusedLaunch& f, const FusedArgs& a) {
  switch (select_kpt(f.ctx->c)) {
    case 1: return b1_m<T, 1, INT4, MAXG>(f, a);
    case 2: return b1_m<T, 2, INT4, MAXG>(f, a);
    case 4: return b1_m<T, 4, INT4, MAXG>(f, a);
    case 8: return b1_m<T, 8, INT4, MAXG>(f, a);
    case 16: return b1_m<T, 16, INT4, MAXG>(f, a);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t b1_t(const FusedLaunch& f, const FusedArgs& a) {
  if (!f.int4) return b1_k<T, false, 1>(f, a);
  switch ((f.ctx->d / 32 + 63) / 64) {
    case 1: return b1_k<T, true, 1>(f, a);
    case 2: return b1_k<T, true, 2>(f, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_batch1(const FusedLaunch& f) {
  const FusedArgs a = fused_args(f);
  return f.ctx->bf16 ? b1_t<uint16_t>(f, a) : b1_t<float>(f, a);
}

}  // namespace fh
