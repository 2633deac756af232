// The offline step that produces C and C2T: balanced spherical k-means on
// gfx950 (FlashHead explainer, framerc.cn, §1.2.1 balanced clustering and
// §2.1 offline clustering; arXiv 2603.14591 abstract, innovation (1)).
//
// Steps, as the pages order them:
//   normalise  every embedding row to unit length (spherical k-means);
//   k-means++  centre 0 is token floor(u_0 v); centre i is drawn with
//              probability proportional to D(t)^2, D(t) = 1 - max_j cos(t, C_j)
//              (inverse CDF over token order, u_i given): per step one
//              kernel refreshes D against the newest centre, one workgroup
//              sums D^2 in fp64 in a fixed order and finds the token;
//   iterate    cosine similarities S = X C^T (bf16 tables: matrix cores with
//              C split exactly into three bf16 pieces; fp32 tables: an fp32
//              tiled GEMM on the vector units); the balanced
//              assignment by rounds (each unassigned token proposes to its
//              most similar non-full cluster, ties to the smaller cluster id;
//              each cluster takes the most similar proposals up to its room,
//              ties to the smaller token id), where the proposals are ranked
//              by one stable radix sort on (cluster, similarity) keys; then
//              C2T (each cluster's tokens ascending, by a stable sort on the
//              cluster) and C_k = normalise(sum of its rows in slot order).
// Every step is deterministic: no floating-point atomics, fixed orders.

#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <cstdio>
#include <vector>

#include "fh_blocks.hpp"

namespace fh {

// ----------------------------------------------------------- normalise ---

// X[t] = E[t] / |E[t]| in fp32 and inv[t] = 1 / |E[t]| (0 for a zero row).
template <typename T>
__global__ __launch_bounds__(256) void k_normalize_rows(const T* __restrict__ E, int64_t v, int d,
                                                        float* __restrict__ X,
                                                        float* __restrict__ inv) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= v) return;
  float ss = 0.f;
  for (int i = lane; i < d; i += 64) {
    const float x = load_elem<T>(E, t * d + i);
    ss = fmaf(x, x, ss);
  }
  ss = wave_sum(ss);
  const float r = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  for (int i = lane; i < d; i += 64) X[t * d + i] = load_elem<T>(E, t * d + i) * r;
  if (lane == 0) inv[t] = r;
}

// ------------------------------------------------------------ k-means++ ---

// Rows per workgroup of the k-means++ step, one per wave: many small
// workgroups keep the most row reads in flight (measured on the 128256 x
// 2048 bf16 table: 4 rows per workgroup stream 5.9 TB/s, 64 rows 4.8 TB/s).
// Also the block of rows the draw scans last.
constexpr int kPpRows = 4;

// One k-means++ step's distance refresh against centre i:
//   D[t] = min(D[t], 1 - inv[t] inv[ct] (E_t . E_ct))   (= when i == 0)
// with the table read in its own storage type (coalesced 16-byte row loads,
// the centre's row in registers), and the sum of D^2 over workgroup w's rows
// in fp64 (row order within each wave, then wave 0..3) stored at
// part[(w % n) * 1024 + w / n], n = ceil(gridDim.x / 1024): the draw's
// thread t, which owns partials t n .. t n + n - 1, reads them 1024 apart,
// coalesced with its neighbours.
template <typename T, int MAXM, int RPI = 1, int ROWS = kPpRows>
__global__ __launch_bounds__(256) void k_pp_step(const T* __restrict__ E,
                                                 const float* __restrict__ inv, int64_t v, int d,
                                                 const int32_t* __restrict__ centers, int i,
                                                 float* __restrict__ D, double* __restrict__ part) {
  __shared__ double wsum[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t ct = centers[i];
  const int nch = d / Chunk<T>::kElems;
  uint4 hv[1][MAXM];
  load_hslice<T, MAXM>(E + ct * d, nch, lane, hv[0]);
  const float ic = inv[ct];
  const int64_t r0 = (int64_t)blockIdx.x * ROWS + wave * (ROWS / 4);
  const int64_t r1 = min(r0 + ROWS / 4, v);
  double s = 0.0;
  auto row = [](int64_t r) -> int64_t { return r; };
  auto sink = [&](int, int64_t r, int64_t, float z) {
    float dist = 1.f - z * inv[r] * ic;
    if (i > 0) dist = fminf(D[r], dist);
    if (lane == 0) D[r] = dist;
    s += (double)dist * (double)dist;
  };
  wave_rows<T, MAXM, 1, RPI>(E, d, lane, hv, 1, r0, r1, 1, row, row, sink);
  if (lane == 0) wsum[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t n = ((int64_t)gridDim.x + 1023) / 1024;
    part[((int64_t)blockIdx.x % n) * 1024 + (int64_t)blockIdx.x / n] =
        ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
}

// Inclusive prefix sum over the 64 lanes of a wave, in fp64 (fixed order).
__device__ __forceinline__ double wave_prefix(double x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// One wave walks vals[lo, hi) 64 at a time from the running sum *base and
// returns the first index whose running sum exceeds target (hi - 1 if
// rounding between the levels leaves none), with *base set to the running
// sum before it.  Wave-uniform.
template <typename Load>
__device__ __forceinline__ int64_t wave_walk(Load load, int64_t lo, int64_t hi, double target,
                                             double* base, int lane) {
  double b = *base;
  for (int64_t j0 = lo; j0 < hi; j0 += 64) {
    const int64_t j = j0 + lane;
    const double x = wave_prefix(j < hi ? load(j) : 0.0, lane);
    const unsigned long long hit = __ballot(j < hi && b + x > target);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      const double before = __shfl(x, l > 0 ? l - 1 : 0);
      *base = l > 0 ? b + before : b;
      return j0 + l;
    }
    b += __shfl(x, 63);
  }
  *base = b;
  return hi - 1;
}

// The draw of centre i (one workgroup of 1024) from the nb workgroup
// partials of k_pp_step.  Thread t sums its n = ceil(nb / 1024) partials
// t n .. t n + n - 1 in order (stored 1024 apart); the running sums over the
// threads (lane prefix per wave, then the earlier waves' totals in order)
// give the total and the first share where the running sum of D^2 exceeds
// u * total; wave 0 then walks that share to the block and the block's
// kPpRows rows to the token.  With a zero total the draw is token floor(u v).
__global__ __launch_bounds__(1024) void k_pp_pick(const float* __restrict__ D,
                                                  const double* __restrict__ part, int64_t nb,
                                                  int64_t v, double u, int32_t* __restrict__ centers,
                                                  int i) {
  __shared__ double wtot[16];
  __shared__ double ps_found;
  __shared__ int found;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = (nb + 1023) / 1024;
  const int64_t lo = min(nb, tid * n), hi = min(nb, lo + n);
  // 16 loads in flight, then added in order (a zero past the share changes
  // nothing: the sums are non-negative)
  double s = 0.0;
  for (int64_t j0 = lo; j0 < hi; j0 += 16) {
    double x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = j0 + k < hi ? part[(j0 + k - lo) * 1024 + tid] : 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += x[k];
  }
  const double incl_w = wave_prefix(s, lane);
  const double prev_w = __shfl_up(incl_w, 1);
  if (lane == 63) wtot[wave] = incl_w;
  if (tid == 0) found = 1024;
  __syncthreads();
  double off = 0.0, total = 0.0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    if (w < wave) off += wtot[w];
    total += wtot[w];
  }
  if (!(total > 0.0)) {
    if (tid == 0) centers[i] = (int32_t)min<int64_t>((int64_t)(u * (double)v), v - 1);
    return;
  }
  const double target = u * total;
  // a thread's exclusive sum is its predecessor's inclusive sum, formed by
  // the same operations, so the crossings are exact; the lowest one counts
  const double incl = off + incl_w, excl = lane ? off + prev_w : off;
  if (incl > target && excl <= target) atomicMin(&found, tid);
  __syncthreads();
  const int f = found < 1024 ? found : 1023;  // no crossing: the last share
  if (tid == f) ps_found = excl;
  __syncthreads();
  if (tid >= 64) return;
  double base = ps_found;
  const int64_t flo = min(nb, f * n), fhi = min(nb, flo + n);
  const int64_t blk = flo < fhi ? wave_walk([&](int64_t j) { return part[(j - flo) * 1024 + f]; },
                                            flo, fhi, target, &base, lane)
                                : nb - 1;
  const int64_t rlo = blk * kPpRows, rhi = min(v, rlo + kPpRows);
  const int64_t r = wave_walk([&](int64_t t) { return (double)D[t] * (double)D[t]; }, rlo, rhi,
                              target, &base, lane);
  if (lane == 0) centers[i] = (int32_t)r;
}

__global__ __launch_bounds__(256) void k_gather_rows(const float* __restrict__ X, int d,
                                                     const int32_t* __restrict__ idx, int64_t n,
                                                     float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * d) return;
  out[i] = X[(int64_t)idx[i / d] * d + i % d];
}

// ------------------------------------------------------ similarity GEMM ---

// S[t][k] = X_t . C_k in fp32 (sequential FMA over d): 64 x 64 tiles, 256
// threads with 4 x 4 outputs each, 32-element slices of d through LDS.
__global__ __launch_bounds__(256) void k_sims(const float* __restrict__ X, int64_t v,
                                              const float* __restrict__ C, int64_t c, int d,
                                              float* __restrict__ S) {
  __shared__ float As[32][65];
  __shared__ float Bs[32][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 64, n0 = (int64_t)blockIdx.y * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 32) {
    // 64 rows x 32 elements of each operand: 8 per thread
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = tid + 256 * e, r = idx >> 5, k = idx & 31;
      const int64_t am = m0 + r, bn = n0 + r;
      As[k][r] = (am < v && k0 + k < d) ? X[am * d + k0 + k] : 0.f;
      Bs[k][r] = (bn < c && k0 + k < d) ? C[bn * d + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[k][ty * 4 + i];
        b[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= v) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n < c) S[m * c + n] = acc[i][j];
    }
  }
}

// S on the matrix cores for bf16 tables.  The centres are fp32; each is
// split exactly into three bf16 pieces, C = hi + mid + lo up to 2^-27
// relative (hi = bf16(C), mid = bf16(C - hi), lo = bf16(C - hi - mid); each
// difference is exact in fp32), so E_t . C_k = E_t . hi + E_t . mid +
// E_t . lo with exact bf16 products and fp32 accumulation in
// v_mfma_f32_16x16x32_bf16, and S[t][k] = inv[t] (E_t . C_k).
typedef __bf16 sim_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sim_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ sim_f32x4 sim_mfma(const uint4& a, const uint4& b, sim_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sim_bf16x8, a),
                                                 __builtin_bit_cast(sim_bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// P[piece][k][i] for the three pieces of C[k][i].
__global__ __launch_bounds__(256) void k_split_pieces(const float* __restrict__ C, int64_t n,
                                                      uint16_t* __restrict__ P) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float x = C[i];
  const uint16_t hi = bf16_rne(x);
  const float r1 = x - __uint_as_float((uint32_t)hi << 16);
  const uint16_t mid = bf16_rne(r1);
  const float r2 = r1 - __uint_as_float((uint32_t)mid << 16);
  P[i] = hi;
  P[n + i] = mid;
  P[2 * n + i] = bf16_rne(r2);
}

constexpr int kSimTile = 128;   // tokens and clusters per workgroup
constexpr int kSimLds = 40;     // LDS row of one 32-element step (bf16), padded

// One workgroup: tokens [128 x, +128) x clusters [128 y, +128); wave w owns
// the 64 x 64 quadrant (w & 1, w >> 1): 4 x 4 tiles of 16 x 16, three
// pieces each.  d is walked in steps of 32 elements through double-buffered
// LDS (one barrier per step: the buffer written during step s was last read
// in step s - 1).  Operand fragments as the instruction takes them: lane l
// holds row (token) or column (cluster) l % 16 at elements 8 (l / 16) .. + 7
// of the step; the result holds cluster l % 16 at tokens 4 (l / 16) .. + 3.
__global__ __launch_bounds__(256) void k_sims_mfma(const uint16_t* __restrict__ E,
                                                   const float* __restrict__ inv, int64_t v, int d,
                                                   const uint16_t* __restrict__ P, int64_t c,
                                                   float* __restrict__ S) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kSimTile * kSimLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][3 * kSimTile * kSimLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t t0 = (int64_t)blockIdx.x * kSimTile, k0 = (int64_t)blockIdx.y * kSimTile;
  const int nks = (d + 31) / 32;
  // per step: A is 128 rows x 4 chunks (2 per thread), B 384 rows x 4 (6 per thread)
  uint4 ra[2], rb[6];
  auto gload = [&](int ks) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + 256 * j, row = idx >> 2, kk = 32 * ks + 8 * (idx & 3);
      const int64_t t = min(t0 + row, v - 1);
      ra[j] = kk < d ? *reinterpret_cast<const uint4*>(E + t * d + kk) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int idx = tid + 256 * j, pr = idx >> 2, kk = 32 * ks + 8 * (idx & 3);
      const int piece = pr >> 7;
      const int64_t k = min(k0 + (pr & 127), c - 1);
      rb[j] = kk < d ? *reinterpret_cast<const uint4*>(P + ((int64_t)piece * c + k) * d + kk)
                     : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + 256 * j;
      *reinterpret_cast<uint4*>(&sA[buf][(idx >> 2) * kSimLds + 8 * (idx & 3)]) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int idx = tid + 256 * j;
      *reinterpret_cast<uint4*>(&sB[buf][(idx >> 2) * kSimLds + 8 * (idx & 3)]) = rb[j];
    }
  };
  sim_f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = sim_f32x4{0.f, 0.f, 0.f, 0.f};
  gload(0);
  sstore(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nks) gload(ks + 1);
    uint4 af[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      af[m] = *reinterpret_cast<const uint4*>(&sA[buf][(64 * wm + 16 * m + col) * kSimLds + 8 * g]);
#pragma unroll
    for (int piece = 0; piece < 3; ++piece)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint4 bf = *reinterpret_cast<const uint4*>(
            &sB[buf][(kSimTile * piece + 64 * wn + 16 * n + col) * kSimLds + 8 * g]);
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m][n] = sim_mfma(af[m], bf, acc[m][n]);
      }
    if (ks + 1 < nks) sstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + 64 * wm + 16 * m + 4 * g + i;
      if (t >= v) continue;
      const float sc = inv[t];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int64_t k = k0 + 64 * wn + 16 * n + col;
        if (k < c) S[t * c + k] = acc[m][n][i] * sc;
      }
    }
}

// ------------------------------------------------- balanced assignment ---

// Every unassigned token proposes to its most similar non-full cluster
// (ties to the smaller id); sort key = cluster << 32 | (~order(similarity))
// so that an ascending stable sort ranks each cluster's proposals by
// similarity descending, then token id ascending.  Assigned tokens get the
// largest key.  One wave per token.
__global__ __launch_bounds__(256) void k_propose(const float* __restrict__ S, int64_t v, int64_t c,
                                                 const int32_t* __restrict__ asg,
                                                 const int32_t* __restrict__ fill, int b,
                                                 uint64_t* __restrict__ keys,
                                                 int32_t* __restrict__ vals) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= v) return;
  if (asg[t] >= 0) {
    if (lane == 0) {
      keys[t] = ~0ull;
      vals[t] = (int32_t)t;
    }
    return;
  }
  const float* row = S + t * c;
  float best = 0.f;
  int64_t bk = -1;
  for (int64_t k = lane; k < c; k += 64) {
    if (fill[k] >= b) continue;
    const float x = row[k];
    if (bk < 0 || x > best) {  // ascending k per lane: keeps the smaller id on ties
      best = x;
      bk = k;
    }
  }
  // wave arg-max, ties to the smaller cluster id
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ob = __shfl_xor(best, m);
    const int64_t ok = __shfl_xor(bk, m);
    const bool take = ok >= 0 && (bk < 0 || ob > best || (ob == best && ok < bk));
    if (take) {
      best = ob;
      bk = ok;
    }
  }
  if (lane == 0) {
    // no open cluster cannot happen while the counts agree (v = b c); the
    // largest key keeps such a token out of every segment regardless
    const uint32_t ord = ordered_bits(best);
    keys[t] = bk < 0 ? ~0ull : ((uint64_t)bk << 32) | (uint64_t)(0xFFFFFFFFu - ord);
    vals[t] = (int32_t)t;
  }
}

// start[k] = first sorted position of cluster k's proposals.
__global__ __launch_bounds__(256) void k_segment_starts(const uint64_t* __restrict__ keys, int64_t n,
                                                        int32_t* __restrict__ start) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint64_t k = keys[i] >> 32;
  if (keys[i] == ~0ull) return;
  if (i == 0 || (keys[i - 1] >> 32) != k) start[k] = (int32_t)i;
}

// The first (b - fill[k]) proposals of cluster k in sorted order are taken.
__global__ __launch_bounds__(256) void k_accept(const uint64_t* __restrict__ keys,
                                                const int32_t* __restrict__ vals, int64_t n,
                                                const int32_t* __restrict__ start,
                                                const int32_t* __restrict__ fill, int b,
                                                int32_t* __restrict__ asg,
                                                int32_t* __restrict__ taken) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n || keys[i] == ~0ull) return;
  const int64_t k = (int64_t)(keys[i] >> 32);
  if (i - start[k] < b - fill[k]) {
    asg[vals[i]] = (int32_t)k;
    atomicAdd(&taken[k], 1);  // integer counts: order does not matter
  }
}

__global__ __launch_bounds__(256) void k_fill_update(int32_t* __restrict__ fill,
                                                     int32_t* __restrict__ taken, int64_t c,
                                                     int32_t* __restrict__ total) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= c) return;
  if (taken[k]) {
    fill[k] += taken[k];
    atomicAdd(total, taken[k]);
    taken[k] = 0;
  }
}

__global__ __launch_bounds__(256) void k_iota(int32_t* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = (int32_t)i;
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t* __restrict__ x, int64_t n, int32_t val) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = val;
}

// --------------------------------------------------------------- update ---

// C_k = normalise(sum_j X[c2t[k][j]]) in slot order; one wave per cluster.
__global__ __launch_bounds__(256) void k_centroids(const float* __restrict__ X, int d,
                                                   const int32_t* __restrict__ c2t, int64_t c,
                                                   int b, float* __restrict__ C) {
  const int lane = threadIdx.x & 63;
  const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (k >= c) return;
  float ss = 0.f;
  for (int i = lane; i < d; i += 64) {
    float s = 0.f;
    for (int j = 0; j < b; ++j) s += X[(int64_t)c2t[k * b + j] * d + i];
    C[k * d + i] = s;
    ss = fmaf(s, s, ss);
  }
  ss = wave_sum(ss);
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  for (int i = lane; i < d; i += 64) C[k * d + i] *= inv;
}

// ----------------------------------------------------------------- host ---

static unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

struct ClusterWork {
  int64_t v = 0, c = 0;
  uint64_t* keys = nullptr;
  uint64_t* keys2 = nullptr;
  int32_t* vals = nullptr;
  int32_t* vals2 = nullptr;
  int32_t* fill = nullptr;
  int32_t* taken = nullptr;
  int32_t* start = nullptr;
  int32_t* total = nullptr;  // tokens assigned so far
  void* temp = nullptr;
  size_t temp_bytes = 0;
};

// Bits that hold every cluster id in [0, c).
static int cluster_bits(int64_t c) {
  int bits = 1;
  while ((int64_t(1) << bits) < c) ++bits;
  return bits;
}

static hipError_t work_alloc(ClusterWork& w, int64_t v, int64_t c, hipStream_t st) {
  w.v = v;
  w.c = c;
  hipError_t r = hipMalloc((void**)&w.keys, sizeof(uint64_t) * v);
  if (r == hipSuccess) r = hipMalloc((void**)&w.keys2, sizeof(uint64_t) * v);
  if (r == hipSuccess) r = hipMalloc((void**)&w.vals, sizeof(int32_t) * v);
  if (r == hipSuccess) r = hipMalloc((void**)&w.vals2, sizeof(int32_t) * v);
  if (r == hipSuccess) r = hipMalloc((void**)&w.fill, sizeof(int32_t) * c);
  if (r == hipSuccess) r = hipMalloc((void**)&w.taken, sizeof(int32_t) * c);
  if (r == hipSuccess) r = hipMalloc((void**)&w.start, sizeof(int32_t) * c);
  if (r == hipSuccess) r = hipMalloc((void**)&w.total, sizeof(int32_t));
  if (r != hipSuccess) return r;
  size_t b1 = 0, b2 = 0;
  r = hipcub::DeviceRadixSort::SortPairs(nullptr, b1, w.keys, w.keys2, w.vals, w.vals2, (int)v, 0,
                                         64, st);
  if (r == hipSuccess)
    r = hipcub::DeviceRadixSort::SortPairs(nullptr, b2, reinterpret_cast<uint32_t*>(w.vals),
                                           reinterpret_cast<uint32_t*>(w.vals2), w.vals, w.vals2,
                                           (int)v, 0, cluster_bits(c), st);
  if (r != hipSuccess) return r;
  w.temp_bytes = std::max(b1, b2);
  return hipMalloc(&w.temp, w.temp_bytes);
}

static void work_free(ClusterWork& w) {
  for (void* p : {(void*)w.keys, (void*)w.keys2, (void*)w.vals, (void*)w.vals2, (void*)w.fill,
                  (void*)w.taken, (void*)w.start, (void*)w.total, w.temp})
    (void)hipFree(p);
  w = ClusterWork{};
}

// The rounds; asg must hold -1 for every token on entry.  Returns the
// number of rounds in *rounds.
static hipError_t assign_rounds(const float* S, int64_t v, int64_t c, int32_t* asg, ClusterWork& w,
                                hipStream_t st, int* rounds) {
  const int b = (int)(v / c);
  hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(c, 256)), dim3(256), 0, st, w.fill, c, 0);
  hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(c, 256)), dim3(256), 0, st, w.taken, c, 0);
  hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, st, w.total, (int64_t)1, 0);
  hipError_t r = hipGetLastError();
  int done = 0, n = 0;
  while (r == hipSuccess && done < v) {
    if (++n > v + 1) return hipErrorUnknown;  // every round assigns at least one token
    hipLaunchKernelGGL(k_propose, dim3(blocks_for(v, 4)), dim3(256), 0, st, S, v, c, asg, w.fill, b,
                       w.keys, w.vals);
    r = hipGetLastError();
    if (r != hipSuccess) break;
    size_t tb = w.temp_bytes;
    r = hipcub::DeviceRadixSort::SortPairs(w.temp, tb, w.keys, w.keys2, w.vals, w.vals2, (int)v, 0,
                                           64, st);
    if (r != hipSuccess) break;
    hipLaunchKernelGGL(k_segment_starts, dim3(blocks_for(v, 256)), dim3(256), 0, st, w.keys2, v,
                       w.start);
    hipLaunchKernelGGL(k_accept, dim3(blocks_for(v, 256)), dim3(256), 0, st, w.keys2, w.vals2, v,
                       w.start, w.fill, b, asg, w.taken);
    hipLaunchKernelGGL(k_fill_update, dim3(blocks_for(c, 256)), dim3(256), 0, st, w.fill, w.taken,
                       c, w.total);
    r = hipGetLastError();
    if (r == hipSuccess) r = hipMemcpyAsync(&done, w.total, sizeof(int), hipMemcpyDeviceToHost, st);
    if (r == hipSuccess) r = hipStreamSynchronize(st);
  }
  if (rounds) *rounds = n;
  return r;
}

// C2T by a stable sort of token ids on their cluster, then the centroids.
static hipError_t update_step(const float* X, int64_t v, int d, int64_t c, const int32_t* asg,
                              int32_t* c2t, float* C, ClusterWork& w, hipStream_t st) {
  hipLaunchKernelGGL(k_iota, dim3(blocks_for(v, 256)), dim3(256), 0, st, w.vals, v);
  hipError_t r = hipGetLastError();
  if (r != hipSuccess) return r;
  size_t tb = w.temp_bytes;
  const int end_bit = cluster_bits(c);
  // cluster ids are non-negative: sort them as unsigned keys
  r = hipcub::DeviceRadixSort::SortPairs(w.temp, tb, reinterpret_cast<const uint32_t*>(asg),
                                         reinterpret_cast<uint32_t*>(w.vals2), w.vals, c2t, (int)v,
                                         0, end_bit, st);
  if (r != hipSuccess) return r;
  hipLaunchKernelGGL(k_centroids, dim3(blocks_for(c, 4)), dim3(256), 0, st, X, d, c2t, c,
                     (int)(v / c), C);
  return hipGetLastError();
}

template <typename T>
static hipError_t pp_step_dispatch(const T* E, const float* inv, int64_t v, int d,
                                   const int32_t* centers, int i, float* D, double* part,
                                   int64_t nb, hipStream_t st) {
  const int maxm = (d / Chunk<T>::kElems + 63) / 64;
  const dim3 grid((unsigned)nb), block(256);
  if (maxm <= 1)
    hipLaunchKernelGGL((k_pp_step<T, 1>), grid, block, 0, st, E, inv, v, d, centers, i, D, part);
  else if (maxm <= 2)
    hipLaunchKernelGGL((k_pp_step<T, 2>), grid, block, 0, st, E, inv, v, d, centers, i, D, part);
  else if (maxm <= 4)
    hipLaunchKernelGGL((k_pp_step<T, 4>), grid, block, 0, st, E, inv, v, d, centers, i, D, part);
  else if (maxm <= 8)
    hipLaunchKernelGGL((k_pp_step<T, 8>), grid, block, 0, st, E, inv, v, d, centers, i, D, part);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

static hipError_t launch_pp_step(const void* E, bool bf16, const float* inv, int64_t v, int d,
                                 const int32_t* centers, int i, float* D, double* part, int64_t nb,
                                 hipStream_t st) {
  return bf16 ? pp_step_dispatch(static_cast<const uint16_t*>(E), inv, v, d, centers, i, D, part,
                                 nb, st)
              : pp_step_dispatch(static_cast<const float*>(E), inv, v, d, centers, i, D, part, nb,
                                 st);
}

hipError_t balanced_assign_device(const float* S, int64_t v, int64_t c, int32_t* asg,
                                  hipStream_t st, int* rounds) {
  ClusterWork w;
  hipError_t r = work_alloc(w, v, c, st);
  if (r == hipSuccess) {
    hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(v, 256)), dim3(256), 0, st, asg, v, -1);
    r = hipGetLastError();
  }
  if (r == hipSuccess) r = assign_rounds(S, v, c, asg, w, st, rounds);
  if (r == hipSuccess) r = hipStreamSynchronize(st);
  work_free(w);
  return r;
}

hipError_t kmeans_device(const void* E, bool bf16, int64_t v, int d, int64_t c, int iters,
                         const double* u, float* C, int32_t* c2t, int32_t* init, int32_t* asg_out,
                         hipStream_t st, ClusterTimes* times) {
  float* X = nullptr;
  float* inv = nullptr;
  float* D = nullptr;
  double* part = nullptr;
  float* S = nullptr;
  int32_t* centers = nullptr;
  int32_t* asg = nullptr;
  uint16_t* pieces = nullptr;  // bf16 tables: the three bf16 pieces of C
  ClusterWork w;
  hipEvent_t ev[5] = {};
  hipError_t r = hipSuccess;
  for (auto& e : ev)
    if (r == hipSuccess) r = hipEventCreate(&e);
  if (r == hipSuccess) r = hipMalloc((void**)&X, sizeof(float) * v * d);
  const int64_t nb = (v + kPpRows - 1) / kPpRows;
  if (r == hipSuccess) r = hipMalloc((void**)&inv, sizeof(float) * v);
  if (r == hipSuccess) r = hipMalloc((void**)&D, sizeof(float) * v);
  // k_pp_step's partials, 1024 x ceil(nb / 1024) slots (see k_pp_pick)
  if (r == hipSuccess) r = hipMalloc((void**)&part, sizeof(double) * 1024 * ((nb + 1023) / 1024));
  if (r == hipSuccess) r = hipMalloc((void**)&S, sizeof(float) * v * c);
  if (r == hipSuccess) r = hipMalloc((void**)&centers, sizeof(int32_t) * c);
  if (r == hipSuccess) r = hipMalloc((void**)&asg, sizeof(int32_t) * v);
  if (r == hipSuccess && bf16) r = hipMalloc((void**)&pieces, sizeof(uint16_t) * 3 * c * d);
  if (r == hipSuccess) r = work_alloc(w, v, c, st);
  int total_rounds = 0;
  if (r == hipSuccess) r = hipEventRecord(ev[0], st);
  if (r == hipSuccess) {
    if (bf16)
      hipLaunchKernelGGL((k_normalize_rows<uint16_t>), dim3(blocks_for(v, 4)), dim3(256), 0, st,
                         static_cast<const uint16_t*>(E), v, d, X, inv);
    else
      hipLaunchKernelGGL((k_normalize_rows<float>), dim3(blocks_for(v, 4)), dim3(256), 0, st,
                         static_cast<const float*>(E), v, d, X, inv);
    r = hipGetLastError();
    const int32_t first = (int32_t)std::min<int64_t>((int64_t)(u[0] * (double)v), v - 1);
    if (r == hipSuccess)
      r = hipMemcpyAsync(centers, &first, sizeof(int32_t), hipMemcpyHostToDevice, st);
    // every 16th distance refresh is bracketed by an event pair
    constexpr int64_t kSample = 16;
    // the host waits for the stream every kDrain centres, so that at most
    // 2 kDrain launches and kDrain / 8 event records are ever queued (a
    // single wait after all c centres queued 2c launches: 16 000 at the
    // Llama-3.2-1B shape, too many for tools that instrument each launch)
    constexpr int64_t kDrain = 256;
    std::vector<hipEvent_t> sev(2 * ((c + kSample - 1) / kSample), nullptr);
    for (auto& e : sev)
      if (r == hipSuccess) r = hipEventCreate(&e);
    for (int64_t i = 0; r == hipSuccess && i < c; ++i) {
      if (i > 0) {
        hipLaunchKernelGGL(k_pp_pick, dim3(1), dim3(1024), 0, st, D, part, nb, v, u[i],
                           centers, (int)i);
        r = hipGetLastError();
      }
      const bool sample = i % kSample == 0;
      if (r == hipSuccess && sample) r = hipEventRecord(sev[2 * (i / kSample)], st);
      if (r == hipSuccess) r = launch_pp_step(E, bf16, inv, v, d, centers, (int)i, D, part, nb, st);
      if (r == hipSuccess && sample) r = hipEventRecord(sev[2 * (i / kSample) + 1], st);
      if (r == hipSuccess && (i + 1) % kDrain == 0) r = hipStreamSynchronize(st);
    }
    if (r == hipSuccess) r = hipStreamSynchronize(st);
    double step_ms = 0.0;
    for (size_t j = 0; r == hipSuccess && j < sev.size(); j += 2) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, sev[j], sev[j + 1]) == hipSuccess) step_ms += ms;
    }
    if (times) times->pp_step_us = (float)(1e3 * step_ms / (double)(sev.size() / 2));
    for (auto& e : sev)
      if (e) (void)hipEventDestroy(e);
    if (r == hipSuccess) {
      hipLaunchKernelGGL(k_gather_rows, dim3(blocks_for(c * d, 256)), dim3(256), 0, st, X, d,
                         centers, c, C);
      r = hipGetLastError();
    }
    if (r == hipSuccess) r = hipEventRecord(ev[1], st);
    if (r == hipSuccess && init)
      r = hipMemcpyAsync(init, centers, sizeof(int32_t) * c, hipMemcpyDeviceToDevice, st);
    float sims_ms = 0.f;
    for (int it = 0; r == hipSuccess && it < iters; ++it) {
      r = hipEventRecord(ev[2], st);
      if (r != hipSuccess) break;
      if (bf16) {
        hipLaunchKernelGGL(k_split_pieces, dim3(blocks_for(c * d, 256)), dim3(256), 0, st, C, c * d,
                           pieces);
        hipLaunchKernelGGL(k_sims_mfma, dim3(blocks_for(v, kSimTile), blocks_for(c, kSimTile)),
                           dim3(256), 0, st, static_cast<const uint16_t*>(E), inv, v, d, pieces, c,
                           S);
      } else {
        hipLaunchKernelGGL(k_sims, dim3(blocks_for(v, 64), blocks_for(c, 64)), dim3(256), 0, st, X,
                           v, C, c, d, S);
      }
      r = hipGetLastError();
      if (r == hipSuccess) r = hipEventRecord(ev[3], st);
      if (r != hipSuccess) break;
      hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(v, 256)), dim3(256), 0, st, asg, v, -1);
      r = hipGetLastError();
      int rounds = 0;
      if (r == hipSuccess) r = assign_rounds(S, v, c, asg, w, st, &rounds);
      total_rounds += rounds;
      float ms = 0.f;
      if (r == hipSuccess && hipEventElapsedTime(&ms, ev[2], ev[3]) == hipSuccess) sims_ms += ms;
      if (r == hipSuccess) r = update_step(X, v, d, c, asg, c2t, C, w, st);
    }
    if (r == hipSuccess && asg_out)
      r = hipMemcpyAsync(asg_out, asg, sizeof(int32_t) * v, hipMemcpyDeviceToDevice, st);
    if (r == hipSuccess) r = hipEventRecord(ev[4], st);
    if (r == hipSuccess) r = hipStreamSynchronize(st);
    if (times && r == hipSuccess) {
      float ms = 0.f;
      (void)hipEventElapsedTime(&ms, ev[0], ev[1]);
      times->init_ms = ms;
      ms = 0.f;
      (void)hipEventElapsedTime(&ms, ev[0], ev[4]);
      times->total_ms = ms;
      times->sims_ms = sims_ms;
      times->rounds = total_rounds;
    }
  }
  for (auto& e : ev)
    if (e) (void)hipEventDestroy(e);
  work_free(w);
  for (void* p : {(void*)X, (void*)inv, (void*)D, (void*)part, (void*)S,
                  (void*)centers, (void*)asg, (void*)pieces})
    (void)hipFree(p);
  return r;
}

}  // namespace fh
