// FlashHead kernels for gfx950 (MI355X): INT4 centroid quantisation, row
// GEMV (stage-1 scores, stage-2 gather-score, dense head) with a fused
// max / log-sum-exp / Gumbel epilogue, probe selection, and the finisher.
//
// Sources (page title and section): FlashHead technical explainer
// (framerc.cn) §1.1, §1.2.1-§1.2.4, §2.2.2, §2.3; "FlashHead: Efficient
// Drop-In Replacement for the Classification Head in Language Model
// Inference" (arXiv 2603.14591), abstract.

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "fh_device.hpp"
#include "fh_internal.hpp"

namespace fh {

// ======================================================================
// INT4 g32 quantisation of the centroids (explainer §1.2.4, §2.3).
// One thread per (row, group of 32 consecutive elements).  sigma is
// fp16(amax / 7) with an IEEE float32 division and round-to-nearest-even to
// fp16; q = clamp(rint(x / sigma), -7, 7) with float32 division (rint ties
// to even); q = 0 where sigma = 0.  Nibbles are packed two's-complement,
// element 2m in the low nibble of byte m.  *bad is set if a scale overflows.
// ======================================================================
template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

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
// Row GEMV with an optional fused epilogue.
//
// Each wave owns RPW consecutive "rows" of the problem and computes, for NQ
// queries, z = M[r] . h_q with M[r] a 16-byte-chunked row of d elements.
// Lane l handles chunks l, l+64, ... (MAXM of them at most), so one row is
// read as fully coalesced 16-byte loads and the lane's slice of h stays in
// registers for all of the wave's rows.  Rows are processed two at a time to
// keep two rows' loads in flight per wave.
//
//   GATHER = false: row r is M's row r (stage 1 over C; the dense head over E).
//   GATHER = true : row r of query q is token t = C2T[S[q, r / b], r % b] of
//                   E (stage 2: retrieved token scoring, explainer §1.2.4).
//   EPI: the wave also folds each (z, t) into a running Part (best key, its
//        logit, and max / sum-exp of z / T'), merged per workgroup and written
//        to parts[q * gridDim.x + blockIdx.x] for the finisher.
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
  float temperature;  // T' (1 unless tokens are sampled)
  uint64_t seed;
  Part* parts;  // [B x gridDim.x] or null
};

template <typename T, int MAXM, int NQ, int RPW, bool GATHER, bool EPI>
__global__ __launch_bounds__(256) void k_rows(RowsArgs a) {
  constexpr int EPC = Chunk<T>::kElems;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nch = a.d / EPC;
  const int q0 = blockIdx.y * NQ;
  const int nq = min(NQ, a.B - q0);
  const T* Mp = static_cast<const T*>(a.M);
  const T* Hp = static_cast<const T*>(a.H);

  // the lane's slice of h for each query
  uint4 hv[NQ][MAXM];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const uint4* hq = reinterpret_cast<const uint4*>(Hp + (int64_t)(q0 + min(q, nq - 1)) * a.d);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      const int ch = lane + 64 * m;
      hv[q][m] = ch < nch ? hq[ch] : uint4{0u, 0u, 0u, 0u};
    }
  }

  Part part[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) part[q] = part_empty();

  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
#pragma unroll 1
  for (int i = 0; i < RPW; i += 2) {
    int64_t rr[2];
    int64_t src[2];
    bool ok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      rr[u] = r0 + i + u;
      ok[u] = (i + u < RPW) && rr[u] < a.nrows;
      src[u] = 0;
      if (ok[u]) {
        if (GATHER) {
          const int k = a.S[(int64_t)q0 * a.ldS + rr[u] / a.bsz];
          src[u] = a.c2t[(int64_t)k * a.bsz + rr[u] % a.bsz];
        } else {
          src[u] = rr[u];
        }
      }
    }
    uint4 mv[2][MAXM];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4* row = reinterpret_cast<const uint4*>(Mp + src[u] * a.d);
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {
        const int ch = lane + 64 * m;
        mv[u][m] = (ok[u] && ch < nch) ? row[ch] : uint4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!ok[u]) continue;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q >= nq) break;
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc = Chunk<T>::dot(mv[u][m], hv[q][m], acc);
        const float z = wave_sum(acc);
        const int64_t oq = (int64_t)(q0 + q);
        if (lane == 0) {
          if (a.out_vals) a.out_vals[oq * a.ld_vals + rr[u]] = z;
          if (GATHER && a.out_ids) a.out_ids[oq * a.ld_vals + rr[u]] = (int32_t)src[u];
        }
        if (EPI) {
          const int32_t t = (int32_t)src[u];
          float key = z;
          if (a.token_sample) key = z / a.temperature + gumbel_at(a.seed, (uint32_t)oq, (uint32_t)t, 1u);
          const Part one{key, z, z / a.temperature, 1.f, t};
          part[q] = part_merge(part[q], one);
        }
      }
    }
  }

  if (EPI) {
    __shared__ Part sp[4][NQ];
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) sp[wave][q] = part[q];
    }
    __syncthreads();
    if (threadIdx.x < nq) {
      const int q = threadIdx.x;
      Part acc = sp[0][q];
      for (int w = 1; w < 4; ++w) acc = part_merge(acc, sp[w][q]);
      a.parts[(int64_t)(q0 + q) * gridDim.x + blockIdx.x] = acc;
    }
  }
}

// ======================================================================
// INT4 stage-1 GEMV: s[q, k] = sum_g sigma[k, g] * sum_{i in g} q[k, i] h[i].
// Lane l owns groups l, l+64, ...: one 16-byte load is exactly one group's
// 32 nibbles.  Nibbles are turned into unsigned bytes u = q + 8 (xor with
// 0x88888888 then two masks), converted with cvt_f32_ubyte, and the offset
// is removed with the group sum of h: sum q h = sum u h - 8 sum h.
// ======================================================================
template <typename T, int MAXG, int NQ, int RPW>
__global__ __launch_bounds__(256) void k_score_int4(const uint8_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ SG, int64_t c,
                                                    int d, const T* __restrict__ H, int B,
                                                    float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = d / 32;
  const int q0 = blockIdx.y * NQ;
  const int nq = min(NQ, B - q0);

  float hf[NQ][MAXG][32];
  float hsum[NQ][MAXG];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const T* hq = H + (int64_t)(q0 + min(q, nq - 1)) * d;
#pragma unroll
    for (int m = 0; m < MAXG; ++m) {
      const int g = lane + 64 * m;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        hf[q][m][i] = g < G ? load_elem<T>(hq, (int64_t)g * 32 + i) : 0.f;
        s += hf[q][m][i];
      }
      hsum[q][m] = s;
    }
  }

  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
#pragma unroll 1
  for (int i = 0; i < RPW; ++i) {
    const int64_t row = r0 + i;
    if (row >= c) break;
    uint4 qv[MAXG];
    float sg[MAXG];
    const uint4* qrow = reinterpret_cast<const uint4*>(Q + row * (d / 2));
#pragma unroll
    for (int m = 0; m < MAXG; ++m) {
      const int g = lane + 64 * m;
      qv[m] = g < G ? qrow[g] : uint4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
      sg[m] = g < G ? __half2float(__ushort_as_half(SG[row * G + g])) : 0.f;
    }
    float acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
#pragma unroll
    for (int m = 0; m < MAXG; ++m) {
      const uint32_t w4[4] = {qv[m].x ^ 0x88888888u, qv[m].y ^ 0x88888888u,
                              qv[m].z ^ 0x88888888u, qv[m].w ^ 0x88888888u};
      float u[32];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = w4[j] & 0x0F0F0F0Fu;         // nibbles 0,2,4,6
        const uint32_t hi = (w4[j] >> 4) & 0x0F0F0F0Fu;  // nibbles 1,3,5,7
        u[8 * j + 0] = (float)(lo & 0xFFu);
        u[8 * j + 1] = (float)(hi & 0xFFu);
        u[8 * j + 2] = (float)((lo >> 8) & 0xFFu);
        u[8 * j + 3] = (float)((hi >> 8) & 0xFFu);
        u[8 * j + 4] = (float)((lo >> 16) & 0xFFu);
        u[8 * j + 5] = (float)((hi >> 16) & 0xFFu);
        u[8 * j + 6] = (float)(lo >> 24);
        u[8 * j + 7] = (float)(hi >> 24);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) t = fmaf(u[e], hf[q][m][e], t);
        acc[q] = fmaf(sg[m], fmaf(-8.f, hsum[q][m], t), acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q >= nq) break;
      const float s = wave_sum(acc[q]);
      if (lane == 0) out[(int64_t)(q0 + q) * c + row] = s;
    }
  }
}

// ======================================================================
// Probe selection (explainer §1.2.2 top-p, §1.2.3 multinomial probes).
//
// One 1024-thread workgroup per query.  Thread t holds keys of clusters
// [t*KPT, t*KPT + KPT) in registers: key = s (TOPK) or s/T + G(seed, q, k, 0)
// (SAMPLE: the top p of Gumbel-perturbed keys are p draws without
// replacement from softmax(s/T)).  The p-th largest key is found by repeated
// bucketing: the active key range [lo, hi] is cut into 2048 equal buckets
// (a monotone map, lo -> bucket 0, hi -> bucket 2047), a histogram and a
// suffix scan locate the bucket holding the boundary, keys above it are
// taken, keys below are dropped, and the boundary bucket becomes the next
// range.  When all remaining keys are equal the smallest ids are taken.  The
// chosen clusters are written in ascending id with a block prefix sum.
// Non-finite keys are saturated to +-FLT_MAX (NaN to -FLT_MAX).
// ======================================================================
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelBins = 2048;

__device__ __forceinline__ float block_min(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_min(x);
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kSelWaves; ++w) r = fminf(r, red[w]);
  return r;
}

__device__ __forceinline__ float block_max(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_max(x);
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kSelWaves; ++w) r = fmaxf(r, red[w]);
  return r;
}

// Exclusive prefix sum over threads in index order; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int x, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(x, lane);
  __syncthreads();
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    const int v = red[w];
    if (w < wave) before += v;
    tot += v;
  }
  *total = tot;
  return before + inc - x;
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ scores, int c,
                                                        int p, int sample, float temperature,
                                                        uint64_t seed, int32_t* __restrict__ S,
                                                        int ldS) {
  __shared__ int hist[kSelBins];
  __shared__ float redf[kSelWaves];
  __shared__ int redi[kSelWaves];
  __shared__ int s_beta, s_above, s_cnt;
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int base = tid * KPT;
  const float* sq = scores + (int64_t)q * c;

  float key[KPT];
  uint32_t act = 0u, sel = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int k = base + i;
    float x = -FLT_MAX;
    if (k < c) {
      x = sq[k];
      if (sample) x = x / temperature + gumbel_at(seed, (uint32_t)q, (uint32_t)k, 0u);
      if (isnan(x)) x = -FLT_MAX;
      x = fminf(fmaxf(x, -FLT_MAX), FLT_MAX);
      act |= 1u << i;
    }
    key[i] = x;
  }

  int need = p;
  int cnt_act = 0;
  {
    int tot;
    (void)block_exclusive_scan(__popc(act), redi, &tot);
    cnt_act = tot;
  }
  if (need >= cnt_act) {
    sel = act;
    need = 0;
  }
  float lo = 0.f, hi = 0.f;
  if (need > 0) {
    float mn = FLT_MAX, mx = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (act & (1u << i)) { mn = fminf(mn, key[i]); mx = fmaxf(mx, key[i]); }
    lo = block_min(mn, redf);
    hi = block_max(mx, redf);
  }

  while (need > 0) {
    if (!(lo < hi)) {
      // every active key is equal: take the `need` smallest ids
      int tot;
      const int before = block_exclusive_scan(__popc(act), redi, &tot);
      int rank = before;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (act & (1u << i)) {
          if (rank < need) sel |= 1u << i;
          ++rank;
        }
      }
      need = 0;
      break;
    }
    const double dlo = (double)lo;
    const double scale = (double)kSelBins / ((double)hi - dlo);
    for (int i = tid; i < kSelBins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    int bin[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      bin[i] = -1;
      if (act & (1u << i)) {
        bin[i] = min(kSelBins - 1, (int)(((double)key[i] - dlo) * scale));
        atomicAdd(&hist[bin[i]], 1);
      }
    }
    __syncthreads();
    // suffix counts: thread t covers buckets jb = 2047-2t and 2046-2t, in
    // descending bucket order
    const int j0 = kSelBins - 1 - 2 * tid, j1 = j0 - 1;
    const int h0 = hist[j0], h1 = hist[j1];
    int tot;
    const int before = block_exclusive_scan(h0 + h1, redi, &tot);
    // keys in buckets above jb: before (+h0 for j1)
    if (before < need && before + h0 >= need) {
      s_beta = j0; s_above = before; s_cnt = h0;
    } else if (before + h0 < need && before + h0 + h1 >= need) {
      s_beta = j1; s_above = before + h0; s_cnt = h1;
    }
    __syncthreads();
    const int beta = s_beta, above = s_above, cntb = s_cnt;
    need -= above;
    float mn = FLT_MAX, mx = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (!(act & (1u << i))) continue;
      if (bin[i] > beta) {
        sel |= 1u << i;
        act &= ~(1u << i);
      } else if (bin[i] < beta) {
        act &= ~(1u << i);
      } else {
        mn = fminf(mn, key[i]);
        mx = fmaxf(mx, key[i]);
      }
    }
    if (cntb == need) {
      sel |= act;
      act = 0u;
      need = 0;
      break;
    }
    lo = block_min(mn, redf);
    hi = block_max(mx, redf);
  }

  int tot;
  int off = block_exclusive_scan(__popc(sel), redi, &tot);
  int32_t* Sq = S + (int64_t)q * ldS;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (sel & (1u << i)) Sq[off++] = base + i;
}

// ======================================================================
// Finisher: merge a query's per-workgroup Parts in a fixed order.
// ======================================================================
__global__ __launch_bounds__(256) void k_finish(const Part* __restrict__ parts, int nparts,
                                                int32_t* __restrict__ out_token,
                                                float* __restrict__ out_logit,
                                                float* __restrict__ out_lse) {
  __shared__ Part sp[256];
  const int q = blockIdx.x;
  const Part* pq = parts + (int64_t)q * nparts;
  Part acc = part_empty();
  for (int i = threadIdx.x; i < nparts; i += 256) acc = part_merge(acc, pq[i]);
  sp[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sp[threadIdx.x] = part_merge(sp[threadIdx.x], sp[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const Part r = sp[0];
    if (out_token) out_token[q] = r.id;
    if (out_logit) out_logit[q] = r.z;
    if (out_lse) out_lse[q] = r.m + logf(r.s);
  }
}

// ======================================================================
// Host-side launchers
// ======================================================================

template <typename T, int NQ, int RPW, bool GATHER, bool EPI>
static hipError_t launch_rows_m(int maxm, dim3 grid, const RowsArgs& a, hipStream_t st) {
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

template <typename T, int NQ, int RPW, bool GATHER, bool EPI>
static hipError_t launch_rows(const RowsArgs& a, hipStream_t st, int64_t* nblocks) {
  const int nch = a.d / Chunk<T>::kElems;
  const int maxm = (nch + 63) / 64;
  const int64_t rows_per_block = 4 * RPW;
  const int64_t gx = (a.nrows + rows_per_block - 1) / rows_per_block;
  const int gy = GATHER ? a.B : (a.B + NQ - 1) / NQ;
  if (nblocks) *nblocks = gx;
  if (gx <= 0 || gy <= 0) return hipSuccess;
  return launch_rows_m<T, NQ, RPW, GATHER, EPI>(maxm, dim3((unsigned)gx, (unsigned)gy), a, st);
}

int64_t rows_blocks(int64_t nrows, int rpw) { return (nrows + 4 * rpw - 1) / (4 * rpw); }

template <typename T>
static hipError_t score_dispatch(const KernelCtx& k, const void* h, int B, float* out) {
  RowsArgs a{};
  a.M = k.C; a.nrows = k.c; a.d = k.d; a.H = h; a.B = B; a.out_vals = out; a.ld_vals = k.c;
  a.temperature = 1.f;
  if (B == 1) return launch_rows<T, 1, kScoreRPW, false, false>(a, k.stream, nullptr);
  if (B == 2) return launch_rows<T, 2, kScoreRPW, false, false>(a, k.stream, nullptr);
  return launch_rows<T, 4, kScoreRPW, false, false>(a, k.stream, nullptr);
}

hipError_t launch_score(const KernelCtx& k, const void* h, int B, float* out) {
  return k.bf16 ? score_dispatch<uint16_t>(k, h, B, out) : score_dispatch<float>(k, h, B, out);
}

template <typename T, int NQ>
static hipError_t int4_m(const KernelCtx& k, const void* h, int B, float* out) {
  const int G = k.d / 32;
  const int maxg = (G + 63) / 64;
  const int64_t gx = (k.c + 4 * kInt4RPW - 1) / (4 * kInt4RPW);
  const dim3 grid((unsigned)gx, (unsigned)((B + NQ - 1) / NQ));
  const T* hp = static_cast<const T*>(h);
  switch (maxg) {
    case 1: hipLaunchKernelGGL((k_score_int4<T, 1, NQ, kInt4RPW>), grid, dim3(256), 0, k.stream, k.cq, k.csig, k.c, k.d, hp, B, out); break;
    case 2: hipLaunchKernelGGL((k_score_int4<T, 2, NQ, kInt4RPW>), grid, dim3(256), 0, k.stream, k.cq, k.csig, k.c, k.d, hp, B, out); break;
    case 3: hipLaunchKernelGGL((k_score_int4<T, 3, NQ, kInt4RPW>), grid, dim3(256), 0, k.stream, k.cq, k.csig, k.c, k.d, hp, B, out); break;
    case 4: hipLaunchKernelGGL((k_score_int4<T, 4, NQ, kInt4RPW>), grid, dim3(256), 0, k.stream, k.cq, k.csig, k.c, k.d, hp, B, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_int4(const KernelCtx& k, const void* h, int B, float* out) {
  if (k.bf16) return B == 1 ? int4_m<uint16_t, 1>(k, h, B, out) : int4_m<uint16_t, 2>(k, h, B, out);
  return B == 1 ? int4_m<float, 1>(k, h, B, out) : int4_m<float, 2>(k, h, B, out);
}

hipError_t launch_quant_int4(const KernelCtx& k, int* bad) {
  const int64_t n = k.c * (k.d / 32);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (k.bf16)
    hipLaunchKernelGGL((k_quant_int4<uint16_t>), grid, dim3(256), 0, k.stream,
                       static_cast<const uint16_t*>(k.C), k.c, k.d, const_cast<uint8_t*>(k.cq), const_cast<uint16_t*>(k.csig), bad);
  else
    hipLaunchKernelGGL((k_quant_int4<float>), grid, dim3(256), 0, k.stream,
                       static_cast<const float*>(k.C), k.c, k.d, const_cast<uint8_t*>(k.cq), const_cast<uint16_t*>(k.csig), bad);
  return hipGetLastError();
}

hipError_t launch_select(const KernelCtx& k, const float* scores, int B, int p, int sample,
                         float temperature, uint64_t seed, int32_t* S, int ldS) {
  const int kpt = (int)((k.c + kSelThreads - 1) / kSelThreads);
  const dim3 grid((unsigned)B), block(kSelThreads);
  const int c = (int)k.c;
  if (kpt <= 1)
    hipLaunchKernelGGL((k_select<1>), grid, block, 0, k.stream, scores, c, p, sample, temperature, seed, S, ldS);
  else if (kpt <= 2)
    hipLaunchKernelGGL((k_select<2>), grid, block, 0, k.stream, scores, c, p, sample, temperature, seed, S, ldS);
  else if (kpt <= 4)
    hipLaunchKernelGGL((k_select<4>), grid, block, 0, k.stream, scores, c, p, sample, temperature, seed, S, ldS);
  else if (kpt <= 8)
    hipLaunchKernelGGL((k_select<8>), grid, block, 0, k.stream, scores, c, p, sample, temperature, seed, S, ldS);
  else if (kpt <= 16)
    hipLaunchKernelGGL((k_select<16>), grid, block, 0, k.stream, scores, c, p, sample, temperature, seed, S, ldS);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
static hipError_t gather_t(const KernelCtx& k, const void* h, int B, const int32_t* S, int p,
                           int token_sample, float tprime, uint64_t seed, int32_t* out_ids,
                           float* out_logits, Part* parts, int64_t* nparts) {
  RowsArgs a{};
  a.M = k.E; a.nrows = (int64_t)p * k.b; a.d = k.d; a.c2t = k.c2t; a.bsz = (int)k.b;
  a.S = S; a.ldS = p; a.H = h; a.B = B; a.out_vals = out_logits; a.ld_vals = a.nrows;
  a.out_ids = out_ids; a.token_sample = token_sample; a.temperature = tprime; a.seed = seed;
  a.parts = parts;
  // gather rows differ per query: one query per grid row (NQ = 1)
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
  a.token_sample = token_sample; a.temperature = tprime; a.seed = seed; a.parts = parts;
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

}  // namespace fh
