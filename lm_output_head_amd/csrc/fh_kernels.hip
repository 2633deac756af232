// FlashHead kernels for gfx950 (MI355X) of the multi-launch path: g32
// centroid quantisation (INT4, INT8), row GEMV (stage-1 scores, stage-2
// gather-score, dense head) with the fused epilogue, probe selection and the
// finisher; plus the host-side launchers.  The single-launch batch-1 kernel
// lives in fh_batch1.inl, the matrix-core paths in fh_mfma.hip.
//
// Sources (page title and section): FlashHead technical explainer
// (framerc.cn) §1.1, §1.2.1-§1.2.4, §2.2.2, §2.3; "FlashHead: Efficient
// Drop-In Replacement for the Classification Head in Language Model
// Inference" (arXiv 2603.14591), abstract.

#include <algorithm>
#include <cmath>

#include "fh_blocks.hpp"

namespace fh {

// ======================================================================
// g32 quantisation of the centroids (explainer §1.2.4, §2.3; INT8 is the
// W8A16 row of §5.2).  One thread per (row, group of 32 consecutive
// elements).  sigma is fp16(amax / qmax) (qmax 7 or 127) with an IEEE float32
// division and round-to-nearest-even to fp16; q = clamp(rint(x / sigma),
// -qmax, qmax) with float32 division (rint ties to even); q = 0 where
// sigma = 0.  INT4 nibbles are packed two's-complement, element 2m in the
// low nibble of byte m; INT8 codes are stored as bytes.  *bad is set if a
// scale overflows.
// ======================================================================
template <typename T, int BITS>
__global__ __launch_bounds__(256) void k_quant_g32(const T* __restrict__ C, int64_t c, int d,
                                                   uint8_t* __restrict__ qout,
                                                   uint16_t* __restrict__ sout,
                                                   int* __restrict__ bad) {
  constexpr int kQmax = BITS == 4 ? 7 : 127;
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
  const __half hs = __float2half_rn(amax / (float)kQmax);
  const float s = __half2float(hs);
  if (!isfinite(s)) atomicOr(bad, 1);
  constexpr int kWords = BITS;  // 32 codes of BITS bits in 32-bit words
  uint32_t words[kWords];
#pragma unroll
  for (int j = 0; j < kWords; ++j) words[j] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int qi = 0;
    if (s > 0.f) qi = (int)fminf(fmaxf(rintf(x[i] / s), (float)-kQmax), (float)kQmax);
    if (BITS == 4)
      words[i >> 3] |= ((uint32_t)qi & 0xFu) << (4 * (i & 7));
    else
      words[i >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (i & 3));
  }
  uint4* dst = reinterpret_cast<uint4*>(qout + row * ((int64_t)d * BITS / 8) + (int64_t)g * 4 * BITS);
#pragma unroll
  for (int j = 0; j < kWords / 4; ++j)
    dst[j] = uint4{words[4 * j], words[4 * j + 1], words[4 * j + 2], words[4 * j + 3]};
  sout[row * G + g] = __half_as_ushort(hs);
}

// ======================================================================
// Cluster-contiguous copy of E (explainer §1.2.1: the C2T table addresses a
// cluster's tokens by slot): Ec[f] = E[C2T[f]] for every slot f, so that a
// probe's b rows are one contiguous block.  One wave per row.
// ======================================================================
__global__ __launch_bounds__(256) void k_permute_rows(const uint4* __restrict__ E,
                                                      const int32_t* __restrict__ c2t,
                                                      uint4* __restrict__ out, int64_t v,
                                                      int nch) {
  const int lane = threadIdx.x & 63;
  const int64_t f = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (f >= v) return;
  const uint4* src = E + (int64_t)c2t[f] * nch;
  uint4* dst = out + f * nch;
  for (int ch = lane; ch < nch; ch += 64) dst[ch] = src[ch];
}

// ======================================================================
// Multi-launch path: row GEMV kernel (any B).
//   GATHER = false: row r is M's row r (stage 1 over C; the dense head over E).
//   GATHER = true : row r of query q is token t = C2T[S[q, r / b], r % b]
//                   (stage 2, explainer §1.2.4), read from the cluster-
//                   contiguous copy of E when there is one; one query per
//                   grid row.
//   EPI: fold each (z, t) into per-query Parts; one Part per workgroup and
//        query goes to parts[q * gridDim.x + blockIdx.x].
// ======================================================================
struct RowsArgs {
  const void* M;
  int64_t nrows;  // rows per query (c, v, or p*b)
  int d;
  const int32_t* c2t;
  bool contiguous;  // GATHER: M is the cluster-contiguous copy of E
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
  KeyXform key;  // stage 1 (neither GATHER nor EPI): scores or selection keys
  const int32_t* nprobe;  // GATHER: probes of each query (its first nprobe[q] of S), or null
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
  LaneParts lp[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) lp[q] = lane_parts_empty();

  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
  int64_t nrows = a.nrows;
  if (GATHER && a.nprobe) nrows = min(nrows, (int64_t)max(a.nprobe[q0], 0) * a.bsz);
  const int64_t r1 = min(r0 + RPW, nrows);
  const int32_t* Sq = GATHER ? a.S + (int64_t)q0 * a.ldS : nullptr;
  // slot f = S[q, r / b] * b + r % b of the clustering; with the
  // cluster-contiguous copy of E that slot is also the row, else the row is
  // the token C2T[f]
  auto src_of = [&](int64_t r) -> int64_t {
    if (!GATHER) return r;
    const int rr = (int)r;  // p b < 2^31
    const int64_t f = (int64_t)Sq[rr / a.bsz] * a.bsz + rr % a.bsz;
    return a.contiguous ? f : (int64_t)a.c2t[f];
  };
  auto tok_of = [&](int64_t src) -> int64_t {
    return GATHER && a.contiguous ? (int64_t)a.c2t[src] : src;
  };
  auto sink = [&](int q, int64_t r, int64_t src, float z) {
    const int64_t oq = q0 + q;
    if (lane == 0) {
      if (a.out_vals)
        a.out_vals[oq * a.ld_vals + r] =
            GATHER || EPI ? z
                          : stage1_value(z, a.key.sample, a.key.temperature, a.key.seed,
                                         (uint32_t)oq, (uint32_t)r);
      if (GATHER && a.out_ids) a.out_ids[oq * a.ld_vals + r] = (int32_t)src;
    }
    if (EPI) lane_parts_add(lp[q], z, (int32_t)src, a.token_sample, a.tprime, a.seed, (uint32_t)oq);
  };
  // rows streamed in order (dense head, scores) take non-temporal loads;
  // gathered rows do not (measured slower with them)
  wave_rows<T, MAXM, NQ, 2, (GATHER ? 0 : kLoadStream)>(static_cast<const T*>(a.M), a.d, lane, hv,
                                                       nq, r0, r1, 1, src_of, tok_of, sink);
  if (EPI) {
    Part part[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      part[q] = lane_parts_finish(lp[q], a.token_sample, a.tprime, a.seed, (uint32_t)(q0 + q));
    const Part wg = block_merge_parts<4, NQ>(part, nq, sh);
    if ((int)threadIdx.x < nq) a.parts[(int64_t)(q0 + threadIdx.x) * gridDim.x + blockIdx.x] = wg;
  }
}

template <typename T, int BITS, int MAXG, int NQ, int RPW>
__global__ __launch_bounds__(256) void k_score_q(const uint8_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ SG, int64_t c,
                                                    int d, const T* __restrict__ H, int B,
                                                    float* __restrict__ out, KeyXform kx) {
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
    if (lane == 0)
      out[(int64_t)(q0 + q) * c + r] =
          stage1_value(s, kx.sample, kx.temperature, kx.seed, (uint32_t)(q0 + q), (uint32_t)r);
  };
  wave_rows_q<BITS, MAXG, NQ>(Q, SG, d, lane, hg, nq, r0, r1, 1, sink);
}

template <int KP>
__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ scores, int c,
                                                        int p, int sample, float temperature,
                                                        uint64_t seed, float zq,
                                                        int32_t* __restrict__ S, int ldS,
                                                        uint32_t* __restrict__ mbits,
                                                        int32_t* __restrict__ mpre) {
  __shared__ SelShared sh;
  FH_TRACE(14);
  const int q = blockIdx.x;
  const float* sq = scores + (int64_t)q * c;
  int32_t* Sq = S + (int64_t)q * ldS;
  select_clear(sh);
  // key = s (top-p), or s/T + G(seed, q, k, 0): the p largest Gumbel-perturbed
  // keys are p draws without replacement from softmax(s/T)
  float x[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int k = (int)threadIdx.x + kSelThreads * i;
    float v = k < c ? sq[k] : 0.f;
    if (sample && k < c) v = v / temperature + gumbel_at(seed, (uint32_t)q, (uint32_t)k, 0u);
    x[i] = k < c ? saturate_key(v) : -FLT_MAX;
  }
  __syncthreads();
  select_bits<KP>(x, c, p, zq, sh);
  emit_selected<KP>(c, [&](int pos, int k) { Sq[pos] = k; }, sh);
  if (mbits) {
    // membership word w of this query, and how many of its probes lie in
    // words before w ([W x B], word-major, for the cluster-major stage 2)
    const int W = (c + 31) / 32, t = threadIdx.x;
    const uint32_t word = t < W ? sh.selbits[t] : 0u;
    int tot;
    const int before = block_exclusive_scan(__popc(word), sh.red_scan, &tot);
    if (t < W) {
      mbits[(int64_t)t * gridDim.x + q] = word;
      mpre[(int64_t)t * gridDim.x + q] = before;
    }
  }
}

// ---- adaptive probe count (explainer §1.2.2, dynamic adjustment of the
// probe count to the query; §4.2, fewer probes for confident queries).
// One workgroup per query, after k_select has taken the top pmax keys (see
// adaptive_count in fh_blocks.hpp for the rule).  S is rewritten in place:
// the n kept probes ascending, then -1; nprobe[q] = n; retrieved slots past
// n b get id -1 and logit -inf; with mbits non-null the kept set also goes
// out as bitset words for the cluster-major stage 2.
struct AdaptShared {
  unsigned long long key[kSelThreads];
  float val[kSelThreads];
  uint32_t keep[kSelMaxC / 32];
  float redf[kSelWaves];
  int red_scan[kSelWaves];
  int red_cnt[kSelWaves];
};

template <int KP>
__global__ __launch_bounds__(kSelThreads) void k_adapt(
    const float* __restrict__ scores, int c, int pmax, int pmin, float tau, int sample,
    float temperature, uint64_t seed, int32_t* __restrict__ S, int32_t* __restrict__ nprobe,
    int b, int32_t* __restrict__ out_ids, float* __restrict__ out_logits,
    uint32_t* __restrict__ mbits, int32_t* __restrict__ mpre) {
  __shared__ AdaptShared sh;
  const int q = blockIdx.x, tid = threadIdx.x;
  const float* sq = scores + (int64_t)q * c;
  int32_t* Sq = S + (int64_t)q * pmax;
  for (int w = tid; w < (c + 31) / 32; w += kSelThreads) sh.keep[w] = 0u;
  float x[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int k = tid + kSelThreads * i;
    x[i] = k < c ? sq[k] : -INFINITY;
  }
  const MassTotal mt = mass_total<KP>(x, c, temperature, sh.redf);
  // the selected probes by key (the same key as k_select takes)
  const int P2 = pow2_at_least(pmax);
  int kj = -1;
  unsigned long long skey = 0ull;  // padding sorts below every real key
  float sval = 0.f;
  if (tid < pmax) {
    kj = min(max(Sq[tid], 0), c - 1);
    sval = sq[kj];
    skey = probe_sort_key(probe_key(sval, sample, temperature, seed, (uint32_t)q, kj), kj);
  }
  unsigned long long top = 0ull;
  int n = adaptive_fast(tid < pmax ? __expf(sval / temperature - mt.M) : 0.f, skey, sval, pmax,
                        pmin, tau, mt, temperature, sh.redf, sh.key, &top);
  if (n == pmax) {  // every probe
    if (tid < pmax) atomicOr(&sh.keep[kj >> 5], 1u << (kj & 31));
  } else if (n == 1) {  // the top probe alone
    if (tid == 0) {
      const int id = (int)(0xFFFFFFFFu - (uint32_t)(top & 0xFFFFFFFFull));
      sh.keep[id >> 5] = 1u << (id & 31);
    }
  } else {
    bitonic_sort_desc(skey, sval, P2, sh.key, sh.val);
    int id;
    n = adaptive_count(skey, sval, pmax, pmin, tau, mt, temperature, sh.redf, sh.red_cnt, &id);
    if (tid < n) atomicOr(&sh.keep[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  const int kept = tid < pmax && (sh.keep[kj >> 5] & (1u << (kj & 31))) ? 1 : 0;
  int tot;
  const int pos = block_exclusive_scan(kept, sh.red_scan, &tot);
  if (kept) Sq[pos] = kj;
  if (tid < pmax && tid >= n) Sq[tid] = -1;
  if (tid == 0) nprobe[q] = n;
  if (mbits) {
    // the kept probes as bitset words and earlier-word counts, word-major
    // [W x B], for the cluster-major stage 2
    const int W = (c + 31) / 32;
    const uint32_t word = tid < W ? sh.keep[tid] : 0u;
    int wt;
    const int before = block_exclusive_scan(__popc(word), sh.red_cnt, &wt);
    if (tid < W) {
      mbits[(int64_t)tid * gridDim.x + q] = word;
      mpre[(int64_t)tid * gridDim.x + q] = before;
    }
  }
  const int64_t nr = (int64_t)pmax * b;
  for (int64_t r = (int64_t)n * b + tid; r < nr; r += kSelThreads) {
    if (out_ids) out_ids[(int64_t)q * nr + r] = -1;
    if (out_logits) out_logits[(int64_t)q * nr + r] = -INFINITY;
  }
}

__global__ __launch_bounds__(256) void k_finish(const Part* __restrict__ parts, int nparts,
                                                const int32_t* __restrict__ nlimit, int scale,
                                                int32_t* __restrict__ out_token,
                                                float* __restrict__ out_logit,
                                                float* __restrict__ out_lse) {
  __shared__ Part sh[256];
  const int q = blockIdx.x;
  const int n = nlimit ? max(0, min(nparts, nlimit[q] * scale)) : nparts;
  const Part r = merge_parts_block<256>(parts + (int64_t)q * nparts, n, sh);
  if (threadIdx.x == 0) write_outputs(r, q, out_token, out_logit, out_lse);
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
static hipError_t score_dispatch(const KernelCtx& k, const void* h, int B, float* out,
                                const KeyXform& kx) {
  RowsArgs a{};
  a.M = k.C; a.nrows = k.c; a.d = k.d; a.H = h; a.B = B; a.out_vals = out; a.ld_vals = k.c;
  a.tprime = 1.f; a.key = kx;
  if (B == 1) return launch_rows<T, 1, kScoreRPW, false, false>(a, k.stream, nullptr);
  if (B == 2) return launch_rows<T, 2, kScoreRPW, false, false>(a, k.stream, nullptr);
  return launch_rows<T, 4, kScoreRPW, false, false>(a, k.stream, nullptr);
}

hipError_t launch_score(const KernelCtx& k, const void* h, int B, float* out,
                        const KeyXform& kx) {
  return k.bf16 ? score_dispatch<uint16_t>(k, h, B, out, kx)
                : score_dispatch<float>(k, h, B, out, kx);
}

template <typename T, int BITS, int NQ>
static hipError_t quant_score_launch(const KernelCtx& k, const void* h, int B, float* out,
                                     const KeyXform& kx) {
  const int G = k.d / 32;
  const int maxg = (G + 63) / 64;
  const int64_t gx = (k.c + 4 * kInt4RPW - 1) / (4 * kInt4RPW);
  const dim3 grid((unsigned)gx, (unsigned)((B + NQ - 1) / NQ));
  const T* hp = static_cast<const T*>(h);
  switch (maxg) {
#define FH_CASE(MG) \
  case MG: hipLaunchKernelGGL((k_score_q<T, BITS, MG, NQ, kInt4RPW>), grid, dim3(256), 0, k.stream, k.cq, k.csig, k.c, k.d, hp, B, out, kx); break;
    FH_CASE(1) FH_CASE(2) FH_CASE(3) FH_CASE(4)
#undef FH_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t quant_score(const KernelCtx& k, const void* h, int B, float* out,
                              const KeyXform& kx) {
  if (k.bf16)
    return B == 1 ? quant_score_launch<uint16_t, BITS, 1>(k, h, B, out, kx)
                  : quant_score_launch<uint16_t, BITS, 2>(k, h, B, out, kx);
  return B == 1 ? quant_score_launch<float, BITS, 1>(k, h, B, out, kx)
                : quant_score_launch<float, BITS, 2>(k, h, B, out, kx);
}

hipError_t launch_score_quant(const KernelCtx& k, const void* h, int B, float* out,
                              const KeyXform& kx) {
  if (k.qbits == 4) return quant_score<4>(k, h, B, out, kx);
  if (k.qbits == 8) return quant_score<8>(k, h, B, out, kx);
  return hipErrorInvalidValue;
}

template <int BITS>
static hipError_t quant_launch(const KernelCtx& k, int* bad) {
  const int64_t n = k.c * (k.d / 32);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (k.bf16)
    hipLaunchKernelGGL((k_quant_g32<uint16_t, BITS>), grid, dim3(256), 0, k.stream,
                       static_cast<const uint16_t*>(k.C), k.c, k.d, const_cast<uint8_t*>(k.cq),
                       const_cast<uint16_t*>(k.csig), bad);
  else
    hipLaunchKernelGGL((k_quant_g32<float, BITS>), grid, dim3(256), 0, k.stream,
                       static_cast<const float*>(k.C), k.c, k.d, const_cast<uint8_t*>(k.cq),
                       const_cast<uint16_t*>(k.csig), bad);
  return hipGetLastError();
}

hipError_t launch_quant(const KernelCtx& k, int* bad) {
  if (k.qbits == 4) return quant_launch<4>(k, bad);
  if (k.qbits == 8) return quant_launch<8>(k, bad);
  return hipErrorInvalidValue;
}

// Standard-normal upper quantile z with P(Z > z) = select_target(p) / c: the
// rational approximation of Abramowitz & Stegun 26.2.23 refined by two
// Newton steps on 0.5 erfc(z / sqrt 2) = q.  It only places the fast-path
// threshold of the selection, so it affects speed, not results.
float select_quantile(int64_t c, int64_t p) {
  if (!select_fast_ok((int)c, (int)p)) return 0.f;
  const double q = (double)select_target((int)p) / (double)c;
  const double t = std::sqrt(-2.0 * std::log(q));
  double z = t - (2.515517 + t * (0.802853 + t * 0.010328)) /
                     (1.0 + t * (1.432788 + t * (0.189269 + t * 0.001308)));
  for (int it = 0; it < 2; ++it) {
    const double tail = 0.5 * std::erfc(z / std::sqrt(2.0));
    const double dens = std::exp(-0.5 * z * z) / std::sqrt(2.0 * 3.14159265358979323846);
    z += (tail - q) / dens;
  }
  return (float)z;
}

hipError_t launch_permute_rows(const KernelCtx& k, void* out) {
  const int nch = k.d * (k.bf16 ? 2 : 4) / 16;
  const unsigned blocks = (unsigned)((k.v + 3) / 4);
  hipLaunchKernelGGL(k_permute_rows, dim3(blocks), dim3(256), 0, k.stream,
                     static_cast<const uint4*>(k.E), k.c2t, static_cast<uint4*>(out), k.v, nch);
  return hipGetLastError();
}

hipError_t launch_select(const KernelCtx& k, const float* scores, int B, int p, int sample,
                         float temperature, uint64_t seed, int32_t* S, int ldS, uint32_t* mbits,
                         int32_t* mpre) {
  const dim3 grid((unsigned)B), block(kSelThreads);
  const int c = (int)k.c;
  const float zq = select_quantile(k.c, p);
  switch (sel_keys_per_thread(k.c)) {
#define FH_CASE(KK) \
  case KK: hipLaunchKernelGGL((k_select<KK>), grid, block, 0, k.stream, scores, c, p, sample, temperature, seed, zq, S, ldS, mbits, mpre); break;
    FH_CASE(1) FH_CASE(2) FH_CASE(8) FH_CASE(16)
#undef FH_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_adapt(const KernelCtx& k, const float* scores, int B, int pmax, int pmin,
                        float tau, int sample, float temperature, uint64_t seed, int32_t* S,
                        int32_t* nprobe, int32_t* out_ids, float* out_logits, uint32_t* mbits,
                        int32_t* mpre) {
  if (pmax < 1 || pmax > kSelThreads || pmin < 1 || pmin > pmax) return hipErrorInvalidValue;
  const dim3 grid((unsigned)B), block(kSelThreads);
  const int c = (int)k.c, b = (int)k.b;
  switch (sel_keys_per_thread(k.c)) {
#define FH_CASE(KK) \
  case KK: hipLaunchKernelGGL((k_adapt<KK>), grid, block, 0, k.stream, scores, c, pmax, pmin, tau, sample, temperature, seed, S, nprobe, b, out_ids, out_logits, mbits, mpre); break;
    FH_CASE(1) FH_CASE(2) FH_CASE(8) FH_CASE(16)
#undef FH_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t gather_t(const KernelCtx& k, const void* h, int B, const int32_t* S, int p,
                           int token_sample, float tprime, uint64_t seed, int32_t* out_ids,
                           float* out_logits, Part* parts, int64_t* nparts, int ldS,
                           const int32_t* nprobe) {
  RowsArgs a{};
  a.M = k.Ec ? k.Ec : k.E; a.contiguous = k.Ec != nullptr;
  a.nrows = (int64_t)p * k.b; a.d = k.d; a.c2t = k.c2t; a.bsz = (int)k.b;
  a.S = S; a.ldS = ldS < 0 ? p : ldS; a.H = h; a.B = B; a.out_vals = out_logits; a.ld_vals = a.nrows;
  a.out_ids = out_ids; a.token_sample = token_sample; a.tprime = tprime; a.seed = seed;
  a.parts = parts; a.nprobe = nprobe;
  return launch_rows<T, 1, kGatherRPW, true, true>(a, k.stream, nparts);
}

hipError_t launch_gather(const KernelCtx& k, const void* h, int B, const int32_t* S, int p,
                         int token_sample, float tprime, uint64_t seed, int32_t* out_ids,
                         float* out_logits, Part* parts, int64_t* nparts, int ldS,
                         const int32_t* nprobe) {
  return k.bf16 ? gather_t<uint16_t>(k, h, B, S, p, token_sample, tprime, seed, out_ids, out_logits, parts, nparts, ldS, nprobe)
                : gather_t<float>(k, h, B, S, p, token_sample, tprime, seed, out_ids, out_logits, parts, nparts, ldS, nprobe);
}

// ---- batch-shared probes (explainer §4.2: share the cluster selection
// across the batch; read as the top p of the summed scores)

// out[k] = sum_b s[b, k], b ascending.
__global__ __launch_bounds__(256) void k_sum_rows(const float* __restrict__ s, int B, int c,
                                                  float* __restrict__ out) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= c) return;
  float acc = 0.f;
#pragma unroll 16
  for (int b = 0; b < B; ++b) acc += s[(int64_t)b * c + k];
  out[k] = acc;
}

// dst[q * n + i] = src[i]: one probe list as every row of [B x n].
__global__ __launch_bounds__(256) void k_broadcast_row(const int32_t* __restrict__ src, int n,
                                                       int B, int32_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (int64_t)n * B) dst[i] = src[i % n];
}

hipError_t launch_sum_rows(const KernelCtx& k, const float* scores, int B, float* out) {
  hipLaunchKernelGGL(k_sum_rows, dim3((unsigned)((k.c + 255) / 256)), dim3(256), 0, k.stream,
                     scores, B, (int)k.c, out);
  return hipGetLastError();
}

hipError_t launch_broadcast_row(const KernelCtx& k, const int32_t* src, int n, int B,
                                int32_t* dst) {
  const int64_t m = (int64_t)n * B;
  hipLaunchKernelGGL(k_broadcast_row, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, k.stream,
                     src, n, B, dst);
  return hipGetLastError();
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
                         int32_t* out_token, float* out_logit, float* out_lse,
                         const int32_t* nlimit, int scale) {
  hipLaunchKernelGGL(k_finish, dim3((unsigned)B), dim3(256), 0, k.stream, parts, (int)nparts,
                     nlimit, scale, out_token, out_logit, out_lse);
  return hipGetLastError();
}

// ---- batch-1 path: one launch (sizing in fh_batch1_sizing.hpp)

hipError_t launch_batched(const BatchedLaunch& f) {
  return f.ctx->bf16 ? launch_batched_bf16(f) : launch_batched_f32(f);
}

hipError_t launch_batch1(const FusedLaunch& f) {
  switch (f.ctx->qbits) {
    case 0: return f.ctx->bf16 ? launch_batch1_bf16(f) : launch_batch1_f32(f);
    case 4: return f.ctx->bf16 ? launch_batch1_bf16_int4(f) : launch_batch1_f32_int4(f);
    case 8: return f.ctx->bf16 ? launch_batch1_bf16_int8(f) : launch_batch1_f32_int8(f);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fh
