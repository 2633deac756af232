// Speculative sampling with a FlashHead draft verified by the dense head
// (FlashHead explainer, framerc.cn, §4.2 "speculative decoding integration":
// a FlashHead draft at temperature T, the original head's probabilities,
// accept or reject), read as the standard speculative-sampling rule
// (Leviathan, Kalman, Matias, ICML 2023; Chen et al. 2023) for one position
// per query:
//   p(t) = softmax(E h / T) over all v tokens (the dense head);
//   q(t) = softmax(E_t h / T) over the retrieved tokens of the draft's probes;
//   accept the draft token x when u < min(1, p(x) / q(x)), u a Philox uniform
//   (stage 2); else draw from max(0, p - q) (Gumbel-max, stage 3).
// Both heads score a retrieved token with the same E_t . h, so for x inside
// the probes p(x) / q(x) = exp(LSE_S - LSE_full), the draft's LSE over its
// retrieved tokens against the full one, and max(0, p - q) is p on the
// tokens outside the probes and 0 inside.  One pass over E therefore gives
// everything: the full LSE, and the Gumbel-max over the tokens whose
// cluster is not among the draft's probes.

#include "fh_blocks.hpp"
#include "fh_internal.hpp"

namespace fh {

constexpr uint32_t kStageAccept = 2u;
constexpr uint32_t kStageResidual = 3u;

// t2c[C2T[f]] = f / b: the cluster of every token.
__global__ __launch_bounds__(256) void k_t2c(const int32_t* __restrict__ c2t, int64_t v, int b,
                                             int32_t* __restrict__ t2c) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f < v) t2c[c2t[f]] = (int32_t)(f / b);
}

// bits[q W + w]: bit k % 32 of word k / 32 set for every probe k of query q
// (ids outside [0, c) are ignored).  One workgroup per query.
__global__ __launch_bounds__(256) void k_probe_bits(const int32_t* __restrict__ S, int p, int c,
                                                    int W, uint32_t* __restrict__ bits) {
  __shared__ uint32_t lb[512];
  const int q = blockIdx.x;
  for (int w = threadIdx.x; w < W; w += 256) lb[w] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < p; i += 256) {
    const int k = S[(int64_t)q * p + i];
    if (k >= 0 && k < c) atomicOr(&lb[k >> 5], 1u << (k & 31));
  }
  __syncthreads();
  for (int w = threadIdx.x; w < W; w += 256) bits[(int64_t)q * W + w] = lb[w];
}

struct SpecArgs {
  const void* E;  // [v x d] token order
  const int32_t* t2c;
  const uint32_t* bits;  // [B x W]
  int W;
  int64_t v;
  int d;
  const void* H;  // [B x d]
  int B;
  float T;
  uint64_t seed;
  Part* parts;  // [B x gridDim.x]
};

// The dense pass of the verification: every token's logit z enters the
// LSE of z / T; the tokens outside the query's probes compete with keys
// z / T + G(seed, q, t, stage 3), the ones inside with -inf.  Rows as in the
// dense head: RPW consecutive rows per wave, NQ queries per workgroup row.
template <typename T, int MAXM, int NQ, int RPW>
__global__ __launch_bounds__(256) void k_spec_rows(SpecArgs a) {
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
  const int64_t r1 = min(r0 + RPW, a.v);
  auto same = [](int64_t r) { return r; };
  auto sink = [&](int q, int64_t t, int64_t, float z) {
    const int oq = q0 + q;
    const int k = a.t2c[t];
    const bool probed = (a.bits[(int64_t)oq * a.W + (k >> 5)] >> (k & 31)) & 1u;
    const float key =
        probed ? -INFINITY : z / a.T + gumbel_at(a.seed, (uint32_t)oq, (uint32_t)t, kStageResidual);
    part[q] = part_merge(part[q], Part{key, z, z / a.T, 1.f, (int32_t)t});
  };
  wave_rows<T, MAXM, NQ>(static_cast<const T*>(a.E), a.d, lane, hv, nq, r0, r1, 1, same, same,
                         sink);
  const Part wg = block_merge_parts<4, NQ>(part, nq, sh);
  if ((int)threadIdx.x < nq) a.parts[(int64_t)(q0 + threadIdx.x) * gridDim.x + blockIdx.x] = wg;
}

// Per query: merge the partials (full LSE, residual draw), then accept the
// draft token x when u < min(1, exp(LSE_S - LSE_full)) with x inside the
// probes (a draft outside its own probes has q(x) = 0: ratio 1), or when the
// residual is empty; otherwise output the residual draw.
__global__ __launch_bounds__(256) void k_spec_finish(const Part* __restrict__ parts, int nparts,
                                                     const int32_t* __restrict__ draft_token,
                                                     const float* __restrict__ draft_lse,
                                                     const int32_t* __restrict__ t2c,
                                                     const uint32_t* __restrict__ bits, int W,
                                                     int64_t v, uint64_t seed,
                                                     int32_t* __restrict__ out_token,
                                                     int32_t* __restrict__ out_accepted,
                                                     float* __restrict__ out_lse) {
  __shared__ Part sh[256];
  const int q = blockIdx.x;
  const Part r = merge_parts_block<256>(parts + (int64_t)q * nparts, nparts, sh);
  if (threadIdx.x != 0) return;
  const float lse = r.m + logf(r.s);
  const int32_t x = draft_token[q];
  const bool valid = x >= 0 && x < v;
  bool inside = false;
  if (valid) {
    const int k = t2c[x];
    inside = (bits[(int64_t)q * W + (k >> 5)] >> (k & 31)) & 1u;
  }
  const float ratio = inside ? fminf(1.f, expf(draft_lse[q] - lse)) : 1.f;
  const U4 blk = philox_block(seed, (uint32_t)q, 0u, kStageAccept);
  const float u = ((float)(blk.x >> 9) + 0.5f) * 1.1920928955078125e-07f;
  const bool empty = r.key == -INFINITY;
  const bool accept = valid && (u < ratio || empty);
  out_token[q] = accept ? x : r.id;
  if (out_accepted) out_accepted[q] = accept ? 1 : 0;
  if (out_lse) out_lse[q] = lse;
}

// ----------------------------------------------------------------- host ---

hipError_t launch_t2c(const KernelCtx& k, int32_t* t2c) {
  hipLaunchKernelGGL(k_t2c, dim3((unsigned)((k.v + 255) / 256)), dim3(256), 0, k.stream, k.c2t,
                     k.v, (int)k.b, t2c);
  return hipGetLastError();
}

template <typename T, int NQ>
static hipError_t spec_rows(const SpecArgs& a, hipStream_t st, int64_t* nblocks) {
  const int nch = a.d / Chunk<T>::kElems;
  const int maxm = (nch + 63) / 64;
  const int64_t gx = rows_blocks(a.v, kDenseRPW);
  const dim3 grid((unsigned)gx, (unsigned)((a.B + NQ - 1) / NQ));
  *nblocks = gx;
  switch (maxm) {
#define FH_CASE(MM) \
  case MM: hipLaunchKernelGGL((k_spec_rows<T, MM, NQ, kDenseRPW>), grid, dim3(256), 0, st, a); break;
    FH_CASE(1) FH_CASE(2) FH_CASE(3) FH_CASE(4) FH_CASE(5) FH_CASE(6) FH_CASE(7) FH_CASE(8)
#undef FH_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t spec_rows_t(const SpecArgs& a, hipStream_t st, int64_t* nblocks) {
  if (a.B == 1) return spec_rows<T, 1>(a, st, nblocks);
  if (a.B == 2) return spec_rows<T, 2>(a, st, nblocks);
  return spec_rows<T, 4>(a, st, nblocks);
}

hipError_t launch_spec_verify(const KernelCtx& k, int cus, const int32_t* t2c, uint32_t* bits, Part* parts,
                              const void* h, int B, int p, const int32_t* draft_clusters,
                              const int32_t* draft_token, const float* draft_lse, float T,
                              uint64_t seed, int32_t* out_token, int32_t* out_accepted,
                              float* out_lse) {
  const int W = (int)((k.c + 31) / 32);
  hipLaunchKernelGGL(k_probe_bits, dim3((unsigned)B), dim3(256), 0, k.stream, draft_clusters, p,
                     (int)k.c, W, bits);
  hipError_t r = hipGetLastError();
  if (r != hipSuccess) return r;
  SpecArgs a{};
  a.E = k.E; a.t2c = t2c; a.bits = bits; a.W = W; a.v = k.v; a.d = k.d; a.H = h; a.B = B;
  a.T = T; a.seed = seed; a.parts = parts;
  int64_t nparts = 0;
  if (k.bf16 && B >= kMfmaMinBatchDense)  // the dense head's matrix-core GEMM, verification epilogue
    r = launch_spec_mfma(k, cus, h, B, T, seed, t2c, bits, W, parts, &nparts);
  else
    r = k.bf16 ? spec_rows_t<uint16_t>(a, k.stream, &nparts) : spec_rows_t<float>(a, k.stream, &nparts);
  if (r != hipSuccess) return r;
  hipLaunchKernelGGL(k_spec_finish, dim3((unsigned)B), dim3(256), 0, k.stream, parts, (int)nparts,
                     draft_token, draft_lse, t2c, bits, W, k.v, seed, out_token, out_accepted,
                     out_lse);
  return hipGetLastError();
}

}  // namespace fh
