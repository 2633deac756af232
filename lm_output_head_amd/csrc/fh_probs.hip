// fp8 probabilities of the retrieved candidates (FlashHead explainer,
// framerc.cn, §2.3: the quantisation config keeps the probability
// intermediate in fp8).  Per row q: p = exp(z / T' - lse[q]); a power-of-two
// scale 2^k, k = 8 - e for p_max = f 2^e with f in [1/2, 1), puts the row's
// largest probability in [128, 256) (exact scaling, no saturation, 17
// binades of range below it); out[q, i] = E4M3(p 2^k), the OCP E4M3 byte
// (bias 7, three mantissa bits, no infinities) rounded to nearest even, and
// out_k[q] = k.  One workgroup per row: a max pass, then the encoding pass
// (4 bytes read, 1 written per candidate; bound by launch latency at the
// sizes a call produces).

#include <hip/hip_runtime.h>

#include "fh_device.hpp"
#include "fh_internal.hpp"

namespace fh {
namespace {

// E4M3 byte of a scaled probability x (x >= 0; NaN gives 0x7F).  From 2^-6
// up the float's exponent and top three mantissa bits are rounded at bit 20
// (the carry runs into the exponent) and rebiased from 127 to 7; below 2^-6
// the code is the subnormal count x 2^9 rounded to nearest even, where a
// count of 8 is the smallest normal's code.  Values above 448 saturate.
__device__ __forceinline__ uint32_t e4m3_byte(float x) {
  if (x != x) return 0x7Fu;
  if (!(x > 0.f)) return 0u;
  x = fminf(x, 448.f);
  if (x < 0.015625f) return (uint32_t)__float2int_rn(x * 512.f);
  const uint32_t b = __float_as_uint(x);
  const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
  return r - (120u << 3);
}

constexpr int kProbThreads = 1024;

__global__ __launch_bounds__(kProbThreads) void k_probs_fp8(const float* __restrict__ z,
                                                            const float* __restrict__ lse,
                                                            int64_t n, float temperature,
                                                            uint8_t* __restrict__ out,
                                                            int32_t* __restrict__ out_k) {
  __shared__ float red[kProbThreads / 64];
  const int64_t q = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float l = lse[q];
  const float* zq = z + q * n;
  uint8_t* oq = out + q * n;
  float pm = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += kProbThreads)
    pm = fmaxf(pm, expf(zq[i] / temperature - l));
  pm = wave_max(pm);
  if (lane == 0) red[wave] = pm;
  __syncthreads();
  pm = readlane_f(row_allreduce(lane < kProbThreads / 64 ? red[lane] : 0.f,
                                [](float a, float b) { return fmaxf(a, b); }), 0);
  int k = 0;
  if (pm > 0.f) {
    int e;
    (void)frexpf(pm, &e);
    k = 8 - e;
  }
  if (threadIdx.x == 0) out_k[q] = k;
  for (int64_t i = threadIdx.x; i < n; i += kProbThreads)
    oq[i] = (uint8_t)e4m3_byte(ldexpf(expf(zq[i] / temperature - l), k));
}

}  // namespace

hipError_t launch_probs_fp8(const float* logits, const float* lse, int64_t B, int64_t n,
                            float temperature, uint8_t* out, int32_t* out_k, hipStream_t stream) {
  if (B < 1 || n < 1 || B > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probs_fp8, dim3((unsigned)B), dim3(kProbThreads), 0, stream, logits, lse, n,
                     temperature, out, out_k);
  return hipGetLastError();
}

}  // namespace fh
