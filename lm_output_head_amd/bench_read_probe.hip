// A plain one-shot read of a device buffer, for bench.py only (--burst and
// the stream rate beside the roofline): it
// measures the memory system the head runs on and computes nothing of the
// head (whose cost the pages place in reading the embedding table from
// memory: FlashHead technical explainer, framerc.cn, §1.1).  Built into its
// own library (libflashhead_bench.so), not the product's C ABI.
//
// One 16-byte load per thread in 1024-thread workgroups; a thread that finds
// a 32-bit word equal to `key` stores 1 to *found, so the call is a search
// and every load is used, with almost no work after the loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(1024) void k_read_probe(const uint4* __restrict__ p, int64_t n16,
                                                     uint32_t key, uint32_t* __restrict__ found) {
  const int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  if (i >= n16) return;
  const uint4 v = p[i];
  // no short-circuit: with || the compiler loads one word first and the rest
  // only after comparing it, two dependent memory round trips
  const uint32_t hit = (uint32_t)(v.x == key) | (uint32_t)(v.y == key) | (uint32_t)(v.z == key) |
                       (uint32_t)(v.w == key);
  if (hit) *found = 1u;
}

}  // namespace

extern "C" {

// buf: device, 16-byte aligned, `bytes` bytes (a positive multiple of 16, at
// most 2^40); found: device uint32 [1], set to 1 if some word equals key
// (the caller clears it); stream: HIP stream (NULL = default).  Returns 0,
// -1 on a NULL pointer, a misaligned buffer or a bad size (nothing launched),
// -3 if the launch failed.  Asynchronous; allocates nothing.
int fhb_read_probe(const void* buf, int64_t bytes, uint32_t key, uint32_t* found, void* stream) {
  if (!buf || !found) return -1;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return -1;
  if (bytes < 16 || bytes % 16 != 0 || bytes > ((int64_t)1 << 40)) return -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)((n16 + 1023) / 1024)), dim3(1024), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), n16, key,
                     found);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
