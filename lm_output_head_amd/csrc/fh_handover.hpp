// Hand-over between workgroups of one launch: 64-bit words tagged with the
// call's epoch (epoch << 32 | payload), written and polled with agent-scope
// relaxed atomics, and a bounded poll.  A workgroup only ever waits for
// words written by workgroups dispatched before it (in-order dispatch), so
// the grid need not be co-resident; a poll that gives up sets a sticky flag
// and lets the grid drain.  Used by the single-launch batch-1 kernel and the
// batched launch after stage 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fh_device.hpp"
#include "fh_internal.hpp"

namespace fh {

constexpr unsigned kSpinLimit = 1u << 20;
// s_sleep argument between polling rounds (units of 64 clocks)
#ifndef FH_POLL_SLEEP
#define FH_POLL_SLEEP 1
#endif

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
__device__ __forceinline__ bool poll_tagged(unsigned long long* const (&p)[N],
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
#pragma unroll
      for (int i = 0; i < N; ++i) out[i] = (uint32_t)v[i];
      return false;
    }
    __builtin_amdgcn_s_sleep(FH_POLL_SLEEP);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((unsigned)(v[i] >> 32) != epoch)
        v[i] = __hip_atomic_load(p[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = (uint32_t)v[i];
  return true;
}

// A stage-2 partial whose workgroup gave up a poll carries this id (never a
// token id, nor part_empty's), so that the finisher can mark the outputs.
constexpr int32_t kBadPart = -1;

// One wave polls the n tagged partials at base (five words each: key, z, m,
// s, id) and merges them: lane l takes partials l, l + 64, ..., three at a
// time with their 15 words in flight together, merging in index order; the
// lanes then merge as a fixed DPP tree.  *bad (uniform) is set if a poll
// gave up or a partial is marked kBadPart.  The result is uniform.
__device__ __forceinline__ Part wave_merge_tagged_parts(unsigned long long* base, int n,
                                                        unsigned epoch, unsigned* err,
                                                        bool* bad_out) {
  const int lane = threadIdx.x & 63;
  Part acc = part_empty();
  bool bad = false;
  constexpr int kU = 3;
  for (int i0 = 0; i0 < n; i0 += 64 * kU) {
    unsigned long long* pb[kU];
    bool lv[kU];
    unsigned long long v[5 * kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + lane + 64 * u;
      lv[u] = i < n;
      pb[u] = base + 5 * (int64_t)(lv[u] ? i : 0);
#pragma unroll
      for (int f = 0; f < 5; ++f)
        v[5 * u + f] = lv[u] ? __hip_atomic_load(pb[u] + f, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : tag(epoch, 0u);
    }
    for (unsigned k = 0;; ++k) {
      bool done = true;
#pragma unroll
      for (int e = 0; e < 5 * kU; ++e) done = done && (unsigned)(v[e] >> 32) == epoch;
      if (done) break;
      if (k >= kSpinLimit) {
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bad = true;
        break;
      }
      __builtin_amdgcn_s_sleep(FH_POLL_SLEEP);
#pragma unroll
      for (int e = 0; e < 5 * kU; ++e)
        if ((unsigned)(v[e] >> 32) != epoch)
          v[e] = __hip_atomic_load(pb[e / 5] + e % 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (!lv[u]) continue;
      if ((int32_t)(uint32_t)v[5 * u + 4] == kBadPart) bad = true;
      acc = part_merge(acc, Part{__uint_as_float((uint32_t)v[5 * u]),
                                 __uint_as_float((uint32_t)v[5 * u + 1]),
                                 __uint_as_float((uint32_t)v[5 * u + 2]),
                                 __uint_as_float((uint32_t)v[5 * u + 3]),
                                 (int32_t)(uint32_t)v[5 * u + 4]});
    }
  }
  *bad_out = __ballot(bad) != 0ull;
  return wave_merge_part(acc);  // fixed DPP pattern, then lanes 0, 16, 32, 48
}

// Publish a workgroup's partial as five tagged words at p (one thread).
__device__ __forceinline__ void publish_part(unsigned long long* p, unsigned epoch, const Part& w) {
  st_tagged(p + 0, tag(epoch, __float_as_uint(w.key)));
  st_tagged(p + 1, tag(epoch, __float_as_uint(w.z)));
  st_tagged(p + 2, tag(epoch, __float_as_uint(w.m)));
  st_tagged(p + 3, tag(epoch, __float_as_uint(w.s)));
  st_tagged(p + 4, tag(epoch, (uint32_t)w.id));
}

}  // namespace fh
