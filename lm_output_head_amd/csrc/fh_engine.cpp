// libflashhead C ABI: argument checking, ownership and launch sequencing.
//
// The path per call follows the FlashHead computation graph (explainer,
// framerc.cn, §2.2.2): centroid scores -> top-p (or sampled) clusters ->
// retrieved-token scores -> argmax / sample.  Every step runs in the HIP
// kernels (fh_kernels.hip, fh_batch1_*.hip, fh_mfma.hip, fh_spec.hip,
// fh_cluster.hip); this file only checks arguments, owns device buffers and
// enqueues work on the caller's stream.

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <new>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "fh_internal.hpp"
#include "flashhead.h"

namespace {

thread_local std::string g_err;

fh_status fail(fh_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

fh_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return e == hipErrorOutOfMemory ? FH_ENOMEM : FH_EHIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxC = 16384;

}  // namespace

struct fh_engine {
  int device = 0;
  fh_dtype dtype = FH_BF16;
  fh_quant quant = FH_QUANT_NONE;
  int64_t v = 0, d = 0, c = 0, b = 0, max_batch = 0;
  const void* E = nullptr;
  const void* C = nullptr;
  int32_t* c2t = nullptr;
  int32_t* t2c = nullptr;     // cluster of every token (speculative verification)
  void* Ec = nullptr;         // cluster-contiguous copy of E: Ec[f] = E[C2T[f]]
  void* Ecm = nullptr;        // Ec in fragment order (bf16 engines taking batches)
  void* Cm = nullptr;         // C in fragment order (the same engines)
  uint8_t* cq = nullptr;
  uint16_t* csig = nullptr;
  uint8_t* cq_mfma = nullptr;    // INT4 codes in the MFMA tile layout (bf16 engines)
  uint16_t* sig_mfma = nullptr;  // INT4 scales, group-major
  float* scores = nullptr;   // [max_batch x c]
  int32_t* sel = nullptr;    // [max_batch x c]
  uint32_t* mbits = nullptr;  // [ceil(c/32) x max_batch] probe bitsets, word-major
  int32_t* mpre = nullptr;    // [ceil(c/32) x max_batch] probes in earlier words
  float* sumscores = nullptr;  // [c] summed scores of a batch (shared probes)
  int32_t* nprobe = nullptr;   // [max_batch] adaptive probe counts
  fh::Part* parts = nullptr;  // partials: [B x parts per query] of the call's stage 2
  int64_t parts_total = 0;
  unsigned* sync = nullptr;   // [0]: sticky flag, a batch-1 poll gave up
  unsigned long long* tagged = nullptr;  // batch-1 hand-over words (fh_batch1_sizing.hpp layout)
  unsigned long long* btag = nullptr;    // batched launch's hand-over words (same header)
  unsigned epoch = 0;
  int cus = 0;                // compute units of the device
  int path = FH_PATH_AUTO;
  // per-kernel timing
  bool prof = false;
  int64_t prof_cap = 0, prof_n = 0;
  std::vector<hipEvent_t> prof_ev;
  std::vector<const char*> prof_name;

  fh::KernelCtx ctx(hipStream_t st) const {
    fh::KernelCtx k;
    k.bf16 = dtype == FH_BF16;
    k.E = E;
    k.Ec = Ec;
    k.Ecm = Ecm;
    k.Cm = Cm;
    k.C = C;
    k.c2t = c2t;
    k.cq = cq;
    k.csig = csig;
    k.cq_mfma = cq_mfma;
    k.sig_mfma = sig_mfma;
    k.v = v;
    k.c = c;
    k.b = b;
    k.d = (int)d;
    k.stream = st;
    k.qbits = quant == FH_QUANT_INT4_G32 ? 4 : quant == FH_QUANT_INT8_G32 ? 8 : 0;
    return k;
  }
};

namespace {

// Run one launcher, bracketed by profiling events when profiling is on.
template <typename F>
hipError_t timed(fh_engine* e, hipStream_t st, const char* name, F&& launch) {
  const bool rec = e->prof && e->prof_n < e->prof_cap;
  if (rec) {
    hipError_t r = hipEventRecord(e->prof_ev[2 * e->prof_n], st);
    if (r != hipSuccess) return r;
  }
  hipError_t r = launch();
  if (r != hipSuccess) return r;
  if (rec) {
    r = hipEventRecord(e->prof_ev[2 * e->prof_n + 1], st);
    if (r != hipSuccess) return r;
    e->prof_name[e->prof_n] = name;
    e->prof_n++;
  }
  return hipSuccess;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

void free_engine(fh_engine* e) {
  if (!e) return;
  (void)hipFree(e->c2t);
  (void)hipFree(e->Ec);
  (void)hipFree(e->Ecm);
  (void)hipFree(e->Cm);
  (void)hipFree(e->t2c);
  (void)hipFree(e->sumscores);
  (void)hipFree(e->nprobe);
  (void)hipFree(e->cq);
  (void)hipFree(e->csig);
  (void)hipFree(e->cq_mfma);
  (void)hipFree(e->sig_mfma);
  (void)hipFree(e->scores);
  (void)hipFree(e->sel);
  (void)hipFree(e->mbits);
  (void)hipFree(e->mpre);
  (void)hipFree(e->parts);
  (void)hipFree(e->sync);
  (void)hipFree(e->tagged);
  (void)hipFree(e->btag);
  for (hipEvent_t ev : e->prof_ev) (void)hipEventDestroy(ev);
  delete e;
}

// Stage-1 scores for B queries (or, with kx.sample, the sampled-probe
// selection keys): matrix cores for batches of bf16 queries, the row GEMV
// otherwise.
hipError_t launch_stage1(fh_engine* e, hipStream_t st, const fh::KernelCtx& k, const void* h,
                         int64_t B, float* out, const fh::KeyXform& kx = fh::KeyXform{}) {
  const bool int4 = e->quant == FH_QUANT_INT4_G32;
  const bool int8 = e->quant == FH_QUANT_INT8_G32;
  const bool bf16 = e->dtype == FH_BF16;
  if (bf16 && int4 && B >= fh::kMfmaMinBatchInt4)
    return timed(e, st, "score_int4_mfma",
                 [&] { return fh::launch_score_mfma(k, e->cus, h, (int)B, out, kx); });
  if (bf16 && int8 && B >= fh::kMfmaMinBatchInt8)
    return timed(e, st, "score_int8_mfma",
                 [&] { return fh::launch_score_mfma(k, e->cus, h, (int)B, out, kx); });
  if (bf16 && e->quant == FH_QUANT_NONE && B >= fh::kMfmaMinBatchBf16)
    return timed(e, st, "score_mfma", [&] { return fh::launch_score_mfma(k, e->cus, h, (int)B, out, kx); });
  if (int4 || int8)
    return timed(e, st, int4 ? "score_int4" : "score_int8",
                 [&] { return fh::launch_score_quant(k, h, (int)B, out, kx); });
  return timed(e, st, "score", [&] { return fh::launch_score(k, h, (int)B, out, kx); });
}

fh_status check_common(const fh_engine* e, const void* h, int64_t B) {
  if (!e) return fail(FH_EINVAL, "engine is NULL");
  if (!h) return fail(FH_EINVAL, "h is NULL");
  if (!aligned16(h)) return fail(FH_EINVAL, "h must be 16-byte aligned");
  if (B < 1 || B > e->max_batch)
    return fail(FH_EINVAL, "B=" + std::to_string(B) + " outside [1, max_batch=" +
                               std::to_string(e->max_batch) + "]");
  return FH_OK;
}

fh_status check_mode(int mode, float temperature) {
  if (mode < 0 || mode > 7) return fail(FH_EINVAL, "mode must be FH_PROBE_* | FH_TOKEN_*");
  if ((mode & FH_PROBE_SHARED) && (mode & FH_PROBE_SAMPLE))
    return fail(FH_EINVAL, "FH_PROBE_SHARED chooses probes by score; it cannot be sampled");
  if (mode != 0 && !(temperature > 0.f && std::isfinite(temperature)))
    return fail(FH_EINVAL, "sampling needs a finite temperature > 0");
  return FH_OK;
}


// One probe set for the whole batch: the top p of the summed stage-1 scores
// (FH_PROBE_SHARED, B > 1), then stage 2 for every query over those probes:
// for bf16 one matrix-core GEMM [B x d] . [d x p b] over the probes' rows of
// the cluster-contiguous E, else the row GEMV reading one shared probe row.
fh_status shared_forward(fh_engine* e, hipStream_t st, const fh::KernelCtx& k, const void* h,
                         int64_t B, int64_t p, int token_sample, float tprime, uint64_t seed,
                         int32_t* out_token, float* out_token_logit, float* out_lse,
                         int32_t* out_clusters, int32_t* out_ids, float* out_logits) {
  hipError_t r = launch_stage1(e, st, k, h, B, e->scores);
  if (r != hipSuccess) return hip_fail(r, "score launch");
  r = timed(e, st, "sum_scores", [&] { return fh::launch_sum_rows(k, e->scores, (int)B, e->sumscores); });
  if (r != hipSuccess) return hip_fail(r, "summed scores");
  r = timed(e, st, "select", [&] {
    return fh::launch_select(k, e->sumscores, 1, (int)p, 0, 1.f, seed, e->sel, (int)p, nullptr,
                             nullptr);
  });
  if (r != hipSuccess) return hip_fail(r, "select launch");
  if (out_clusters) {
    r = fh::launch_broadcast_row(k, e->sel, (int)p, (int)B, out_clusters);
    if (r != hipSuccess) return hip_fail(r, "probe broadcast");
  }
  int64_t nparts = 0;
  if (e->dtype == FH_BF16) {
    r = timed(e, st, "gather_shared_mfma", [&] {
      return fh::launch_gather_shared_mfma(k, e->cus, h, (int)B, e->sel, (int)p, token_sample,
                                           tprime, seed, out_ids, out_logits, e->parts, &nparts);
    });
  } else {
    r = timed(e, st, "gather", [&] {
      return fh::launch_gather(k, h, (int)B, e->sel, (int)p, token_sample, tprime, seed, out_ids,
                               out_logits, e->parts, &nparts, 0);
    });
  }
  if (r != hipSuccess) return hip_fail(r, "gather launch");
  r = timed(e, st, "finish", [&] {
    return fh::launch_finish(k, e->parts, (int)B, nparts, out_token, out_token_logit, out_lse);
  });
  return r == hipSuccess ? FH_OK : hip_fail(r, "finish launch");
}

}  // namespace

// ---- workspace of fh_forward_noalloc: a file-scope device array (one copy
// per GPU, held until the process ends), for callers that cannot allocate.
// Host code never passes the array's name to a kernel: it takes the device
// address once per device (hipGetSymbolAddress, with that device current)
// and uses that address everywhere.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;  // 8 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};  // device -> address of its scratch

// The current device's scratch address (set up on first use on the device).
hipError_t scratch_for(int dev, void** out) {
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (r != hipSuccess) return r;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

extern "C" {

fh_status fh_balanced_assign(const float* sims, int64_t v, int64_t c, int32_t* out_assign,
                             int* out_rounds, void* stream) {
  g_err.clear();
  if (!sims || !out_assign) return fail(FH_EINVAL, "sims and out_assign must not be NULL");
  if (c < 1 || v < c || v % c != 0 || v > INT32_MAX)
    return fail(FH_EINVAL, "need 1 <= c, v a multiple of c and v < 2^31 (v=" + std::to_string(v) +
                               ", c=" + std::to_string(c) + ")");
  int rounds = 0;
  hipError_t r = fh::balanced_assign_device(sims, v, c, out_assign,
                                            static_cast<hipStream_t>(stream), &rounds);
  if (r != hipSuccess) return hip_fail(r, "balanced assignment");
  if (out_rounds) *out_rounds = rounds;
  return FH_OK;
}

fh_status fh_cluster(const void* E, fh_dtype dtype, int64_t v, int64_t d, int64_t c, int iters,
                     const double* u, float* out_C, int32_t* out_c2t, int32_t* out_init,
                     int32_t* out_assign, fh_cluster_times* out_times, void* stream) {
  g_err.clear();
  if (!E || !u || !out_C || !out_c2t) return fail(FH_EINVAL, "E, u, out_C and out_c2t must not be NULL");
  if (dtype != FH_F32 && dtype != FH_BF16) return fail(FH_EINVAL, "unknown dtype");
  if (c < 1 || c > 65536 || v < c || v % c != 0 || v > INT32_MAX)
    return fail(FH_EINVAL, "need 1 <= c <= 65536, v a multiple of c and v < 2^31 (v=" +
                               std::to_string(v) + ", c=" + std::to_string(c) + ")");
  const int64_t epc = dtype == FH_BF16 ? 8 : 4;  // elements per 16-byte chunk
  if (d < 1 || d % epc != 0)
    return fail(FH_EINVAL, dtype == FH_BF16 ? "bf16 needs d % 8 == 0" : "f32 needs d % 4 == 0");
  if (d > 64 * 8 * epc) return fail(FH_EUNSUPPORTED, "d too large for this library");
  if (iters < 1) return fail(FH_EINVAL, "iters must be >= 1");
  for (int64_t i = 0; i < c; ++i)
    if (!(u[i] >= 0.0 && u[i] < 1.0))
      return fail(FH_EINVAL, "u[" + std::to_string(i) + "] outside [0, 1)");
  fh::ClusterTimes t{};
  hipError_t r = fh::kmeans_device(E, dtype == FH_BF16, v, (int)d, c, iters, u, out_C, out_c2t,
                                   out_init, out_assign, static_cast<hipStream_t>(stream), &t);
  if (r != hipSuccess) return hip_fail(r, "clustering");
  if (out_times) {
    out_times->init_ms = t.init_ms;
    out_times->sims_ms = t.sims_ms;
    out_times->total_ms = t.total_ms;
    out_times->pp_step_us = t.pp_step_us;
    out_times->rounds = t.rounds;
  }
  return FH_OK;
}

const char* fh_last_error(void) { return g_err.c_str(); }

const char* fh_version(void) { return "flashhead-mi355x 0.1.0 (gfx950)"; }

fh_status fh_create(const void* E, const void* C, const int32_t* C2T, fh_dtype dtype, int64_t v,
                    int64_t d, int64_t c, fh_quant quant, int64_t max_batch, void* stream,
                    fh_engine** out) {
  g_err.clear();
  if (!out) return fail(FH_EINVAL, "out is NULL");
  if (!E || !C || !C2T) return fail(FH_EINVAL, "E, C and C2T must be non-NULL");
  if (dtype != FH_F32 && dtype != FH_BF16) return fail(FH_EINVAL, "unknown dtype");
  if (quant != FH_QUANT_NONE && quant != FH_QUANT_INT4_G32 && quant != FH_QUANT_INT8_G32)
    return fail(FH_EINVAL, "unknown quant");
  if (v <= 0 || d <= 0 || c <= 0) return fail(FH_EINVAL, "v, d and c must be positive");
  if (v % c != 0) return fail(FH_EINVAL, "v must be a multiple of c (balanced clusters)");
  if (v >= (int64_t(1) << 31)) return fail(FH_EUNSUPPORTED, "v must be below 2^31");
  if (c > kMaxC) return fail(FH_EUNSUPPORTED, "c above 16384 is not supported");
  const int epc = dtype == FH_BF16 ? 8 : 4;
  if (d % epc != 0)
    return fail(FH_EINVAL, dtype == FH_BF16 ? "bf16 needs d % 8 == 0" : "f32 needs d % 4 == 0");
  if (d > 64 * 8 * epc) return fail(FH_EUNSUPPORTED, "d too large for this library");
  if (quant != FH_QUANT_NONE && d % 32 != 0)
    return fail(FH_EUNSUPPORTED, "g32 quantisation needs d % 32 == 0");
  if (max_batch < 1 || max_batch > 65535) return fail(FH_EINVAL, "max_batch outside [1, 65535]");
  if (!aligned16(E) || !aligned16(C)) return fail(FH_EINVAL, "E and C must be 16-byte aligned");
  const int64_t b = v / c;
  {  // balanced clustering: C2T is a permutation of [0, v)
    std::vector<uint8_t> seen((size_t)v, 0);
    for (int64_t i = 0; i < v; ++i) {
      const int32_t t = C2T[i];
      if (t < 0 || t >= v) return fail(FH_EINVAL, "C2T holds a token id outside [0, v)");
      if (seen[(size_t)t]) return fail(FH_EINVAL, "C2T lists a token twice (not a permutation)");
      seen[(size_t)t] = 1;
    }
  }

  fh_engine* e = new (std::nothrow) fh_engine();
  if (!e) return fail(FH_ENOMEM, "host allocation failed");
  e->dtype = dtype;
  e->quant = quant;
  e->v = v;
  e->d = d;
  e->c = c;
  e->b = b;
  e->max_batch = max_batch;
  e->E = E;
  e->C = C;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t r = hipGetDevice(&e->device);
  if (r != hipSuccess) { free_engine(e); return hip_fail(r, "hipGetDevice"); }
  r = hipDeviceGetAttribute(&e->cus, hipDeviceAttributeMultiprocessorCount, e->device);
  if (r != hipSuccess || e->cus <= 0) { free_engine(e); return hip_fail(r, "device attributes"); }
  // batch-1 hand-over words: enough partials for the largest stage-2 grid of
  // any p (batch1_stage2_blocks never exceeds batch1_slots2)
  const int64_t ntag = fh::batch1_tag_words(c, e->cus);
  const int64_t nbtag = fh::batched_tag_words(c, (int)std::min<int64_t>(max_batch, 65535), e->cus);

  // partials per query: the row kernels' and the dense GEMMs' workgroups, or
  // (cluster-major stage 2, at most gather_cm_max_batch queries) one per
  // probe, p <= c
  const int64_t parts_per_q = std::max<int64_t>(
      {fh::rows_blocks(v, fh::kGatherRPW), fh::rows_blocks(v, fh::kDenseRPW),
       fh::mfma_blocks(v), fh::splitd_blocks(v), 4096});
  e->parts_total = std::max<int64_t>(
      max_batch * parts_per_q,
      std::min<int64_t>(max_batch, fh::gather_cm_max_batch()) * c * ((b + 15) / 16));
  struct Alloc { void** p; size_t bytes; const char* what; };
  const Alloc allocs[] = {
      {(void**)&e->c2t, sizeof(int32_t) * (size_t)v, "C2T"},
      {(void**)&e->t2c, sizeof(int32_t) * (size_t)v, "token clusters"},
      {(void**)&e->sumscores, sizeof(float) * (size_t)c, "summed scores"},
      {(void**)&e->nprobe, sizeof(int32_t) * (size_t)max_batch, "probe counts"},
      {(void**)&e->Ec, (size_t)(v * d) * (dtype == FH_BF16 ? 2 : 4), "cluster-contiguous E"},
      {(void**)&e->scores, sizeof(float) * (size_t)(max_batch * c), "scores"},
      {(void**)&e->sel, sizeof(int32_t) * (size_t)(max_batch * c), "selection"},
      {(void**)&e->mbits, sizeof(uint32_t) * (size_t)(max_batch * ((c + 31) / 32)), "probe bitsets"},
      {(void**)&e->mpre, sizeof(int32_t) * (size_t)(max_batch * ((c + 31) / 32)), "probe prefix counts"},
      {(void**)&e->parts, sizeof(fh::Part) * (size_t)e->parts_total, "partials"},
      {(void**)&e->sync, 4 * sizeof(unsigned), "sync flags"},
      {(void**)&e->tagged, sizeof(unsigned long long) * (size_t)ntag, "tagged hand-over words"},
      {(void**)&e->btag, sizeof(unsigned long long) * (size_t)nbtag, "batched hand-over words"},
  };
  for (const Alloc& a : allocs) {
    r = hipMalloc(a.p, a.bytes);
    if (r != hipSuccess) { free_engine(e); return hip_fail(r, a.what); }
  }
  r = hipMemcpyAsync(e->c2t, C2T, sizeof(int32_t) * (size_t)v, hipMemcpyHostToDevice, st);
  if (r == hipSuccess) r = hipMemsetAsync(e->sync, 0, 4 * sizeof(unsigned), st);
  if (r == hipSuccess)
    r = hipMemsetAsync(e->tagged, 0, sizeof(unsigned long long) * (size_t)ntag, st);
  if (r == hipSuccess)
    r = hipMemsetAsync(e->btag, 0, sizeof(unsigned long long) * (size_t)nbtag, st);
  if (r != hipSuccess) { free_engine(e); return hip_fail(r, "copy C2T"); }
  r = fh::launch_permute_rows(e->ctx(st), e->Ec);
  if (r != hipSuccess) { free_engine(e); return hip_fail(r, "cluster-contiguous E"); }
  if (dtype == FH_BF16 && max_batch >= 2) {  // what the batched matrix-core kernels read
    r = hipMalloc(&e->Ecm, (size_t)fh::fragment_order_bytes(c, b, (int)d));
    if (r == hipSuccess) r = fh::launch_fragment_order(e->Ec, c, b, (int)d, e->Ecm, st);
    if (r == hipSuccess && quant == FH_QUANT_NONE) {  // quantised centroids have their own layouts
      r = hipMalloc(&e->Cm, (size_t)fh::fragment_order_bytes(1, c, (int)d));
      if (r == hipSuccess) r = fh::launch_fragment_order(C, 1, c, (int)d, e->Cm, st);
    }
    if (r != hipSuccess) { free_engine(e); return hip_fail(r, "fragment-order E and C"); }
  }
  r = fh::launch_t2c(e->ctx(st), e->t2c);
  if (r != hipSuccess) { free_engine(e); return hip_fail(r, "token clusters"); }

  if (quant != FH_QUANT_NONE) {
    const int bits = quant == FH_QUANT_INT4_G32 ? 4 : 8;
    int* bad = nullptr;
    r = hipMalloc((void**)&e->cq, (size_t)(c * d * bits / 8));
    if (r == hipSuccess) r = hipMalloc((void**)&e->csig, sizeof(uint16_t) * (size_t)(c * d / 32));
    if (r == hipSuccess) r = hipMalloc((void**)&bad, sizeof(int));
    if (r == hipSuccess) r = hipMemsetAsync(bad, 0, sizeof(int), st);
    if (r == hipSuccess) r = fh::launch_quant(e->ctx(st), bad);
    int hbad = 0;
    if (r == hipSuccess) r = hipMemcpyAsync(&hbad, bad, sizeof(int), hipMemcpyDeviceToHost, st);
    if (r == hipSuccess) r = hipStreamSynchronize(st);
    (void)hipFree(bad);
    if (r != hipSuccess) { free_engine(e); return hip_fail(r, "centroid quantisation"); }
    if (hbad) { free_engine(e); return fail(FH_EINVAL, "a centroid group's scale overflows fp16"); }
    if (dtype == FH_BF16) {  // the MFMA layouts for batched stage 1 (INT8 rows are read as stored)
      if (bits == 4)  // fragment order: whole tiles of 16 rows
        r = hipMalloc((void**)&e->cq_mfma, (size_t)((c + 15) / 16 * 16 * fh::mfma_int4_row_bytes((int)d)));
      if (r == hipSuccess)
        r = hipMalloc((void**)&e->sig_mfma,
                      sizeof(uint16_t) * (size_t)((d / 32) * fh::mfma_sig_ld(c)));
      if (r == hipSuccess) r = fh::launch_mfma_relayout(e->ctx(st), e->cq_mfma, e->sig_mfma);
      if (r == hipSuccess) r = hipStreamSynchronize(st);
      if (r != hipSuccess) { free_engine(e); return hip_fail(r, "MFMA layout"); }
    }
    e->C = nullptr;  // not borrowed in quantised modes
  } else {
    r = hipStreamSynchronize(st);
    if (r != hipSuccess) { free_engine(e); return hip_fail(r, "create"); }
  }
  *out = e;
  return FH_OK;
}

void fh_destroy(fh_engine* e) {
  if (!e) return;
  DeviceGuard g(e->device);
  (void)hipDeviceSynchronize();
  free_engine(e);
}

fh_status fh_score(fh_engine* e, const void* h, int64_t B, float* out_scores, void* stream) {
  g_err.clear();
  fh_status s = check_common(e, h, B);
  if (s != FH_OK) return s;
  if (!out_scores) return fail(FH_EINVAL, "out_scores is NULL");
  DeviceGuard g(e->device);
  if (!g.ok) return fail(FH_EHIP, "cannot select the engine's device");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const fh::KernelCtx k = e->ctx(st);
  hipError_t r = launch_stage1(e, st, k, h, B, out_scores);
  return r == hipSuccess ? FH_OK : hip_fail(r, "score launch");
}

fh_status fh_forward(fh_engine* e, const void* h, int64_t B, int64_t p, int mode, float temperature,
                     uint64_t seed, int32_t* out_token, float* out_token_logit, float* out_lse,
                     int32_t* out_clusters, int32_t* out_ids, float* out_logits, void* stream) {
  g_err.clear();
  fh_status s = check_common(e, h, B);
  if (s != FH_OK) return s;
  if (p < 1 || p > e->c)
    return fail(FH_EINVAL, "p=" + std::to_string(p) + " outside [1, c=" + std::to_string(e->c) + "]");
  s = check_mode(mode, temperature);
  if (s != FH_OK) return s;
  DeviceGuard g(e->device);
  if (!g.ok) return fail(FH_EHIP, "cannot select the engine's device");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const fh::KernelCtx k = e->ctx(st);
  const int probe_sample = mode & FH_PROBE_SAMPLE;
  const int token_sample = (mode & FH_TOKEN_SAMPLE) ? 1 : 0;
  const float tprime = token_sample ? temperature : 1.f;
  int32_t* S = out_clusters ? out_clusters : e->sel;

  // The single launch identifies a call by a host-side epoch baked into its
  // arguments, which a captured graph would replay unchanged; under stream
  // capture the per-stage launches (no state between calls) are used.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &capture) != hipSuccess) capture = hipStreamCaptureStatusNone;
  if (B == 1 && e->path == FH_PATH_AUTO && capture == hipStreamCaptureStatusNone &&
      fh::batch1_fits(p, e->b, e->cus)) {
    fh::FusedLaunch f{};
    f.ctx = &k;
    f.cus = e->cus;
    f.h = h;
    f.p = (int)p;
    f.probe_sample = probe_sample;
    f.token_sample = token_sample;
    f.temperature = temperature;
    f.tprime = tprime;
    f.seed = seed;
    e->epoch = e->epoch == 0xFFFFFFFFu ? 1u : e->epoch + 1u;
    f.epoch = e->epoch;
    f.tscores = e->tagged;
    f.tsel = e->tagged + fh::batch1_off_sel(e->c);
    f.tparts = e->tagged + fh::batch1_off_parts(e->c);
    f.out_clusters = out_clusters;
    f.out_ids = out_ids;
    f.out_logits = out_logits;
    f.out_token = out_token;
    f.out_logit = out_token_logit;
    f.out_lse = out_lse;
    f.err = e->sync;
    hipError_t r = timed(e, st, "batch1", [&] { return fh::launch_batch1(f); });
    return r == hipSuccess ? FH_OK : hip_fail(r, "batch-1 launch");
  }

  if (mode & FH_PROBE_SHARED)
    return shared_forward(e, st, k, h, B, p, token_sample, tprime, seed, out_token, out_token_logit,
                          out_lse, out_clusters, out_ids, out_logits);

  // batches of bf16 queries that share probes: stage 2 cluster-major on the
  // matrix cores, each probed cluster's rows read once for all its queries
  const bool cm = e->dtype == FH_BF16 && e->Ecm && fh::gather_cm_fits((int)B, p, e->c);
  if (!cm && e->path == FH_PATH_AUTO && capture == hipStreamCaptureStatusNone &&
      fh::batched_fits(p, e->b, (int)B, e->cus)) {
    // small batches, query-major stage 2: stage 1, then the selection, stage 2
    // and the finish in one launch (its epoch, like the batch-1 kernel's, is
    // why captured calls take the per-stage launches)
    fh::KeyXform kx;
    kx.sample = probe_sample; kx.temperature = temperature; kx.seed = seed;
    hipError_t r = launch_stage1(e, st, k, h, B, e->scores, kx);
    if (r != hipSuccess) return hip_fail(r, "score launch");
    fh::BatchedLaunch f{};
    f.ctx = &k;
    f.cus = e->cus;
    f.H = h;
    f.B = (int)B;
    f.keys = e->scores;
    f.p = (int)p;
    f.token_sample = token_sample;
    f.tprime = tprime;
    f.seed = seed;
    e->epoch = e->epoch == 0xFFFFFFFFu ? 1u : e->epoch + 1u;
    f.epoch = e->epoch;
    f.tagged = e->btag;
    f.out_clusters = out_clusters;
    f.out_ids = out_ids;
    f.out_logits = out_logits;
    f.out_token = out_token;
    f.out_logit = out_token_logit;
    f.out_lse = out_lse;
    f.err = e->sync;
    r = timed(e, st, "batched", [&] { return fh::launch_batched(f); });
    return r == hipSuccess ? FH_OK : hip_fail(r, "batched launch");
  }
  // with sampled probes stage 1 stores the selection keys (the Gumbel draws
  // spread over its grid) and the selection takes them as they are
  fh::KeyXform kx;
  kx.sample = probe_sample; kx.temperature = temperature; kx.seed = seed;
  hipError_t r = launch_stage1(e, st, k, h, B, e->scores, kx);
  if (r != hipSuccess) return hip_fail(r, "score launch");
  r = timed(e, st, "select", [&] {
    return fh::launch_select(k, e->scores, (int)B, (int)p, 0, 1.f, seed, S, (int)p,
                             cm ? e->mbits : nullptr, cm ? e->mpre : nullptr);
  });
  if (r != hipSuccess) return hip_fail(r, "select launch");
  int64_t nparts = 0;
  if (cm)
    r = timed(e, st, "gather_cm", [&] {
      return fh::launch_gather_cm(k, e->cus, h, (int)B, (int)p, e->mbits, e->mpre, token_sample, tprime,
                                  seed, out_ids, out_logits, e->parts, &nparts);
    });
  else
    r = timed(e, st, "gather", [&] {
      return fh::launch_gather(k, h, (int)B, S, (int)p, token_sample, tprime, seed, out_ids,
                               out_logits, e->parts, &nparts);
    });
  if (r != hipSuccess) return hip_fail(r, "gather launch");
  r = timed(e, st, "finish", [&] {
    return fh::launch_finish(k, e->parts, (int)B, nparts, out_token, out_token_logit, out_lse);
  });
  if (r != hipSuccess) return hip_fail(r, "finish launch");
  return FH_OK;
}

fh_status fh_forward_adaptive(fh_engine* e, const void* h, int64_t B, int64_t p_max,
                              int64_t p_min, float tau, int mode, float temperature,
                              uint64_t seed, int32_t* out_nprobe, int32_t* out_token,
                              float* out_token_logit, float* out_lse, int32_t* out_clusters,
                              int32_t* out_ids, float* out_logits, void* stream) {
  g_err.clear();
  fh_status s = check_common(e, h, B);
  if (s != FH_OK) return s;
  const int64_t pcap = std::min<int64_t>(e->c, 1024);
  if (p_min < 1 || p_min > p_max || p_max > pcap)
    return fail(FH_EINVAL, "need 1 <= p_min <= p_max <= min(c, 1024) (p_min=" +
                               std::to_string(p_min) + ", p_max=" + std::to_string(p_max) + ")");
  if (!(tau > 0.f && tau <= 1.f)) return fail(FH_EINVAL, "tau must lie in (0, 1]");
  if (mode & FH_PROBE_SHARED)
    return fail(FH_EINVAL, "the adaptive count is per query; FH_PROBE_SHARED does not apply");
  s = check_mode(mode, temperature);
  if (s != FH_OK) return s;
  if (!(temperature > 0.f && std::isfinite(temperature)))
    return fail(FH_EINVAL, "the probe mass needs a finite temperature > 0");
  DeviceGuard g(e->device);
  if (!g.ok) return fail(FH_EHIP, "cannot select the engine's device");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const fh::KernelCtx k = e->ctx(st);
  const int probe_sample = mode & FH_PROBE_SAMPLE;
  const int token_sample = (mode & FH_TOKEN_SAMPLE) ? 1 : 0;
  const float tprime = token_sample ? temperature : 1.f;
  int32_t* S = out_clusters ? out_clusters : e->sel;
  int32_t* np = out_nprobe ? out_nprobe : e->nprobe;

  // B = 1: the single launch, its selector taking the count (as fh_forward)
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &capture) != hipSuccess) capture = hipStreamCaptureStatusNone;
  if (B == 1 && e->path == FH_PATH_AUTO && capture == hipStreamCaptureStatusNone &&
      fh::batch1_fits(p_max, e->b, e->cus)) {
    fh::FusedLaunch f{};
    f.ctx = &k;
    f.cus = e->cus;
    f.h = h;
    f.p = (int)p_max;
    f.probe_sample = probe_sample;
    f.token_sample = token_sample;
    f.temperature = temperature;
    f.tprime = tprime;
    f.seed = seed;
    e->epoch = e->epoch == 0xFFFFFFFFu ? 1u : e->epoch + 1u;
    f.epoch = e->epoch;
    f.tscores = e->tagged;
    f.tsel = e->tagged + fh::batch1_off_sel(e->c);
    f.tparts = e->tagged + fh::batch1_off_parts(e->c);
    f.tau = tau;
    f.pmin = (int)p_min;
    f.out_nprobe = out_nprobe;
    f.out_clusters = out_clusters;
    f.out_ids = out_ids;
    f.out_logits = out_logits;
    f.out_token = out_token;
    f.out_logit = out_token_logit;
    f.out_lse = out_lse;
    f.err = e->sync;
    hipError_t r = timed(e, st, "batch1_adaptive", [&] { return fh::launch_batch1(f); });
    return r == hipSuccess ? FH_OK : hip_fail(r, "batch-1 launch");
  }

  // stage 1 keeps the raw scores (the mass needs them); the selection forms
  // the keys itself
  hipError_t r = launch_stage1(e, st, k, h, B, e->scores);
  if (r != hipSuccess) return hip_fail(r, "score launch");
  r = timed(e, st, "select", [&] {
    return fh::launch_select(k, e->scores, (int)B, (int)p_max, probe_sample, temperature, seed, S,
                             (int)p_max);
  });
  if (r != hipSuccess) return hip_fail(r, "select launch");
  // batches of bf16 queries: the cluster-major stage 2 over the kept probes'
  // bitsets, each kept cluster's rows read once for all queries keeping it
  const bool cm = e->dtype == FH_BF16 && e->Ecm && fh::gather_cm_fits((int)B, p_max, e->c);
  r = timed(e, st, "adapt", [&] {
    return fh::launch_adapt(k, e->scores, (int)B, (int)p_max, (int)p_min, tau, probe_sample,
                            temperature, seed, S, np, out_ids, out_logits,
                            cm ? e->mbits : nullptr, cm ? e->mpre : nullptr);
  });
  if (r != hipSuccess) return hip_fail(r, "adaptive count launch");
  int64_t nparts = 0;
  if (cm)
    r = timed(e, st, "gather_cm", [&] {
      return fh::launch_gather_cm(k, e->cus, h, (int)B, (int)p_max, e->mbits, e->mpre,
                                  token_sample, tprime, seed, out_ids, out_logits, e->parts,
                                  &nparts);
    });
  else
    r = timed(e, st, "gather", [&] {
      return fh::launch_gather(k, h, (int)B, S, (int)p_max, token_sample, tprime, seed, out_ids,
                               out_logits, e->parts, &nparts, -1, np);
    });
  if (r != hipSuccess) return hip_fail(r, "gather launch");
  // the cluster-major partials of a query's ranks past its count are unwritten
  r = timed(e, st, "finish", [&] {
    return fh::launch_finish(k, e->parts, (int)B, nparts, out_token, out_token_logit, out_lse,
                             cm ? np : nullptr, (int)((e->b + 15) / 16));
  });
  return r == hipSuccess ? FH_OK : hip_fail(r, "finish launch");
}

fh_status fh_forward_noalloc(const void* E, const void* C, const int32_t* c2t, fh_dtype dtype,
                             int64_t v, int64_t d, int64_t c, const void* h, int64_t B, int64_t p,
                             int mode, float temperature, uint64_t seed, int32_t* out_token,
                             float* out_token_logit, float* out_lse, int32_t* out_clusters,
                             int32_t* out_ids, float* out_logits, void* stream) {
  g_err.clear();
  if (!E || !C || !c2t || !h) return fail(FH_EINVAL, "E, C, C2T and h must be non-NULL");
  if (dtype != FH_F32 && dtype != FH_BF16) return fail(FH_EINVAL, "unknown dtype");
  if (v <= 0 || d <= 0 || c <= 0) return fail(FH_EINVAL, "v, d and c must be positive");
  if (v % c != 0) return fail(FH_EINVAL, "v must be a multiple of c (balanced clusters)");
  if (v >= (int64_t(1) << 31)) return fail(FH_EUNSUPPORTED, "v must be below 2^31");
  if (c > kMaxC) return fail(FH_EUNSUPPORTED, "c above 16384 is not supported");
  const int epc = dtype == FH_BF16 ? 8 : 4;
  if (d % epc != 0)
    return fail(FH_EINVAL, dtype == FH_BF16 ? "bf16 needs d % 8 == 0" : "f32 needs d % 4 == 0");
  if (d > 64 * 8 * epc) return fail(FH_EUNSUPPORTED, "d too large for this library");
  if (!aligned16(E) || !aligned16(C) || !aligned16(h))
    return fail(FH_EINVAL, "E, C and h must be 16-byte aligned");
  if (B < 1 || B > 65535) return fail(FH_EINVAL, "B outside [1, 65535]");
  if (p < 1 || p > c)
    return fail(FH_EINVAL, "p=" + std::to_string(p) + " outside [1, c=" + std::to_string(c) + "]");
  if (mode & FH_PROBE_SHARED) return fail(FH_EUNSUPPORTED, "FH_PROBE_SHARED is not offered here");
  fh_status s = check_mode(mode, temperature);
  if (s != FH_OK) return s;
  const int64_t b = v / c;
  // workspace: scores [B x c] fp32, probe lists [B x p] (unless out_clusters
  // takes them), stage-2 partials [B x rows_blocks(p b)]
  const int64_t nparts = fh::rows_blocks(p * b, fh::kGatherRPW);
  const size_t off_sel = align256(sizeof(float) * (size_t)(B * c));
  const size_t off_parts = off_sel + align256(sizeof(int32_t) * (size_t)(B * p));
  const size_t need = off_parts + sizeof(fh::Part) * (size_t)(B * nparts);
  if (need > kNoAllocScratchBytes)
    return fail(FH_EINVAL, "this call needs " + std::to_string(need) +
                               " bytes of workspace; fh_forward_noalloc has " +
                               std::to_string(kNoAllocScratchBytes) + " (use fh_forward)");
  int dev = -1;
  hipError_t r = hipGetDevice(&dev);
  if (r != hipSuccess) return hip_fail(r, "hipGetDevice");
  unsigned char* ws = nullptr;
  r = scratch_for(dev, reinterpret_cast<void**>(&ws));
  if (r != hipSuccess) return hip_fail(r, "workspace address (hipGetSymbolAddress)");
  float* scores = reinterpret_cast<float*>(ws);
  int32_t* S = out_clusters ? out_clusters : reinterpret_cast<int32_t*>(ws + off_sel);
  fh::Part* parts = reinterpret_cast<fh::Part*>(ws + off_parts);

  hipStream_t st = static_cast<hipStream_t>(stream);
  fh::KernelCtx k;
  k.bf16 = dtype == FH_BF16;
  k.E = E;
  k.Ec = nullptr;  // rows of E are found through C2T
  k.C = C;
  k.c2t = c2t;
  k.cq = nullptr;
  k.csig = nullptr;
  k.cq_mfma = nullptr;
  k.sig_mfma = nullptr;
  k.v = v;
  k.c = c;
  k.b = b;
  k.d = (int)d;
  k.stream = st;
  k.qbits = 0;
  const int probe_sample = mode & FH_PROBE_SAMPLE;
  const int token_sample = (mode & FH_TOKEN_SAMPLE) ? 1 : 0;
  const float tprime = token_sample ? temperature : 1.f;
  fh::KeyXform kx;
  kx.sample = probe_sample; kx.temperature = temperature; kx.seed = seed;
  r = fh::launch_score(k, h, (int)B, scores, kx);
  if (r != hipSuccess) return hip_fail(r, "score launch");
  r = fh::launch_select(k, scores, (int)B, (int)p, 0, 1.f, seed, S, (int)p);
  if (r != hipSuccess) return hip_fail(r, "select launch");
  int64_t np = 0;
  r = fh::launch_gather(k, h, (int)B, S, (int)p, token_sample, tprime, seed, out_ids, out_logits,
                        parts, &np);
  if (r != hipSuccess) return hip_fail(r, "gather launch");
  r = fh::launch_finish(k, parts, (int)B, np, out_token, out_token_logit, out_lse);
  return r == hipSuccess ? FH_OK : hip_fail(r, "finish launch");
}

fh_status fh_probs_fp8(const float* logits, const float* lse, int64_t B, int64_t n,
                       float temperature, uint8_t* out_probs, int32_t* out_scale_exp,
                       void* stream) {
  g_err.clear();
  if (!logits || !lse || !out_probs || !out_scale_exp)
    return fail(FH_EINVAL, "logits, lse, out_probs and out_scale_exp must not be NULL");
  if (B < 1 || B > 65535) return fail(FH_EINVAL, "B outside [1, 65535]");
  if (n < 1 || n > (int64_t(1) << 31)) return fail(FH_EINVAL, "n outside [1, 2^31]");
  if (!(temperature > 0.f && std::isfinite(temperature)))
    return fail(FH_EINVAL, "temperature must be finite and > 0");
  hipError_t r = fh::launch_probs_fp8(logits, lse, B, n, temperature, out_probs, out_scale_exp,
                                      static_cast<hipStream_t>(stream));
  return r == hipSuccess ? FH_OK : hip_fail(r, "fp8 probabilities launch");
}

fh_status fh_dense_forward(fh_engine* e, const void* h, int64_t B, int mode, float temperature,
                           uint64_t seed, int32_t* out_token, float* out_token_logit,
                           float* out_lse, float* out_logits, void* stream) {
  g_err.clear();
  fh_status s = check_common(e, h, B);
  if (s != FH_OK) return s;
  if (mode & FH_PROBE_SAMPLE) return fail(FH_EINVAL, "the dense head has no probe stage");
  s = check_mode(mode, temperature);
  if (s != FH_OK) return s;
  DeviceGuard g(e->device);
  if (!g.ok) return fail(FH_EHIP, "cannot select the engine's device");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const fh::KernelCtx k = e->ctx(st);
  const int token_sample = (mode & FH_TOKEN_SAMPLE) ? 1 : 0;
  const float tprime = token_sample ? temperature : 1.f;
  int64_t nparts = 0;
  hipError_t r;
  if (e->dtype == FH_BF16 && B >= fh::kMfmaMinBatchDense)
    r = timed(e, st, "dense_mfma", [&] {
      return fh::launch_dense_mfma(k, e->cus, h, (int)B, token_sample, tprime, seed, out_logits,
                                   e->parts, &nparts);
    });
  else
    r = timed(e, st, "dense", [&] {
      return fh::launch_dense(k, h, (int)B, token_sample, tprime, seed, out_logits, e->parts,
                              &nparts);
    });
  if (r != hipSuccess) return hip_fail(r, "dense launch");
  r = timed(e, st, "finish", [&] {
    return fh::launch_finish(k, e->parts, (int)B, nparts, out_token, out_token_logit, out_lse);
  });
  if (r != hipSuccess) return hip_fail(r, "finish launch");
  return FH_OK;
}

fh_status fh_spec_verify(fh_engine* e, const void* h, int64_t B, int64_t p,
                         const int32_t* draft_clusters, const int32_t* draft_token,
                         const float* draft_lse, float temperature, uint64_t seed,
                         int32_t* out_token, int32_t* out_accepted, float* out_lse,
                         void* stream) {
  g_err.clear();
  fh_status s = check_common(e, h, B);
  if (s != FH_OK) return s;
  if (p < 1 || p > e->c)
    return fail(FH_EINVAL, "p=" + std::to_string(p) + " outside [1, c=" + std::to_string(e->c) + "]");
  if (!draft_clusters || !draft_token || !draft_lse || !out_token)
    return fail(FH_EINVAL, "draft_clusters, draft_token, draft_lse and out_token must not be NULL");
  if (!(temperature > 0.f && std::isfinite(temperature)))
    return fail(FH_EINVAL, "speculative sampling needs a finite temperature > 0");
  DeviceGuard g(e->device);
  if (!g.ok) return fail(FH_EHIP, "cannot select the engine's device");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const fh::KernelCtx k = e->ctx(st);
  const hipError_t r = timed(e, st, "spec_verify", [&] {
    return fh::launch_spec_verify(k, e->cus, e->t2c, e->mbits, e->parts, h, (int)B, (int)p, draft_clusters,
                                  draft_token, draft_lse, temperature, seed, out_token,
                                  out_accepted, out_lse);
  });
  return r == hipSuccess ? FH_OK : hip_fail(r, "speculative verification");
}

fh_status fh_set_path(fh_engine* e, int path) {
  g_err.clear();
  if (!e) return fail(FH_EINVAL, "engine is NULL");
  if (path != FH_PATH_AUTO && path != FH_PATH_MULTI) return fail(FH_EINVAL, "unknown path");
  e->path = path;
  return FH_OK;
}

fh_status fh_sync_status(fh_engine* e, void* stream) {
  g_err.clear();
  if (!e) return fail(FH_EINVAL, "engine is NULL");
  DeviceGuard g(e->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned flags[4] = {0, 0, 0, 0};
  hipError_t r = hipMemcpyAsync(flags, e->sync, sizeof(flags), hipMemcpyDeviceToHost, st);
  if (r == hipSuccess) r = hipStreamSynchronize(st);
  if (r != hipSuccess) return hip_fail(r, "sync status");
  if (flags[0]) return fail(FH_EHIP, "a batch-1 hand-over poll gave up (outputs invalid)");
  return FH_OK;
}

fh_status fh_get_int4(fh_engine* e, uint8_t* packed, uint16_t* scales, void* stream) {
  g_err.clear();
  if (!e) return fail(FH_EINVAL, "engine is NULL");
  if (e->quant != FH_QUANT_INT4_G32) return fail(FH_EINVAL, "engine is not INT4");
  if (!packed || !scales) return fail(FH_EINVAL, "NULL output");
  DeviceGuard g(e->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t r = hipMemcpyAsync(packed, e->cq, (size_t)(e->c * e->d / 2), hipMemcpyDeviceToDevice, st);
  if (r == hipSuccess)
    r = hipMemcpyAsync(scales, e->csig, sizeof(uint16_t) * (size_t)(e->c * e->d / 32),
                       hipMemcpyDeviceToDevice, st);
  return r == hipSuccess ? FH_OK : hip_fail(r, "copy INT4 centroids");
}

fh_status fh_get_int8(fh_engine* e, int8_t* codes, uint16_t* scales, void* stream) {
  g_err.clear();
  if (!e) return fail(FH_EINVAL, "engine is NULL");
  if (e->quant != FH_QUANT_INT8_G32) return fail(FH_EINVAL, "engine is not INT8");
  if (!codes || !scales) return fail(FH_EINVAL, "NULL output");
  DeviceGuard g(e->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t r = hipMemcpyAsync(codes, e->cq, (size_t)(e->c * e->d), hipMemcpyDeviceToDevice, st);
  if (r == hipSuccess)
    r = hipMemcpyAsync(scales, e->csig, sizeof(uint16_t) * (size_t)(e->c * e->d / 32),
                       hipMemcpyDeviceToDevice, st);
  return r == hipSuccess ? FH_OK : hip_fail(r, "copy INT8 centroids");
}

fh_status fh_profile_begin(fh_engine* e, int64_t max_launches) {
  g_err.clear();
  if (!e) return fail(FH_EINVAL, "engine is NULL");
  if (max_launches < 1 || max_launches > (1 << 20)) return fail(FH_EINVAL, "max_launches outside [1, 2^20]");
  DeviceGuard g(e->device);
  for (hipEvent_t ev : e->prof_ev) (void)hipEventDestroy(ev);
  e->prof_ev.assign((size_t)(2 * max_launches), nullptr);
  e->prof_name.assign((size_t)max_launches, nullptr);
  for (auto& ev : e->prof_ev) {
    hipError_t r = hipEventCreate(&ev);
    if (r != hipSuccess) {
      e->prof = false;
      return hip_fail(r, "hipEventCreate");
    }
  }
  e->prof_cap = max_launches;
  e->prof_n = 0;
  e->prof = true;
  return FH_OK;
}

fh_status fh_profile_end(fh_engine* e, fh_kernel_time* out, int max, int* count) {
  g_err.clear();
  if (!e) return fail(FH_EINVAL, "engine is NULL");
  if (!e->prof) return fail(FH_EINVAL, "profiling was not started");
  DeviceGuard g(e->device);
  e->prof = false;
  std::vector<std::pair<const char*, std::pair<int64_t, double>>> agg;
  for (int64_t i = 0; i < e->prof_n; ++i) {
    hipError_t r = hipEventSynchronize(e->prof_ev[2 * i + 1]);
    if (r != hipSuccess) return hip_fail(r, "hipEventSynchronize");
    float ms = 0.f;
    r = hipEventElapsedTime(&ms, e->prof_ev[2 * i], e->prof_ev[2 * i + 1]);
    if (r != hipSuccess) return hip_fail(r, "hipEventElapsedTime");
    const char* nm = e->prof_name[i];
    size_t j = 0;
    while (j < agg.size() && std::strcmp(agg[j].first, nm) != 0) ++j;
    if (j == agg.size()) agg.push_back({nm, {0, 0.0}});
    agg[j].second.first += 1;
    agg[j].second.second += ms;
  }
  int n = 0;
  for (size_t j = 0; j < agg.size() && n < max; ++j, ++n) {
    out[n].name = agg[j].first;
    out[n].launches = agg[j].second.first;
    out[n].total_ms = agg[j].second.second;
  }
  if (count) *count = n;
  for (hipEvent_t ev : e->prof_ev) (void)hipEventDestroy(ev);
  e->prof_ev.clear();
  e->prof_name.clear();
  e->prof_n = e->prof_cap = 0;
  return FH_OK;
}

}  // extern "C"
