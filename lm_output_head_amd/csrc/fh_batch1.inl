// The single-launch batch-1 kernel, instantiated per storage type and
// stage-1 storage by the fh_batch1_*.hip translation units, which define
//   FH_BATCH1_T      element type of E, C and h (uint16_t = bf16, float)
//   FH_BATCH1_QB     stage-1 centroid codes: 0 (as stored), 4 (INT4 g32), 8 (INT8 g32)
//   FH_BATCH1_ENTRY  name of the exported launcher
//
// Sources (page title and section): FlashHead technical explainer
// (framerc.cn) §1.2.2-§1.2.4, §2.2.2; "FlashHead: Efficient Drop-In
// Replacement for the Classification Head in Language Model Inference"
// (arXiv 2603.14591), abstract.

#include "fh_blocks.hpp"

namespace fh {

// ======================================================================
// Batch-1 path: the whole call in one launch.
//
// The grid's workgroups (1024 threads) take roles by index, in the order
// they are dispatched:
//   [0, G1)        stage 1: rows1 centroid rows each (wave w takes rows w,
//                  w + 16, ...), each score stored as soon as it is reduced;
//   [G1, G1+G2)    stage 2: rows2 of the p*b retrieved tokens each, with the
//                  fused epilogue.  The first of them (G1) is also the
//                  selector: before its own rows it waits for the c scores,
//                  selects the probes and publishes them as a bitset over
//                  the clusters; each stage-2 workgroup finds the probes of
//                  its rows by a prefix count over that bitset.
//   G1+G2          the finisher: polls the G2 stage-2 partials and merges
//                  them in index order.  G2 <= CUs - 1, so it finds a CU as
//                  soon as stage 1 retires and its polls overlap stage 2.
// Results pass between workgroups as 64-bit words tagged with the call's
// epoch (epoch << 32 | payload), written and polled with agent-scope (sc1)
// accesses.  A workgroup only ever waits for words written by workgroups
// with smaller indices.  Like a decoupled look-back scan, this relies on
// workgroups being dispatched in index order, so every awaited workgroup is
// already running and never waits for its waiter; the grid need not be
// co-resident.  Sizes keep G1 < CUs and G2 < CUs so that at one workgroup
// per CU the selector starts at once and every stage-2 workgroup and the
// finisher are resident when stage 1 retires.  Every wait is bounded: past kSpinLimit polls the waiter sets
// *err and goes on with what it has, so the grid always drains.
// ======================================================================
struct FusedArgs {
  const void* E;
  const void* Ec;  // cluster-contiguous copy of E, or null
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
  float zq;  // selection threshold quantile (select_quantile)
  uint64_t seed;
  int g1, g2;                   // stage-1 and stage-2 workgroup counts
  int rows1, rows2;             // rows per stage-1 / stage-2 workgroup
  unsigned epoch;               // never 0
  unsigned long long* tscores;  // [c] tagged scores
  unsigned long long* tsel;     // [ceil(c/32)] tagged bitset of the probes
  unsigned long long* tparts;   // [5 x g2] tagged Parts
  int32_t* out_clusters;        // [p] or null
  int32_t* out_ids;
  float* out_logits;
  int32_t* out_token;
  float* out_logit;
  float* out_lse;
  unsigned* err;  // sticky: a poll gave up
};

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

template <typename T, int MAXM, int KP, int QB, int MAXG>
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
    // probe sampling: the Gumbel-perturbed key s/T + G is formed here, one
    // row per lane-0 store, so the selector only ranks (keys saturate as in
    // the selection)
    auto sink = [&](int, int64_t r, int64_t, float s) {
      if (lane == 0) {
        if (a.probe_sample) s = s / a.temperature + gumbel_at(a.seed, 0u, (uint32_t)r, 0u);
        st_tagged(a.tscores + r, tag(a.epoch, __float_as_uint(saturate_key(s))));
      }
    };
    if constexpr (QB != 0) {
      HGroups<MAXG> hg[1];
      load_hgroups<T, MAXG>(hp, a.d / 32, lane, hg[0]);
      wave_rows_q<QB, MAXG, 1>(a.cq, a.csig, a.d, lane, hg, 1, r_lo + wave, r_hi, 16, sink);
    } else {
      uint4 hv[1][MAXM];
      load_hslice<T, MAXM>(hp, a.d / Chunk<T>::kElems, lane, hv[0]);
      auto same = [](int64_t r) { return r; };
      wave_rows<T, MAXM, 1>(static_cast<const T*>(a.C), a.d, lane, hv, 1, r_lo + wave, r_hi, 16,
                            same, same, sink);
    }
    FH_TRACE(1);
#ifdef FH_PHASE_TRACE
    __syncthreads();
    FH_TRACE(7);  // every wave of this workgroup is done
#endif
    return;
  }

  if (w == a.g1 + a.g2) {  // ---- finisher: the stage-2 partials in a fixed order
    // waves [0, nwv) hold partials: part i goes to thread i mod 1024
    const int nwv = min(16, (a.g2 + 63) / 64);
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
    if (wave < nwv) {
      acc = wave_merge_part(acc);
      if (lane == 0) sh.parts[wave] = acc;
    }
    __syncthreads();
    Part r = sh.parts[0];
    for (int w2 = 1; w2 < nwv; ++w2) r = part_merge(r, sh.parts[w2]);
    if (threadIdx.x == 0) write_outputs(r, 0, a.out_token, a.out_logit, a.out_lse);
    FH_TRACE(14);
    return;
  }

  const int j = w - a.g1;  // stage-2 workgroup index
  if (j == 0) {            // ---- selector
    FH_TRACE(2);
    // every thread waits for the keys of clusters k = tid + 1024 i, which
    // stage 1 has already Gumbel-perturbed when probes are sampled
    select_clear(sh.sel);
    unsigned long long* ptr[KP];
    bool live[KP];
    uint32_t raw[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int k = (int)threadIdx.x + kSelThreads * i;
      live[i] = k < a.c;
      ptr[i] = a.tscores + (live[i] ? k : 0);
    }
    poll_tagged<KP>(ptr, live, a.epoch, a.err, raw);
    float x[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) x[i] = live[i] ? __uint_as_float(raw[i]) : -FLT_MAX;
    __syncthreads();
    select_bits<KP>(x, a.c, a.p, a.zq, sh.sel);
    // publish the chosen clusters as a bitset, one tagged word per 32
    for (int t = threadIdx.x; t < (a.c + 31) / 32; t += kSelThreads)
      st_tagged(a.tsel + t, tag(a.epoch, sh.sel.selbits[t]));
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
  // the probes this workgroup's rows come from: positions [pos0, pos0+npos)
  // of the ascending probe list, read off the selector's bitset
  const int pos0 = (int)(r_lo / a.bsz);
  const int npos = r_hi > r_lo ? (int)((r_hi - 1) / a.bsz) - pos0 + 1 : 0;
  if (npos > 0) {
    const int nw = (a.c + 31) / 32;
    const int t = threadIdx.x;
    uint32_t word = 0u;
    if (t < nw) {
      unsigned long long* const ptr[1] = {a.tsel + t};
      const bool live[1] = {true};
      uint32_t got[1];
      poll_tagged<1>(ptr, live, a.epoch, a.err, got);
      word = got[0];
    }
    int tot;
    int pos = block_exclusive_scan(__popc(word), sh.sel.red_scan, &tot);
    if (pos < pos0 + npos && pos + __popc(word) > pos0) {
      for (uint32_t bitsleft = word; bitsleft; bitsleft &= bitsleft - 1, ++pos) {
        if (pos < pos0 || pos >= pos0 + npos) continue;
        const int k = 32 * t + __builtin_ctz(bitsleft);
        sh.probes[pos - pos0] = k;
        // the workgroup holding a probe's first row reports it
        if (a.out_clusters && (int64_t)pos * a.bsz >= r_lo) a.out_clusters[pos] = k;
      }
    }
  }
  __syncthreads();
  FH_TRACE(5);
  Part part[1] = {part_empty()};
  // slot f of the clustering; with the cluster-contiguous copy of E it is
  // also the row, else the row is the token C2T[f]
  auto src_of = [&](int64_t r) -> int64_t {
    const int64_t f = (int64_t)sh.probes[r / a.bsz - pos0] * a.bsz + r % a.bsz;
    return a.Ec ? f : (int64_t)a.c2t[f];
  };
  auto tok_of = [&](int64_t src) -> int64_t { return a.Ec ? (int64_t)a.c2t[src] : src; };
  auto sink = [&](int, int64_t r, int64_t src, float z) {
    if (lane == 0) {
      if (a.out_logits) a.out_logits[r] = z;
      if (a.out_ids) a.out_ids[r] = (int32_t)src;
    }
    part[0] = part_merge(part[0], part_of(z, (int32_t)src, a.token_sample, a.tprime, a.seed, 0u));
  };
  // four rows in flight per wave when the register slice allows it
  wave_rows<T, MAXM, 1, (MAXM <= 4 ? 4 : 2)>(static_cast<const T*>(a.Ec ? a.Ec : a.E), a.d, lane,
                                             hv, 1, r_lo + wave, r_hi, 16, src_of, tok_of, sink);
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
}

static FusedArgs fused_args(const FusedLaunch& f) {
  const KernelCtx& k = *f.ctx;
  FusedArgs a{};
  a.E = k.E; a.Ec = k.Ec; a.C = k.C; a.cq = k.cq; a.csig = k.csig; a.c2t = k.c2t;
  a.c = (int)k.c; a.bsz = (int)k.b; a.d = k.d; a.h = f.h; a.p = f.p;
  a.probe_sample = f.probe_sample; a.token_sample = f.token_sample;
  a.temperature = f.temperature; a.tprime = f.tprime; a.seed = f.seed;
  a.rows1 = (int)batch1_rows(k.c, batch1_slots1(f.cus));
  a.rows2 = (int)batch1_rows((int64_t)f.p * k.b, batch1_slots2(f.cus));
  a.g1 = batch1_stage1_blocks(k.c, f.cus);
  a.g2 = batch1_stage2_blocks(f.p, k.b, f.cus);
  a.epoch = f.epoch; a.tscores = f.tscores; a.tsel = f.tsel; a.tparts = f.tparts;
  a.out_clusters = f.out_clusters; a.out_ids = f.out_ids; a.out_logits = f.out_logits;
  a.out_token = f.out_token; a.out_logit = f.out_logit; a.out_lse = f.out_lse;
  a.err = f.err;
  a.zq = select_quantile(k.c, f.p);
  return a;
}

template <typename T, int MAXM, int KP, int QB, int MAXG>
static hipError_t b1_go(const FusedLaunch& f, const FusedArgs& a) {
  const unsigned grid = (unsigned)(a.g1 + a.g2 + 1);
  hipLaunchKernelGGL((k_batch1<T, MAXM, KP, QB, MAXG>), dim3(grid), dim3(1024), 0,
                     f.ctx->stream, a);
  return hipGetLastError();
}

template <typename T, int KP, int QB, int MAXG>
static hipError_t b1_m(const FusedLaunch& f, const FusedArgs& a) {
  const int nch = f.ctx->d / Chunk<T>::kElems;
  // register slices rounded up to 1, 2, 4, 6 or 8 chunks per lane (the
  // extra ones stay zero and load nothing)
  switch ((nch + 63) / 64) {
    case 1: return b1_go<T, 1, KP, QB, MAXG>(f, a);
    case 2: return b1_go<T, 2, KP, QB, MAXG>(f, a);
    case 3: case 4: return b1_go<T, 4, KP, QB, MAXG>(f, a);
    case 5: case 6: return b1_go<T, 6, KP, QB, MAXG>(f, a);
    case 7: case 8: return b1_go<T, 8, KP, QB, MAXG>(f, a);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int QB, int MAXG>
static hipError_t b1_k(const FusedLaunch& f, const FusedArgs& a) {
  switch (sel_keys_per_thread(f.ctx->c)) {
    case 1: return b1_m<T, 1, QB, MAXG>(f, a);
    case 2: return b1_m<T, 2, QB, MAXG>(f, a);
    case 8: return b1_m<T, 8, QB, MAXG>(f, a);
    case 16: return b1_m<T, 16, QB, MAXG>(f, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t FH_BATCH1_ENTRY(const FusedLaunch& f) {
  const FusedArgs a = fused_args(f);
  if constexpr (FH_BATCH1_QB == 0) {
    return b1_k<FH_BATCH1_T, 0, 1>(f, a);
  } else {
    switch ((f.ctx->d / 32 + 63) / 64) {
      case 1: return b1_k<FH_BATCH1_T, FH_BATCH1_QB, 1>(f, a);
      case 2: return b1_k<FH_BATCH1_T, FH_BATCH1_QB, 2>(f, a);
      default: return hipErrorInvalidValue;
    }
  }
}

}  // namespace fh
