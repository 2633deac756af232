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
#include "fh_handover.hpp"

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
//                  its rows by a prefix count over that bitset.  With the
//                  adaptive count (tau > 0) stage 1 publishes raw scores, the
//                  selector forms the keys, takes the top p, keeps the first
//                  n of them in key order (adaptive_count) and publishes only
//                  those; stage 2 then scores the n b rows the bitset's
//                  total names and pads the rest of its range.
//   G1+G2          the finisher: one wave polls the G2 stage-2 partials and
//                  merges them in a fixed order.  G2 <= CUs - 1, so it finds a CU as
//                  soon as stage 1 retires and its polls overlap stage 2.
// Results pass between workgroups as 64-bit words tagged with the call's
// epoch (epoch << 32 | payload), written and polled with agent-scope (sc1)
// accesses.  A workgroup only ever waits for words written by workgroups
// with smaller indices.  Like a decoupled look-back scan, this relies on
// workgroups being dispatched in index order, so every awaited workgroup is
// already running and never waits for its waiter; the grid need not be
// co-resident.  Sizes keep G1 < CUs and G2 < CUs so that at one workgroup
// per CU the selector starts at once and every stage-2 workgroup and the
// finisher are resident when stage 1 retires.  Every wait is bounded: past
// kSpinLimit polls the waiter sets *err and goes on with what it has, so the
// grid always drains; indices derived from a word that never arrived are
// clamped to valid rows, a stage-2 workgroup that gave up (the selector's
// key poll included) publishes its partial with id kBadPart, and the
// finisher then writes token -1 with a NaN logit and LSE.
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
  float tau;  // adaptive probe count: the mass to reach (0: a fixed p)
  int pmin;   // adaptive: the smallest count
  uint64_t seed;
  int g1, g2;                   // stage-1 and stage-2 workgroup counts
  int rows1, rows2;             // rows per stage-1 / stage-2 workgroup
  unsigned epoch;               // never 0
  unsigned long long* tscores;  // [c] tagged scores
  unsigned long long* tsel;     // [ceil(c/32)] tagged bitset of the probes
  unsigned long long* tparts;   // [5 x g2] tagged Parts
  int32_t* out_clusters;        // [p] or null
  int32_t* out_nprobe;          // [1] or null (adaptive)
  int32_t* out_ids;
  float* out_logits;
  int32_t* out_token;
  float* out_logit;
  float* out_lse;
  unsigned* err;  // sticky: a poll gave up
};

union Batch1Shared {
  SelShared sel;
  Part parts[1024];
  int probes[1024];
};

// What a stage-2 workgroup works on: rows [r_lo, r_hi) of one query's p b
// retrieved rows, that query's tagged probe bitset, its outputs, and the
// five words its partial goes to.
struct Stage2Job {
  const void* E;
  const void* Ec;
  const int32_t* c2t;
  int c, bsz, d, p;
  float tau;                     // adaptive count: the bitset's total is n (0: fixed p)
  const void* h;                 // the query's hidden state
  uint32_t row;                  // the query's index (its Philox row)
  int token_sample;
  float tprime;
  uint64_t seed;
  int64_t r_lo, r_hi;
  unsigned long long* tsel;      // the query's ceil(c/32) tagged bitset words
  unsigned long long* tpart;     // this workgroup's five partial words
  unsigned epoch;
  unsigned* err;
  int32_t* out_clusters;         // the query's [p], or null
  int32_t* out_ids;              // the query's [p b], or null
  float* out_logits;
};

// The stage-2 role (all 1024 threads): find the probes of the rows from the
// bitset (a prefix count over its words), score the rows, merge and publish
// the partial.  `gave_up`: this thread already gave up a poll.
template <typename T, int MAXM>
__device__ __forceinline__ void stage2_role(const Stage2Job& a, Batch1Shared& sh, bool gave_up) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  FH_TRACE(4);
  const int64_t r_lo = a.r_lo, r_hi = a.r_hi;
  uint4 hv[1][MAXM];
  load_hslice<T, MAXM>(static_cast<const T*>(a.h), a.d / Chunk<T>::kElems, lane, hv[0]);
  // the probes this workgroup's rows come from: positions [pos0, pos0+npos)
  // of the ascending probe list, read off the selector's bitset
  const int pos0 = (int)(r_lo / a.bsz);
  const int npos = r_hi > r_lo ? (int)((r_hi - 1) / a.bsz) - pos0 + 1 : 0;
  int nkept = a.p;  // probes in the published bitset
  if (npos > 0) {
    const int nw = (a.c + 31) / 32;
    const int t = threadIdx.x;
    // every listed probe starts as a valid cluster: if a bitset word never
    // arrives, the popcounts need not reach p and some positions stay unset
    for (int i = t; i < npos; i += 1024) sh.probes[i] = 0;
    uint32_t word = 0u;
    if (t < nw) {
      unsigned long long* const ptr[1] = {a.tsel + t};
      const bool live[1] = {true};
      uint32_t got[1];
      if (!poll_tagged<1>(ptr, live, a.epoch, a.err, got)) gave_up = true;
      word = got[0];
      // bits past c (a stale or foreign word) name no cluster
      if (t == nw - 1 && (a.c & 31)) word &= (1u << (a.c & 31)) - 1u;
    }
    int tot;
    int pos = block_exclusive_scan(__popc(word), sh.sel.red_scan, &tot);
    nkept = min(tot, a.p);
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
  int64_t r_end = r_hi;
  if (a.tau > 0.f) {
    // adaptive: only the n b rows of the n kept probes; the rest of this
    // workgroup's range, and the probe positions past n it owns, are padding
    const int64_t nr = (int64_t)nkept * a.bsz;
    r_end = min(r_hi, nr);
    for (int64_t r = max(r_lo, nr) + threadIdx.x; r < r_hi; r += 1024) {
      if (a.out_ids) a.out_ids[r] = -1;
      if (a.out_logits) a.out_logits[r] = -INFINITY;
    }
    if (a.out_clusters)
      for (int pos = max(pos0, nkept) + (int)threadIdx.x; pos < pos0 + npos; pos += 1024)
        if ((int64_t)pos * a.bsz >= r_lo) a.out_clusters[pos] = -1;
  }
  LaneParts lp = lane_parts_empty();
  // slot f of the clustering; with the cluster-contiguous copy of E it is
  // also the row, else the row is the token C2T[f]
  auto src_of = [&](int64_t r) -> int64_t {
    const int rr = (int)r;  // p b < 2^31
    const int64_t f = (int64_t)sh.probes[rr / a.bsz - pos0] * a.bsz + rr % a.bsz;
    return a.Ec ? f : (int64_t)a.c2t[f];
  };
  auto tok_of = [&](int64_t src) -> int64_t { return a.Ec ? (int64_t)a.c2t[src] : src; };
  auto sink = [&](int, int64_t r, int64_t src, float z) {
    if (lane == 0) {
      if (a.out_logits) a.out_logits[r] = z;
      if (a.out_ids) a.out_ids[r] = (int32_t)src;
    }
    lane_parts_add(lp, z, (int32_t)src, a.token_sample, a.tprime, a.seed, a.row);
  };
  // four rows in flight per wave when the register slice allows it
  wave_rows<T, MAXM, 1, (MAXM <= 4 ? 4 : 2)>(static_cast<const T*>(a.Ec ? a.Ec : a.E), a.d, lane,
                                             hv, 1, r_lo + wave, r_end, 16, src_of, tok_of, sink);
  FH_TRACE(22);
  const Part part[1] = {lane_parts_finish(lp, a.token_sample, a.tprime, a.seed, a.row)};
  // sh.probes is read above; sh.parts aliases it
  const bool wg_bad = __syncthreads_or(gave_up);
  Part wg = block_merge_parts<16, 1>(part, 1, sh.parts);
  if (wg_bad) wg.id = kBadPart;
  if (threadIdx.x == 0) publish_part(a.tpart, a.epoch, wg);
  FH_TRACE(6);
}

template <typename T, int MAXM, int KP, int QB, int MAXG>
__global__ __launch_bounds__(1024) void k_batch1(FusedArgs a) {
  __shared__ Batch1Shared sh;
  __shared__ unsigned long long s_akey[kSelThreads];  // adaptive: the top p's sort images
  __shared__ float s_aval[kSelThreads];               // and their scores
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
    // (with sampled probes a row's score is parked in lane i mod 64 of the
    // wave's rows and the lanes draw their Gumbel noise together, as in
    // lane_parts_add)
    const bool draw = a.probe_sample && !(a.tau > 0.f);
    float ps = 0.f;
    int64_t pr = -1;
    int np = 0;
    auto publish_parked = [&]() {
      if (lane < np)
        st_tagged(a.tscores + pr, tag(a.epoch, __float_as_uint(saturate_key(
                                          ps / a.temperature + gumbel_at(a.seed, 0u, (uint32_t)pr, 0u)))));
      np = 0;
    };
    auto sink = [&](int, int64_t r, int64_t, float s) {
      if (!draw) {
        if (lane == 0) st_tagged(a.tscores + r, tag(a.epoch, __float_as_uint(saturate_key(s))));
        return;
      }
      if (lane == np) {
        ps = s;
        pr = r;
      }
      if (++np == 64) publish_parked();
    };
    if constexpr (QB != 0) {
      HGroups<MAXG> hg[1];
      load_hgroups<T, MAXG>(hp, a.d / 32, lane, hg[0]);
      wave_rows_q<QB, MAXG, 1>(a.cq, a.csig, a.d, lane, hg, 1, r_lo + wave, r_hi, 16, sink);
    } else {
      uint4 hv[1][MAXM];
      load_hslice<T, MAXM>(hp, a.d / Chunk<T>::kElems, lane, hv[0]);
      auto same = [](int64_t r) { return r; };
      // C is streamed once per call: non-temporal loads
      wave_rows<T, MAXM, 1, 2, kLoadStream>(static_cast<const T*>(a.C), a.d, lane, hv, 1,
                                            r_lo + wave, r_hi, 16, same, same, sink);
    }
    if (draw) publish_parked();
    FH_TRACE(1);
#ifdef FH_PHASE_TRACE
    __syncthreads();
    FH_TRACE(7);  // every wave of this workgroup is done
#endif
    return;
  }

  if (w == a.g1 + a.g2) {  // ---- finisher: the stage-2 partials in a fixed order
    // One wave does it all (block-wide code costs 16 waves' issue slots on
    // the critical path): lane l takes parts l, l + 64, ... in order, the
    // lanes merge as a DPP tree, and lane 0 writes the outputs.  The other
    // waves have nothing to do; no barrier follows.
    if (wave != 0) return;
    bool bad = false;
    const Part r = wave_merge_tagged_parts(a.tparts, a.g2, a.epoch, a.err, &bad);
    FH_TRACE(23);
    const bool anybad = bad;
    if (lane == 0) {
      if (anybad) {
        if (a.out_token) a.out_token[0] = -1;
        if (a.out_logit) a.out_logit[0] = __int_as_float(0x7FC00000);
        if (a.out_lse) a.out_lse[0] = __int_as_float(0x7FC00000);
      } else {
        write_outputs(r, 0, a.out_token, a.out_logit, a.out_lse);
      }
    }
    FH_TRACE(14);
    return;
  }

  const int j = w - a.g1;  // stage-2 workgroup index
  bool gave_up = false;    // a poll of this thread gave up
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
    if (!poll_tagged<KP>(ptr, live, a.epoch, a.err, raw)) gave_up = true;
    FH_TRACE(21);
    const bool adaptive = a.tau > 0.f;
    float x[KP], sraw[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) x[i] = live[i] ? __uint_as_float(raw[i]) : -FLT_MAX;
    MassTotal mt{0.f, 0.f};
    if (adaptive) {  // x holds raw scores: the mass totals, then the keys
      mt = mass_total<KP>(x, a.c, a.temperature, sh.sel.red[2]);
      FH_TRACE(16);
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const int k = (int)threadIdx.x + kSelThreads * i;
        sraw[i] = x[i];
        if (live[i]) x[i] = probe_key(x[i], a.probe_sample, a.temperature, a.seed, 0u, k);
      }
    }
    __syncthreads();
    select_bits<KP>(x, a.c, a.p, a.zq, sh.sel);
    FH_TRACE(17);
    const uint32_t* pub = sh.sel.selbits;
    if (adaptive) {
      // this thread's selected probes: their weight and the top sort image
      uint32_t mine = 0u;
      float wsel = 0.f, best_s = 0.f;
      unsigned long long best = 0ull;
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const int k = (int)threadIdx.x + kSelThreads * i;
        if (live[i] && (sh.sel.selbits[k >> 5] >> (k & 31)) & 1u) {
          mine |= 1u << i;
          wsel += __expf(sraw[i] / a.temperature - mt.M);
          const unsigned long long img = probe_sort_key(x[i], k);
          if (img > best) {
            best = img;
            best_s = sraw[i];
          }
        }
      }
      unsigned long long top = 0ull;
      int n = adaptive_fast(wsel, best, best_s, a.p, a.pmin, a.tau, mt, a.temperature,
                            sh.sel.red[2], s_akey, &top);
      if (n == 1) {  // the top probe alone
        for (int t = threadIdx.x; t < (a.c + 31) / 32; t += kSelThreads) sh.sel.tiebits[t] = 0u;
        __syncthreads();
        if (threadIdx.x == 0) {
          const int id = (int)(0xFFFFFFFFu - (uint32_t)(top & 0xFFFFFFFFull));
          sh.sel.tiebits[id >> 5] = 1u << (id & 31);
        }
        __syncthreads();
        pub = sh.sel.tiebits;
      } else if (n == 0) {
        // the general case: file the top p's sort images and scores at slots
        // from a prefix count, sort them, scan the weights in key order
        const int P2 = pow2_at_least(a.p);
        int filed;
        int slot = block_exclusive_scan(__popc(mine), sh.sel.red_out, &filed);
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          if ((mine >> i) & 1u) {
            if (slot < a.p) {  // the selection flags exactly p
              s_akey[slot] = probe_sort_key(x[i], (int)threadIdx.x + kSelThreads * i);
              s_aval[slot] = sraw[i];
            }
            ++slot;
          }
        }
        __syncthreads();
        unsigned long long skey = 0ull;  // padding sorts below every real key
        float sval = 0.f;
        if ((int)threadIdx.x < a.p) {
          skey = s_akey[threadIdx.x];
          sval = s_aval[threadIdx.x];
        }
        FH_TRACE(20);
        bitonic_sort_desc(skey, sval, P2, s_akey, s_aval);
        FH_TRACE(18);
        int id;
        n = adaptive_count(skey, sval, a.p, a.pmin, a.tau, mt, a.temperature, sh.sel.red[2],
                           sh.sel.red_scan, &id);
        // the kept set, in the (free) tie bitset
        for (int t = threadIdx.x; t < (a.c + 31) / 32; t += kSelThreads) sh.sel.tiebits[t] = 0u;
        __syncthreads();
        if ((int)threadIdx.x < n) atomicOr(&sh.sel.tiebits[id >> 5], 1u << (id & 31));
        __syncthreads();
        pub = sh.sel.tiebits;
      }
      // n == p: all selected probes, the selection's own bitset
      FH_TRACE(19);
      if (threadIdx.x == 0 && a.out_nprobe) a.out_nprobe[0] = n;
    }
    // publish the chosen clusters as a bitset, one tagged word per 32
    for (int t = threadIdx.x; t < (a.c + 31) / 32; t += kSelThreads)
      st_tagged(a.tsel + t, tag(a.epoch, pub[t]));
    FH_TRACE(3);
    __syncthreads();  // sh.sel is reused below
  }

  // ---- stage 2
  Stage2Job s2{};
  s2.E = a.E; s2.Ec = a.Ec; s2.c2t = a.c2t;
  s2.c = a.c; s2.bsz = a.bsz; s2.d = a.d; s2.p = a.p; s2.tau = a.tau;
  s2.h = a.h; s2.row = 0u;
  s2.token_sample = a.token_sample; s2.tprime = a.tprime; s2.seed = a.seed;
  s2.r_lo = (int64_t)j * a.rows2;
  s2.r_hi = min((int64_t)a.p * a.bsz, s2.r_lo + a.rows2);
  s2.tsel = a.tsel; s2.tpart = a.tparts + 5 * (int64_t)j;
  s2.epoch = a.epoch; s2.err = a.err;
  s2.out_clusters = a.out_clusters; s2.out_ids = a.out_ids; s2.out_logits = a.out_logits;
  stage2_role<T, MAXM>(s2, sh, gave_up);
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
  a.tau = f.tau; a.pmin = f.pmin; a.out_nprobe = f.out_nprobe;
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

#if FH_BATCH1_QB == 0
namespace fh {

// ======================================================================
// Batched calls after stage 1, in one launch (2 <= B <= 16 queries; stage 1
// ran as its own launch and stored each query's selection keys).  Roles by
// workgroup index, in dispatch order:
//   [0, B)           selector q: reads query q's keys, selects its p probes
//                    and publishes them as a tagged bitset;
//   [B, B + B G2q)   stage 2: query q = (w - B) / G2q, rows of its p b
//                    retrieved rows (stage2_role, as in the batch-1 kernel);
//   B + B G2q        finisher: wave q merges query q's G2q partials.
// Every workgroup waits only for lower-indexed ones (see fh_handover.hpp),
// so each query's stage 2 starts as soon as its own selector is done.
// ======================================================================
struct BatchedArgs {
  const void* E;
  const void* Ec;
  const int32_t* c2t;
  int c, bsz, d;
  const void* H;       // [B x d]
  int B;
  const float* keys;   // [B x c] stage 1's selection keys
  int p;
  float zq;
  int token_sample;
  float tprime;
  uint64_t seed;
  int g2, rows2;       // stage-2 workgroups per query and rows per workgroup
  unsigned epoch;
  unsigned long long* tsel;    // [B x ceil(c/32)]
  unsigned long long* tparts;  // [B x g2 x 5]
  int32_t* out_clusters;       // [B x p] or null
  int32_t* out_ids;            // [B x p b] or null
  float* out_logits;
  int32_t* out_token;
  float* out_logit;
  float* out_lse;
  unsigned* err;
};

template <typename T, int MAXM, int KP>
__global__ __launch_bounds__(1024) void k_batched(BatchedArgs a) {
  __shared__ Batch1Shared sh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int w = blockIdx.x;
  const int W = (a.c + 31) / 32;
  if (w < a.B) {  // ---- selector of query w (the keys as k_select takes them)
    FH_TRACE(16);
    const float* kq = a.keys + (int64_t)w * a.c;
    select_clear(sh.sel);
    float x[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int k = (int)threadIdx.x + kSelThreads * i;
      x[i] = k < a.c ? saturate_key(kq[k]) : -FLT_MAX;
    }
    __syncthreads();
    select_bits<KP>(x, a.c, a.p, a.zq, sh.sel);
    FH_TRACE(17);
    for (int t = threadIdx.x; t < W; t += kSelThreads)
      st_tagged(a.tsel + (int64_t)w * W + t, tag(a.epoch, sh.sel.selbits[t]));
    FH_TRACE(3);
    return;
  }
  if (w == a.B + a.B * a.g2) {  // ---- finisher: wave q merges query q's partials
    if (wave >= a.B) return;
    bool bad = false;
    const Part r = wave_merge_tagged_parts(a.tparts + 5 * (int64_t)wave * a.g2, a.g2, a.epoch,
                                           a.err, &bad);
    FH_TRACE(23);
    if (lane == 0) {
      if (bad) {
        if (a.out_token) a.out_token[wave] = -1;
        if (a.out_logit) a.out_logit[wave] = __int_as_float(0x7FC00000);
        if (a.out_lse) a.out_lse[wave] = __int_as_float(0x7FC00000);
      } else {
        write_outputs(r, wave, a.out_token, a.out_logit, a.out_lse);
      }
    }
    return;
  }
  // ---- stage 2
  const int j = w - a.B;
  const int q = j / a.g2, jj = j - q * a.g2;
  const int64_t nb = (int64_t)a.p * a.bsz;
  Stage2Job s2{};
  s2.E = a.E; s2.Ec = a.Ec; s2.c2t = a.c2t;
  s2.c = a.c; s2.bsz = a.bsz; s2.d = a.d; s2.p = a.p; s2.tau = 0.f;
  s2.h = static_cast<const T*>(a.H) + (int64_t)q * a.d;
  s2.row = (uint32_t)q;
  s2.token_sample = a.token_sample; s2.tprime = a.tprime; s2.seed = a.seed;
  s2.r_lo = (int64_t)jj * a.rows2;
  s2.r_hi = min(nb, s2.r_lo + a.rows2);
  s2.tsel = a.tsel + (int64_t)q * W;
  s2.tpart = a.tparts + 5 * ((int64_t)q * a.g2 + jj);
  s2.epoch = a.epoch; s2.err = a.err;
  s2.out_clusters = a.out_clusters ? a.out_clusters + (int64_t)q * a.p : nullptr;
  s2.out_ids = a.out_ids ? a.out_ids + (int64_t)q * nb : nullptr;
  s2.out_logits = a.out_logits ? a.out_logits + (int64_t)q * nb : nullptr;
  stage2_role<T, MAXM>(s2, sh, false);
}

static BatchedArgs batched_args(const BatchedLaunch& f) {
  const KernelCtx& k = *f.ctx;
  BatchedArgs a{};
  a.E = k.E; a.Ec = k.Ec; a.c2t = k.c2t;
  a.c = (int)k.c; a.bsz = (int)k.b; a.d = k.d;
  a.H = f.H; a.B = f.B; a.keys = f.keys; a.p = f.p;
  a.zq = select_quantile(k.c, f.p);
  a.token_sample = f.token_sample; a.tprime = f.tprime; a.seed = f.seed;
  a.g2 = batched_stage2_blocks(f.p, k.b, f.B, f.cus);
  a.rows2 = (int)batched_rows2(f.p, k.b, f.B, f.cus);
  a.epoch = f.epoch;
  a.tsel = f.tagged;
  a.tparts = f.tagged + batched_off_parts(k.c, f.B);
  a.out_clusters = f.out_clusters; a.out_ids = f.out_ids; a.out_logits = f.out_logits;
  a.out_token = f.out_token; a.out_logit = f.out_logit; a.out_lse = f.out_lse;
  a.err = f.err;
  return a;
}

template <typename T, int MAXM, int KP>
static hipError_t bt_go(const BatchedLaunch& f, const BatchedArgs& a) {
  const unsigned grid = (unsigned)(a.B + a.B * a.g2 + 1);
  hipLaunchKernelGGL((k_batched<T, MAXM, KP>), dim3(grid), dim3(1024), 0, f.ctx->stream, a);
  return hipGetLastError();
}

template <typename T, int KP>
static hipError_t bt_m(const BatchedLaunch& f, const BatchedArgs& a) {
  switch ((f.ctx->d / Chunk<T>::kElems + 63) / 64) {
    case 1: return bt_go<T, 1, KP>(f, a);
    case 2: return bt_go<T, 2, KP>(f, a);
    case 3: case 4: return bt_go<T, 4, KP>(f, a);
    case 5: case 6: return bt_go<T, 6, KP>(f, a);
    case 7: case 8: return bt_go<T, 8, KP>(f, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t FH_BATCHED_ENTRY(const BatchedLaunch& f) {
  if (!batched_fits(f.p, f.ctx->b, f.B, f.cus)) return hipErrorInvalidValue;
  const BatchedArgs a = batched_args(f);
  switch (sel_keys_per_thread(f.ctx->c)) {
    case 1: return bt_m<FH_BATCH1_T, 1>(f, a);
    case 2: return bt_m<FH_BATCH1_T, 2>(f, a);
    case 8: return bt_m<FH_BATCH1_T, 8>(f, a);
    case 16: return bt_m<FH_BATCH1_T, 16>(f, a);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace fh
#endif  // FH_BATCH1_QB == 0

#ifdef FH_PHASE_TRACE
// Trace builds only: copy this variant's phase timestamps to the host.
#define FH_B1_CAT2(a, b) a##b
#define FH_B1_CAT(a, b) FH_B1_CAT2(a, b)
extern "C" int FH_B1_CAT(FH_BATCH1_ENTRY, _trace_read)(void* dst, size_t bytes) {
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(fh::g_fh_trace), bytes) == hipSuccess ? 0 : -1;
}
#endif
