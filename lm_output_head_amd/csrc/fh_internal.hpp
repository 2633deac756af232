// Internal interface between the C-ABI engine and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fh_batch1_sizing.hpp"

namespace fh {

// A partial epilogue result over a set of candidate tokens: the best
// (key, id) pair with the logit z of that token, and (m, s) with
// m = max x, s = sum exp(x - m) over x = z / T'.
struct Part {
  float key;
  float z;
  float m;
  float s;
  int32_t id;
};

// Rows per wave of each row-GEMV launch.
constexpr int kScoreRPW = 2;
constexpr int kGatherRPW = 2;
constexpr int kDenseRPW = 4;
constexpr int kInt4RPW = 2;

// What every launcher needs to know about the engine and the call.
struct KernelCtx {
  bool bf16;
  const void* E;
  const void* Ec;  // cluster-contiguous copy of E (Ec[f] = E[C2T[f]]), or null
  const void* Ecm = nullptr;  // its fragment-order copy (cluster-major stage 2), or null
  const void* Cm = nullptr;   // the centroids' fragment-order copy (batched bf16 stage 1), or null
  const void* C;
  const int32_t* c2t;
  const uint8_t* cq;
  const uint16_t* csig;
  const uint8_t* cq_mfma;    // INT4 codes re-laid for the MFMA tiles, or null
  const uint16_t* sig_mfma;  // INT4 / INT8 scales group-major [G x mfma_sig_ld(c)], or null
  int64_t v, c, b;
  int d;
  hipStream_t stream;
  int qbits = 0;  // stage-1 codes: 0 (C as stored), 4 (INT4 g32) or 8 (INT8 g32)
};

int64_t rows_blocks(int64_t nrows, int rpw);

// What a stage-1 launch stores: the score s, or with sampled probes the
// selection key s / T + G(seed, q, k, 0) of query q and cluster k (k_select
// then takes the keys as they are).  Computing the keys in the stage-1
// epilogue spreads the Gumbel draws over the whole grid instead of one
// workgroup per query.
struct KeyXform {
  int sample = 0;
  float temperature = 1.f;
  uint64_t seed = 0;
};

// g32 quantisation of C into cq / csig (k.qbits = 4 or 8)
hipError_t launch_quant(const KernelCtx& k, int* bad);
hipError_t launch_permute_rows(const KernelCtx& k, void* out);
hipError_t launch_score(const KernelCtx& k, const void* h, int B, float* out,
                        const KeyXform& kx = KeyXform{});
// stage-1 scores from the g32 codes (k.qbits = 4 or 8), on the vector units
hipError_t launch_score_quant(const KernelCtx& k, const void* h, int B, float* out,
                              const KeyXform& kx = KeyXform{});
float select_quantile(int64_t c, int64_t p);
// S [B x ldS]: the p probes of each query, ascending.  With mbits/mpre non-
// null also the probe bitsets word-major, mbits[w * B + q], and the probes of
// q in words before w, mpre[w * B + q] (W = ceil(c/32) words).
hipError_t launch_select(const KernelCtx& k, const float* scores, int B, int p, int sample,
                         float temperature, uint64_t seed, int32_t* S, int ldS,
                         uint32_t* mbits = nullptr, int32_t* mpre = nullptr);
// Stage 2 over the probe lists S [B x ldS] (ldS < 0: p).  With nprobe non-null
// query q scores only its first nprobe[q] probes (the adaptive count).
hipError_t launch_gather(const KernelCtx& k, const void* h, int B, const int32_t* S, int p,
                         int token_sample, float tprime, uint64_t seed, int32_t* out_ids,
                         float* out_logits, Part* parts, int64_t* nparts,
                         int ldS = -1, const int32_t* nprobe = nullptr);
// Adaptive probe count: per query, of the pmax probes in S [B x pmax]
// (ascending, from launch_select over raw scores with the same sample,
// temperature and seed), keep the first n in key order whose softmax(s/T)
// mass reaches tau of all c clusters, n clamped to [pmin, pmax] (pmax <= 1024).
// Rewrites S (n ascending, then -1), writes nprobe [B], and pads the retrieved
// outputs [B x pmax b] (if non-null) past n b with id -1 and logit -inf.
// With mbits/mpre non-null also the kept probes' bitsets and earlier-word
// counts, word-major [ceil(c/32) x B], for launch_gather_cm.
hipError_t launch_adapt(const KernelCtx& k, const float* scores, int B, int pmax, int pmin,
                        float tau, int sample, float temperature, uint64_t seed, int32_t* S,
                        int32_t* nprobe, int32_t* out_ids, float* out_logits,
                        uint32_t* mbits = nullptr, int32_t* mpre = nullptr);
// batch-shared probes: summed scores, and one probe list broadcast to every row
hipError_t launch_sum_rows(const KernelCtx& k, const float* scores, int B, float* out);
hipError_t launch_broadcast_row(const KernelCtx& k, const int32_t* src, int n, int B,
                                int32_t* dst);
hipError_t launch_dense(const KernelCtx& k, const void* h, int B, int token_sample, float tprime,
                        uint64_t seed, float* out_logits, Part* parts, int64_t* nparts);
// Matrix-core (MFMA) paths for batches of bf16 queries.
constexpr int kMfmaMinBatchBf16 = 8;  // bf16 stage 1
constexpr int kMfmaMinBatchDense = 2;  // the dense head and the speculative verification (bf16)
constexpr int kMfmaMinBatchInt4 = 2;  // INT4 stage 1
constexpr int kMfmaMinBatchInt8 = 2;  // INT8 stage 1 (split over d at small B: 13.7 us at B = 16)
int64_t mfma_int4_row_bytes(int d);
int64_t mfma_blocks(int64_t R);    // row blocks (partials per query) of the MFMA dense head
int64_t splitd_blocks(int64_t R);  // the same for the dense pass split over d (16 rows each)
int64_t mfma_sig_ld(int64_t c);
hipError_t launch_mfma_relayout(const KernelCtx& k, uint8_t* cq_mfma, uint16_t* sigT);
hipError_t launch_score_mfma(const KernelCtx& k, int cus, const void* h, int B, float* out,
                             const KeyXform& kx = KeyXform{});
// Cluster-major stage 2 on the matrix cores (bf16 engines, B >= 2): every
// probed cluster's rows are read once for all queries that probe it.
bool gather_cm_fits(int B, int64_t p, int64_t c);
// Fragment-order copies (layout in fh_mfma.hip) of c clusters of b
// contiguous bf16 rows of d elements: the cluster-contiguous E (read by the
// cluster-major stage 2 and the dense passes) and the centroids (c = 1,
// b = their count; read by batched stage 1).  Their bytes, and the launch
// that writes one.
int64_t fragment_order_bytes(int64_t c, int64_t b, int d);
hipError_t launch_fragment_order(const void* rows, int64_t c, int64_t b, int d, void* out,
                                 hipStream_t st);
int gather_cm_max_batch();  // queries the cluster-major stage 2 can take
// stage 2 over one probe list shared by the batch, as the matrix-core GEMM
// with a row map (bf16 engines with the cluster-contiguous E)
hipError_t launch_gather_shared_mfma(const KernelCtx& k, int cus, const void* h, int B,
                                     const int32_t* S, int p, int token_sample, float tprime,
                                     uint64_t seed, int32_t* out_ids, float* out_logits,
                                     Part* parts, int64_t* nparts);
// Partials [B x p nrt], nrt = ceil(b / 16) row tiles per cluster: query q's
// partial over row tile t of its probe of rank r (ascending cluster id) at
// parts[(q p + r) nrt + t]; *nparts = p nrt.  A query with fewer than p
// probes in its bitset (the adaptive count n) leaves the partials past
// n nrt unwritten: launch_finish then takes n (scaled by nrt) as its limit.
hipError_t launch_gather_cm(const KernelCtx& k, int cus, const void* h, int B, int p,
                            const uint32_t* mbits,
                            const int32_t* mpre, int token_sample, float tprime, uint64_t seed,
                            int32_t* out_ids, float* out_logits, Part* parts, int64_t* nparts);
hipError_t launch_dense_mfma(const KernelCtx& k, int cus, const void* h, int B, int token_sample,
                             float tprime, uint64_t seed, float* out_logits, Part* parts,
                             int64_t* nparts);

// fp8 E4M3 probabilities of [B x n] logits, exp(z / T' - lse[q]) scaled by
// 2^out_k[q] (fh_probs.hip).
hipError_t launch_probs_fp8(const float* logits, const float* lse, int64_t B, int64_t n,
                            float temperature, uint8_t* out, int32_t* out_k, hipStream_t stream);

// Merge each query's partials parts[q nparts, q nparts + n_q) in order, n_q
// = nparts, or min(nparts, nlimit[q] scale) with nlimit (device, [B]) non-null.
hipError_t launch_finish(const KernelCtx& k, const Part* parts, int B, int64_t nparts,
                         int32_t* out_token, float* out_logit, float* out_lse,
                         const int32_t* nlimit = nullptr, int scale = 1);

// The single-launch batch-1 path (stage 1, selection, stage 2 and the
// finish by workgroups in dispatch order, handed over through tagged words).
struct FusedLaunch {
  const KernelCtx* ctx;
  int cus;                        // compute units of the device
  const void* h;
  int p;
  int probe_sample, token_sample;
  float temperature, tprime;
  uint64_t seed;
  unsigned epoch;                 // this call's tag, never 0
  unsigned long long* tscores;    // [c] tagged scores (zeroed at create)
  unsigned long long* tsel;       // [ceil(c/32)] tagged probe bitset (zeroed at create)
  unsigned long long* tparts;     // [5 x batch1_slots2(cus)] (zeroed at create)
  float tau = 0.f;                // adaptive probe count: mass to reach, or 0 (fixed p)
  int pmin = 1;                   // adaptive: the smallest count (p is the largest)
  int32_t* out_nprobe = nullptr;  // adaptive: [1] or null
  int32_t* out_clusters;          // [p] or null
  int32_t* out_ids;
  float* out_logits;
  int32_t* out_token;
  float* out_logit;
  float* out_lse;
  unsigned* err;                  // sticky flag: a bounded poll gave up
};
// The offline balanced spherical k-means (fh_cluster.hip).
struct ClusterTimes {
  float init_ms;  // normalisation and k-means++
  float sims_ms;  // similarity GEMMs, all iterations
  float total_ms;
  float pp_step_us;  // average k-means++ distance-refresh kernel, sampled launches
  int rounds;     // balanced-assignment rounds, all iterations
};
hipError_t balanced_assign_device(const float* S, int64_t v, int64_t c, int32_t* asg,
                                  hipStream_t st, int* rounds);
hipError_t kmeans_device(const void* E, bool bf16, int64_t v, int d, int64_t c, int iters,
                         const double* u, float* C, int32_t* c2t, int32_t* init, int32_t* asg_out,
                         hipStream_t st, ClusterTimes* times);

// Speculative verification (fh_spec.hip): the token -> cluster map, and the
// verification of B draft tokens against the dense head.
hipError_t launch_t2c(const KernelCtx& k, int32_t* t2c);
// the dense pass of the verification on the matrix cores (bf16, B >= kMfmaMinBatchDense)
hipError_t launch_spec_mfma(const KernelCtx& k, int cus, const void* h, int B, float T,
                            uint64_t seed, const int32_t* t2c, const uint32_t* bits, int W,
                            Part* parts, int64_t* nparts);
hipError_t launch_spec_verify(const KernelCtx& k, int cus, const int32_t* t2c, uint32_t* bits, Part* parts,
                              const void* h, int B, int p, const int32_t* draft_clusters,
                              const int32_t* draft_token, const float* draft_lse, float T,
                              uint64_t seed, int32_t* out_token, int32_t* out_accepted,
                              float* out_lse);

hipError_t launch_batch1(const FusedLaunch& f);

// Batched calls (2 <= B <= kBatchedMaxB) after stage 1: selection, stage 2
// and the finish in one launch, handed over through tagged words
// (fh_batch1.inl, sizing in fh_batch1_sizing.hpp).
struct BatchedLaunch {
  const KernelCtx* ctx;
  int cus;
  const void* H;                  // [B x d] queries
  int B;
  const float* keys;              // [B x c] stage 1's selection keys
  int p;
  int token_sample;
  float tprime;
  uint64_t seed;
  unsigned epoch;                 // this call's tag, never 0
  unsigned long long* tagged;     // batched_tag_words(c, max_batch, cus) words (zeroed at create)
  int32_t* out_clusters;          // [B x p] or null
  int32_t* out_ids;               // [B x p b] or null
  float* out_logits;
  int32_t* out_token;
  float* out_logit;
  float* out_lse;
  unsigned* err;                  // sticky flag: a bounded poll gave up
};
hipError_t launch_batched(const BatchedLaunch& f);
hipError_t launch_batched_bf16(const BatchedLaunch& f);
hipError_t launch_batched_f32(const BatchedLaunch& f);
// per storage variant, one translation unit each
hipError_t launch_batch1_bf16(const FusedLaunch& f);
hipError_t launch_batch1_bf16_int4(const FusedLaunch& f);
hipError_t launch_batch1_f32(const FusedLaunch& f);
hipError_t launch_batch1_f32_int4(const FusedLaunch& f);
hipError_t launch_batch1_bf16_int8(const FusedLaunch& f);
hipError_t launch_batch1_f32_int8(const FusedLaunch& f);

}  // namespace fh
