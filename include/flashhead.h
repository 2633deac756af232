/*
 * flashhead.h — C ABI of libflashhead, an MI355X (gfx950) implementation of
 * FlashHead inference: a drop-in replacement for a language model's dense
 * output head z = E h by two-stage retrieval over a balanced clustering of
 * E's rows.
 *
 * Sources, cited by page title and section:
 *   [X]  FlashHead technical explainer (framerc.cn), §1.1 dense head cost,
 *        §1.2.1 balanced clustering and the dense C2T table, §1.2.2 multi-probe
 *        top-p retrieval, §1.2.3 multinomial probe sampling with temperature,
 *        §1.2.4 selective (INT4 stage-1) quantisation, §2.2.2 the computation
 *        graph h -> centroid scores -> top-p clusters -> token scores,
 *        §2.3 the quantisation config (centroid int4, token bf16).
 *   [A]  "FlashHead: Efficient Drop-In Replacement for the Classification Head
 *        in Language Model Inference" (arXiv 2603.14591), abstract,
 *        innovations (1)-(4).
 *
 * Conventions for every entry point:
 *   - Tensors are dense and row-major.  "Device" pointers address GPU memory
 *     on the engine's device; "host" pointers address CPU memory.
 *   - Work is enqueued on the HIP stream passed as `stream` (NULL = the
 *     default stream) and the call returns without waiting for it, except
 *     fh_create, which waits for its own set-up work.  Outputs are valid once
 *     that stream has reached the call.
 *   - Argument errors are detected before anything is enqueued: the call
 *     returns FH_EINVAL or FH_EUNSUPPORTED, writes nothing, and
 *     fh_last_error() describes the problem.  A failing HIP call returns
 *     FH_EHIP; allocation failure returns FH_ENOMEM.
 *   - Results are deterministic: the same inputs, p, mode, temperature and
 *     seed give bit-identical outputs on the same device.
 *   - One engine may be used from several threads only if the calls do not
 *     overlap: calls share the engine's workspace.
 */
#ifndef FLASHHEAD_H
#define FLASHHEAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fh_engine fh_engine; /* opaque */

typedef enum {
  FH_OK = 0,
  FH_EINVAL = -1,       /* invalid argument                                 */
  FH_ENOMEM = -2,       /* device or host allocation failed                 */
  FH_EHIP = -3,         /* a HIP runtime call or kernel launch failed       */
  FH_EUNSUPPORTED = -4  /* valid, but outside what this library implements  */
} fh_status;

/* Storage type shared by E, C and h. */
typedef enum { FH_F32 = 0, FH_BF16 = 1 } fh_dtype;

/* Stage-1 centroid storage ([X] §1.2.4, §2.3; the W4A16 and W8A16 rows of
 * the tuning table, [X] §5.2).  Both integer forms are symmetric with one
 * fp16 scale per 32 consecutive elements of a centroid row:
 * sigma = fp16_rne(amax / qmax) (fp32 division), q = clamp(rint(x / sigma),
 * -qmax, qmax) with ties to even, q = 0 where sigma = 0; the score is
 * sum_g sigma_g sum_{i in g} q_i h_i.  Queries and token embeddings stay in
 * the engine's dtype. */
typedef enum {
  FH_QUANT_NONE = 0,      /* centroids used as given                         */
  FH_QUANT_INT4_G32 = 1,  /* qmax 7, two's-complement nibbles                */
  FH_QUANT_INT8_G32 = 2   /* qmax 127, int8                                  */
} fh_quant;

/* `mode` is the OR of one probe flag and one token flag. */
enum {
  FH_PROBE_TOPK = 0,   /* the p highest-scoring clusters ([X] §1.2.2)       */
  FH_PROBE_SAMPLE = 1, /* p distinct clusters drawn from softmax(s/T)
                          without replacement ([X] §1.2.3)                  */
  FH_TOKEN_ARGMAX = 0, /* highest logit among retrieved tokens              */
  FH_TOKEN_SAMPLE = 2, /* one draw from softmax(z/T) over retrieved tokens  */
  FH_PROBE_SHARED = 4  /* one probe set for the whole batch: the p clusters
                          with the largest summed score sum_b s[b, k]
                          (ties to the smaller id) -- [X] §4.2's shared
                          selection across samples, read this way; changes
                          results for B > 1, equals FH_PROBE_TOPK at B = 1;
                          not combinable with FH_PROBE_SAMPLE               */
};

/*
 * fh_create — build an engine over one output head.
 *
 *   E        device, [v x d] of `dtype`: output embeddings, one row per token
 *            ([X] §1.1).  BORROWED: not copied; keep it alive and unchanged
 *            until fh_destroy.
 *   C        device, [c x d] of `dtype`: cluster centroids ([X] §1.2.1).
 *            Borrowed for FH_QUANT_NONE.  For FH_QUANT_INT4_G32 and
 *            FH_QUANT_INT8_G32 it is read once here and may be freed after
 *            the call returns.
 *   C2T      HOST, [c x b] int32 with b = v / c: C2T[k*b + j] is the token in
 *            slot j of cluster k ([X] §1.2.1, [A] (1)).  Copied.  Must hold
 *            every token of [0, v) exactly once (balanced clustering).
 *   v, d, c  vocabulary size, hidden size, cluster count; v % c == 0.
 *            d % 4 == 0 for FH_F32, d % 8 == 0 for FH_BF16, and
 *            d % 32 == 0 with a quantised stage 1.  c <= 16384; d <= 4096
 *            for FH_BF16, d <= 2048 for FH_F32 (else FH_EUNSUPPORTED).
 *   quant    FH_QUANT_INT4_G32 / FH_QUANT_INT8_G32 quantise C here (the
 *            scheme above, qmax 7 or 127).  A scale that overflows fp16
 *            gives FH_EINVAL.
 *   max_batch largest B any later call will use (sizes the workspace).
 *            Besides the workspace, the engine keeps a cluster-contiguous
 *            copy of E (v x d of `dtype`, row f = E[C2T[f]]) so that each
 *            probe's b rows are read as one block ([X] §1.2.1); FH_ENOMEM if
 *            it does not fit.
 *   stream   stream for the set-up work; fh_create waits for it.
 *   out      receives the engine (set only on FH_OK).
 */
fh_status fh_create(const void* E, const void* C, const int32_t* C2T, fh_dtype dtype,
                    int64_t v, int64_t d, int64_t c, fh_quant quant, int64_t max_batch,
                    void* stream, fh_engine** out);

/* fh_destroy — release everything the engine owns (NULL is a no-op).  Waits
 * for the device to finish work that may still use it. */
void fh_destroy(fh_engine* e);

/*
 * fh_forward — one FlashHead call over B hidden states ([X] §2.2.2).
 *
 *   h        device, [B x d] of the engine's dtype.
 *   B        1 <= B <= max_batch.
 *   p        probes per query, 1 <= p <= c ([X] §1.2.2).
 *   mode     FH_PROBE_* | FH_TOKEN_*.
 *   temperature  > 0 when either stage samples ([X] §1.2.3); otherwise
 *            ignored.  One temperature serves both stages.
 *   seed     keys the Philox4x32-10 stream of every draw: probe k of row b
 *            uses counter (k/4, b, 0, 0), token t uses (t/4, b, 1, 0), key
 *            (seed mod 2^32, seed >> 32), word k mod 4 (resp. t mod 4),
 *            u = ((w >> 9) + 1/2) 2^-23, Gumbel noise -ln(-ln u).
 *
 * Outputs (device; any of the last four may be NULL to skip it):
 *   out_token        [B] int32: the chosen token id.
 *   out_token_logit  [B] float: its logit z = E[token] . h.
 *   out_lse          [B] float: log sum exp(z / T') over the retrieved
 *                    tokens, T' = temperature if tokens are sampled, else 1.
 *   out_clusters     [B x p] int32: the probed clusters, ascending id.
 *   out_ids          [B x p*b] int32: retrieved token ids, in cluster order
 *                    (ascending id) then slot order.
 *   out_logits       [B x p*b] float: their logits z = E[t] . h (float32
 *                    accumulation of the stored values).
 * Selection keys are compared in float32; equal keys go to the smaller
 * cluster / token id.
 */
fh_status fh_forward(fh_engine* e, const void* h, int64_t B, int64_t p, int mode,
                     float temperature, uint64_t seed, int32_t* out_token,
                     float* out_token_logit, float* out_lse, int32_t* out_clusters,
                     int32_t* out_ids, float* out_logits, void* stream);

/*
 * fh_forward_adaptive — fh_forward with a probe count per query ([X] §1.2.2:
 * the number of probes adapts to the distribution of h; §4.2: fewer probes
 * for confident queries, such as frequent tokens).  The pages give no
 * formula; this library's reading: the clusters are taken in the order of the
 * selection keys (by score, or with FH_PROBE_SAMPLE the draws without
 * replacement from softmax(s/T)), and query b stops at the first count n whose
 * clusters hold at least tau of softmax(s/T) over all c clusters; n is then
 * clamped to [p_min, p_max].  The mass is accumulated in float32.
 *   p_min, p_max  1 <= p_min <= p_max <= min(c, 1024).
 *   tau           in (0, 1].
 *   mode          FH_PROBE_TOPK or FH_PROBE_SAMPLE | FH_TOKEN_*; not
 *                 FH_PROBE_SHARED (FH_EINVAL).  temperature > 0 always (it
 *                 sets the mass even for greedy calls).
 *   out_nprobe    device [B] int32: n per query, or NULL.
 *   out_clusters  device [B x p_max] int32 or NULL: the n probes ascending,
 *                 then -1.
 *   out_ids, out_logits  device [B x p_max b] or NULL: the n b retrieved
 *                 tokens (cluster ascending, slot order), then id -1 and
 *                 logit -inf.
 *   out_token, out_token_logit, out_lse: as for fh_forward, over the n b
 *                 retrieved tokens.
 * B = 1 runs the single launch of fh_forward (its selector takes the count
 * and publishes only the kept probes); larger batches, stream capture and
 * FH_PATH_MULTI run per-stage launches (stage 1, selection of p_max, the
 * count, stage 2 over the kept probes, finish).  Stream-ordered, no host
 * synchronisation.
 */
fh_status fh_forward_adaptive(fh_engine* e, const void* h, int64_t B, int64_t p_max,
                              int64_t p_min, float tau, int mode, float temperature,
                              uint64_t seed, int32_t* out_nprobe, int32_t* out_token,
                              float* out_token_logit, float* out_lse, int32_t* out_clusters,
                              int32_t* out_ids, float* out_logits, void* stream);

/*
 * fh_probs_fp8 — the candidates' probabilities in fp8 ([X] §2.3: the
 * quantisation config keeps the probability intermediate as fp8).  Per row
 * q, p = exp(logits[q*n + i] / T' - lse[q]) (a -inf logit, an empty adaptive
 * slot, gives 0).  The pages do not say how the fp8 tensor is scaled; here a
 * power of two per row: k = 8 - e for the row's largest p = f 2^e, f in
 * [1/2, 1), which puts it in [128, 256) (no saturation, exact scaling, 17
 * binades below it).  out_probs[q*n + i] = E4M3(p 2^k), the OCP E4M3 byte
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7F
 * NaN) rounded to nearest even; out_scale_exp[q] = k, so p = value(byte)
 * 2^-k.  Engine-free; stream-ordered.
 *   logits     device [B x n] float, e.g. fh_forward's out_logits (n = p b)
 *              or fh_forward_adaptive's (n = p_max b).
 *   lse        device [B] float: each row's log-sum-exp taken at T'
 *              (fh_forward's out_lse).
 *   temperature  T' > 0, the temperature of that LSE: the call's temperature
 *              when tokens were sampled, else 1.
 *   out_probs  device [B x n] uint8; out_scale_exp device [B] int32.
 * FH_EINVAL for NULL pointers, B outside [1, 65535], n outside [1, 2^31] or
 * a temperature that is not finite and > 0.
 */
fh_status fh_probs_fp8(const float* logits, const float* lse, int64_t B, int64_t n,
                       float temperature, uint8_t* out_probs, int32_t* out_scale_exp,
                       void* stream);

/*
 * fh_forward_noalloc — fh_forward without an engine and without allocating:
 * for callers that cannot call hipMalloc (code under HIP graph capture,
 * tight serving loops, harnesses that forbid it).  It runs the per-stage
 * launches (stage-1 scores, selection, stage 2, finish) on caller-owned
 * tables and keeps its workspace (scores, probe lists, stage-2 partials) in
 * a fixed 8 MiB device array of the library, one per GPU, held until the
 * process ends; it calls no hipMalloc, hipFree or allocating routine.
 *
 *   E, C     device [v x d] and [c x d] of dtype, 16-byte aligned (as for
 *            fh_create; C as stored, no quantisation).
 *   c2t      device int32 [c x b], b = v / c: a permutation of [0, v) (the
 *            caller's responsibility; fh_create checks it, this does not).
 *   h        device [B x d] of dtype, 16-byte aligned; 1 <= B <= 65535.
 *   p, mode, temperature, seed, outputs: as for fh_forward, except that
 *            FH_PROBE_SHARED is not offered (FH_EUNSUPPORTED).
 * Results equal fh_forward's per-stage path (fh_set_path FH_PATH_MULTI)
 * bit for bit.  FH_EINVAL, before anything is launched, when the call's
 * workspace, 4 B c + 4 B p + 20 B ceil(p b / 8) bytes (each term rounded up
 * to 256), exceeds 8 MiB, and for the argument errors of fh_create and
 * fh_forward.  Every call on a GPU shares that GPU's array, and the array
 * keeps the last call's contents (each call writes all it reads, so nothing
 * needs clearing): calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 */
fh_status fh_forward_noalloc(const void* E, const void* C, const int32_t* c2t, fh_dtype dtype,
                             int64_t v, int64_t d, int64_t c, const void* h, int64_t B, int64_t p,
                             int mode, float temperature, uint64_t seed, int32_t* out_token,
                             float* out_token_logit, float* out_lse, int32_t* out_clusters,
                             int32_t* out_ids, float* out_logits, void* stream);

/*
 * fh_score — stage 1 alone: out_scores[b*c + k] = C_hat[k] . h[b] in float32
 * accumulation, with C_hat the centroids as stored (INT4: sigma * q)
 * ([X] §1.2.4 stage 1).
 *   h device [B x d]; out_scores device [B x c] float.  1 <= B <= max_batch.
 */
fh_status fh_score(fh_engine* e, const void* h, int64_t B, float* out_scores, void* stream);

/*
 * fh_dense_forward — the dense head z = E h over all v tokens ([X] §1.1),
 * finished exactly like fh_forward (argmax or one draw from softmax(z/T), the
 * same Philox stream for tokens, LSE over all v).  The comparison baseline.
 *   out_logits may be NULL; otherwise device [B x v] float.
 */
fh_status fh_dense_forward(fh_engine* e, const void* h, int64_t B, int mode,
                           float temperature, uint64_t seed, int32_t* out_token,
                           float* out_token_logit, float* out_lse, float* out_logits,
                           void* stream);

/*
 * fh_get_int4 — copy the engine's quantised centroids out (FH_QUANT_INT4_G32
 * only, else FH_EINVAL).
 *   packed  device [c x d/2] uint8: two's-complement nibbles, element 2m in
 *           the low nibble of byte m.
 *   scales  device [c x d/32] uint16: fp16 bit patterns of sigma.
 */
fh_status fh_get_int4(fh_engine* e, uint8_t* packed, uint16_t* scales, void* stream);

/*
 * fh_get_int8 — copy the engine's INT8 centroids out (FH_QUANT_INT8_G32
 * only, else FH_EINVAL).
 *   codes   device [c x d] int8, row-major.
 *   scales  device [c x d/32] uint16: fp16 bit patterns of sigma.
 */
fh_status fh_get_int8(fh_engine* e, int8_t* codes, uint16_t* scales, void* stream);

/*
 * fh_spec_verify — verify B FlashHead draft tokens against the dense head
 * with the standard speculative-sampling rule ([X] §4.2 speculative
 * decoding: a FlashHead draft, the original head's probabilities, accept or
 * reject; the rule is Leviathan et al. 2023 / Chen et al. 2023).  Query q
 * is one position with hidden state h[q]:
 *   p(t) = softmax(E h / T) over all v tokens;
 *   q(t) = softmax(E_t h / T) over the retrieved tokens of the draft's
 *          probes, 0 elsewhere (what the draft sampled from);
 *   the draft token x is kept when u < min(1, p(x) / q(x)) with
 *   u = Philox uniform (seed, q, 0, stage 2); otherwise the output is a draw
 *   from max(0, p - q), i.e. from p over the tokens outside the probes
 *   (Gumbel-max with Philox (seed, q, t, stage 3)).
 * The output token is distributed exactly as p.  As both heads score a
 * retrieved token with the same E_t . h, p(x) / q(x) = exp(draft_lse -
 * LSE_full) for x inside the probes.
 *   h               device [B x d] of the engine's dtype, 16-byte aligned.
 *   p               probes per draft, 1 <= p <= c.
 *   draft_clusters  device [B x p] int32: the draft's probes (out_clusters
 *                   of fh_forward); ids outside [0, c) are ignored.
 *   draft_token     device [B] int32: the draft's tokens (out_token of
 *                   fh_forward with FH_TOKEN_SAMPLE at this temperature); a
 *                   token outside [0, v) is rejected, one outside its own
 *                   probes (q = 0) is kept.
 *   draft_lse       device [B] float: the draft's out_lse (log sum exp(z/T)
 *                   over its retrieved tokens).
 *   temperature     T > 0, the draft's temperature.
 *   out_token       device [B] int32: the verified token.
 *   out_accepted    device [B] int32, may be NULL: 1 where the draft was kept.
 *   out_lse         device [B] float, may be NULL: log sum exp(z/T) over all v.
 * Uses the engine's workspace like the other calls (B <= max_batch).
 */
fh_status fh_spec_verify(fh_engine* e, const void* h, int64_t B, int64_t p,
                         const int32_t* draft_clusters, const int32_t* draft_token,
                         const float* draft_lse, float temperature, uint64_t seed,
                         int32_t* out_token, int32_t* out_accepted, float* out_lse,
                         void* stream);

/*
 * Per-kernel timing.  fh_profile_begin(e, n) makes the engine record a HIP
 * event pair on the launch stream around each of its next n kernel launches.
 * fh_profile_end waits for those events and fills up to `max` records
 * (kernel name, launches, total milliseconds) aggregated by kernel, returning
 * how many it wrote in *count.  Names point to static strings.
 */
typedef struct {
  const char* name;
  int64_t launches;
  double total_ms;
} fh_kernel_time;

fh_status fh_profile_begin(fh_engine* e, int64_t max_launches);
fh_status fh_profile_end(fh_engine* e, fh_kernel_time* out, int max, int* count);

/*
 * fh_set_path — choose how fh_forward runs a batch-1 call.
 *   FH_PATH_AUTO  (default) one launch for the whole call when p probes fit
 *                 it: stage-1 workgroups, a selecting workgroup, stage-2
 *                 workgroups and a finishing workgroup hand over through
 *                 device memory.  Batches of B > 1 use one launch per stage.
 *   FH_PATH_MULTI always one launch per stage.
 * Both paths return the same ids and logits; the LSE may differ in the last
 * bits (a different merge order).  While `stream` is being captured into a
 * graph, fh_forward uses the per-stage launches whatever the path: they keep
 * no state between calls, so the graph can be replayed (the single launch
 * tells calls apart by a counter kept on the host).
 */
enum { FH_PATH_AUTO = 0, FH_PATH_MULTI = 1 };
fh_status fh_set_path(fh_engine* e, int path);

/*
 * fh_sync_status — wait for `stream`, then report FH_OK, or FH_EHIP if a
 * bounded wait inside a batch-1 call ever gave up (that call's outputs are
 * invalid; the flag stays set).  Calls that overlap on one engine (see
 * above) are what can cause it.
 */
fh_status fh_sync_status(fh_engine* e, void* stream);

/*
 * Offline clustering: the step that produces C and C2T for fh_create
 * ([X] §1.2.1 balanced clustering, §2.1 offline clustering; [A] abstract,
 * innovation (1)).  Balanced spherical k-means: rows are L2-normalised; c
 * centres are seeded with k-means++; every iteration computes the cosine
 * similarity of every token to every centre, assigns tokens so that every
 * cluster holds exactly b = v / c of them, and moves every centre to the
 * normalised mean of its tokens.  The pages leave these steps open; this
 * library reads them as:
 *   - k-means++ on the sphere: D(t) = 1 - max_j cos(t, C_j); centre 0 is
 *     token floor(u[0] v); centre i is the first token, in id order, whose
 *     running sum of D^2 exceeds u[i] * sum(D^2) (token floor(u[i] v) if
 *     every D is 0).  The uniforms u are inputs, so a run is repeatable.
 *   - balanced assignment by rounds: each unassigned token proposes to its
 *     most similar cluster that is not yet full (ties: smaller cluster id);
 *     each cluster accepts, up to its remaining room, the proposals with the
 *     highest similarity (ties: smaller token id); accepted tokens are final
 *     and the rest propose again.
 *   - update: C_k = normalise(sum of its tokens' unit rows); C2T[k] lists
 *     cluster k's tokens in ascending id.
 * Both calls allocate their own device workspace, run on `stream`, and
 * return after waiting for it (the rounds need the host).
 */

/*
 * fh_balanced_assign — the balanced assignment alone.
 *   sims        device [v x c] float: similarity of token t to cluster k at
 *               sims[t * c + k]; compared as given (no NaN).
 *   v, c        v a positive multiple of c; b = v / c tokens per cluster.
 *   out_assign  device [v] int32: the cluster of every token.
 *   out_rounds  host, may be NULL: the number of rounds taken.
 */
fh_status fh_balanced_assign(const float* sims, int64_t v, int64_t c, int32_t* out_assign,
                             int* out_rounds, void* stream);

typedef struct {
  float init_ms;  /* normalisation and k-means++ seeding                    */
  float sims_ms;  /* the similarity products, summed over iterations        */
  float total_ms; /* the whole call                                         */
  float pp_step_us; /* average duration of the k-means++ distance refresh
                       (one pass over the table), from HIP events around
                       every 16th launch                                    */
  int rounds;     /* balanced-assignment rounds, summed over iterations     */
} fh_cluster_times;

/*
 * fh_cluster — the whole offline clustering.
 *   E           device [v x d] of `dtype` (rows need not be unit length).
 *   v, d, c     v a positive multiple of c, c <= 65536; d as for fh_create
 *               (a multiple of 8 for bf16, of 4 for f32; at most 4096 bf16
 *               or 2048 f32 elements).
 *   iters       >= 1 iterations of (similarities, assignment, update).
 *   u           host [c] double, each in [0, 1): the k-means++ uniforms.
 *   out_C       device [c x d] float: unit centres after the last update.
 *   out_c2t     device [c x b] int32: C2T from the last assignment.
 *   out_init    device [c] int32, may be NULL: the k-means++ token ids.
 *   out_assign  device [v] int32, may be NULL: the last assignment.
 *   out_times   host, may be NULL.
 * out_C and out_c2t are what fh_create takes (after a cast of C to `dtype`
 * for bf16 engines).
 */
fh_status fh_cluster(const void* E, fh_dtype dtype, int64_t v, int64_t d, int64_t c, int iters,
                     const double* u, float* out_C, int32_t* out_c2t, int32_t* out_init,
                     int32_t* out_assign, fh_cluster_times* out_times, void* stream);

/* Thread-local description of the last error on this thread ("" if none). */
const char* fh_last_error(void);

/* Library version string. */
const char* fh_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHHEAD_H */
