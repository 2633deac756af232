// Host-side sizing of the single-launch batch-1 kernel: rows per workgroup
// and workgroup counts of its two stages, and the layout of the tagged
// hand-over words.  Plain C++ (no HIP), so that the bounds can be checked on
// any host.
//
// Sources (page title and section): FlashHead technical explainer
// (framerc.cn) §1.2.2 (top-p probes over the centroid scores), §2.2.2 (the
// computation graph: centroid scores, a selection step, token scores).
#pragma once

#include <stdint.h>

#include <algorithm>

namespace fh {

// Rows per workgroup are a multiple of this (one row for each of the 16
// waves of a 1024-thread workgroup).
#ifndef FH_B1_ROWS_UNIT
#define FH_B1_ROWS_UNIT 16
#endif
constexpr int kBatch1RowsUnit = FH_B1_ROWS_UNIT;
// Probes a stage-2 workgroup can list in LDS (its rows' clusters).
constexpr int kBatch1MaxProbesPerWg = 1024;

// Rows per workgroup: a multiple of kBatch1RowsUnit, large enough that a
// stage over n rows needs at most `slots` workgroups.
inline int64_t batch1_rows(int64_t n, int64_t slots) {
  slots = std::max<int64_t>(slots, 1);
  const int64_t units = (n + kBatch1RowsUnit - 1) / kBatch1RowsUnit;
  return kBatch1RowsUnit * std::max<int64_t>(1, (units + slots - 1) / slots);
}
// Stage-1 workgroup budget: cus - 4, so that the selector and a few stage-2
// workgroups start at once.
inline int64_t batch1_slots1(int cus) { return cus > 8 ? cus - 4 : 4; }
inline int batch1_stage1_blocks(int64_t c, int cus) {
  const int64_t r = batch1_rows(c, batch1_slots1(cus));
  return (int)((c + r - 1) / r);
}
// Stage-2 workgroup budget: cus - 1 (one compute unit for the finisher).
inline int64_t batch1_slots2(int cus) { return std::max(1, cus - 1); }
// At most batch1_slots2(cus) for every p (batch1_rows rounds the rows per
// workgroup up), so the hand-over words are sized by that budget, not by p.
inline int batch1_stage2_blocks(int64_t p, int64_t b, int cus) {
  const int64_t r = batch1_rows(p * b, batch1_slots2(cus));
  return (int)std::max<int64_t>(1, (p * b + r - 1) / r);
}
// Whether a call with p probes of b rows fits the single launch: a stage-2
// workgroup lists the probes of its rows (at most rows / b + 2 of them).
inline bool batch1_fits(int64_t p, int64_t b, int cus) {
  const int64_t rows2 = batch1_rows(p * b, batch1_slots2(cus));
  return rows2 / b + 2 <= kBatch1MaxProbesPerWg;
}

// Tagged words, in this order: scores [c]; the probe bitset [ceil(c / 32)];
// five words per stage-2 partial [5 x batch1_slots2(cus)].
// Batched calls after stage 1 (2 <= B <= kBatchedMaxB queries): one launch of
// B selectors, B x G2q stage-2 workgroups and a finisher, all resident at one
// workgroup per CU: the stage-2 slots CUs - 1 - B are shared by the queries.
constexpr int kBatchedMaxB = 16;
inline int64_t batched_slots2(int B, int cus) { return std::max<int64_t>(1, (cus - 1 - B) / B); }
inline int64_t batched_rows2(int64_t p, int64_t b, int B, int cus) {
  return batch1_rows(p * b, batched_slots2(B, cus));
}
inline int batched_stage2_blocks(int64_t p, int64_t b, int B, int cus) {
  const int64_t r = batched_rows2(p, b, B, cus);
  return (int)std::max<int64_t>(1, (p * b + r - 1) / r);
}
inline bool batched_fits(int64_t p, int64_t b, int B, int cus) {
  return B >= 2 && B <= kBatchedMaxB && cus - 1 - B >= B &&
         batched_rows2(p, b, B, cus) / b + 2 <= kBatch1MaxProbesPerWg;
}
// Tagged words of a batched launch: [B x ceil(c/32)] probe bitsets, then
// [B x G2q x 5] stage-2 partials (at most 5 x (CUs - 1) words).
inline int64_t batched_off_parts(int64_t c, int B) { return (int64_t)B * ((c + 31) / 32); }
inline int64_t batched_tag_words(int64_t c, int max_batch, int cus) {
  return (int64_t)std::min(max_batch, kBatchedMaxB) * ((c + 31) / 32) + 5 * (int64_t)std::max(1, cus - 1);
}

inline int64_t batch1_off_sel(int64_t c) { return c; }
inline int64_t batch1_off_parts(int64_t c) { return c + (c + 31) / 32; }
inline int64_t batch1_tag_words(int64_t c, int cus) {
  return batch1_off_parts(c) + 5 * batch1_slots2(cus);
}

}  // namespace fh
