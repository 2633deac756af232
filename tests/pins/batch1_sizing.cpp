// Host check of the single-launch batch-1 sizing (fh_batch1_sizing.hpp): for
// the given (v, c, cus) and every p in [1, c] that the single launch takes,
// every hand-over word the kernel writes lies inside the buffer the engine
// allocates (scores, probe bitset, five words per stage-2 partial), the
// stage-1 workgroups cover the c centroid rows, and a stage-2 workgroup's
// probe list fits its LDS array.  Prints "ok ..." or the failure.
#include <cstdio>
#include <cstdlib>

#include "fh_batch1_sizing.hpp"

using namespace fh;

static int fail(const char* what, long long v, long long c, int cus, long long p) {
  std::printf("FAIL %s v=%lld c=%lld cus=%d p=%lld\n", what, v, c, cus, p);
  return 1;
}

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const long long v = std::atoll(argv[1]), c = std::atoll(argv[2]);
  const int cus = std::atoi(argv[3]);
  const long long b = v / c;
  const long long words = batch1_tag_words(c, cus);
  // stage 1 covers [0, c) with rows1 rows per workgroup
  const long long r1 = batch1_rows(c, batch1_slots1(cus));
  const int g1 = batch1_stage1_blocks(c, cus);
  if ((long long)g1 * r1 < c || (long long)(g1 - 1) * r1 >= c) return fail("stage-1 cover", v, c, cus, 0);
  if (g1 > batch1_slots1(cus)) return fail("stage-1 workgroups over budget", v, c, cus, 0);
  if (batch1_off_sel(c) < c || batch1_off_parts(c) < batch1_off_sel(c) + (c + 31) / 32)
    return fail("score and bitset regions overlap", v, c, cus, 0);
  long long fits = 0, maxg2 = 0;
  for (long long p = 1; p <= c; ++p) {
    if (!batch1_fits(p, b, cus)) continue;
    ++fits;
    const long long r2 = batch1_rows(p * b, batch1_slots2(cus));
    const long long g2 = batch1_stage2_blocks(p, b, cus);
    if (g2 * r2 < p * b) return fail("stage-2 cover", v, c, cus, p);
    // the partials: five words per stage-2 workgroup, the last at
    // off_parts + 5 g2 - 1
    if (batch1_off_parts(c) + 5 * g2 > words) return fail("stage-2 partials overflow", v, c, cus, p);
    if (g2 > maxg2) maxg2 = g2;
    // each workgroup lists the probes of its rows: positions [r_lo / b,
    // (r_hi - 1) / b] of the probe list
    for (long long j = 0; j < g2; ++j) {
      const long long lo = j * r2, hi = (lo + r2 < p * b) ? lo + r2 : p * b;
      if (hi <= lo) continue;
      const long long npos = (hi - 1) / b - lo / b + 1;
      if (npos > kBatch1MaxProbesPerWg) return fail("probe list exceeds LDS", v, c, cus, p);
    }
  }
  // batched launches after stage 1: B selectors, B x g2q stage-2 workgroups
  // and a finisher, all within the CUs; every tagged word inside the buffer
  const long long bwords = batched_tag_words(c, kBatchedMaxB, cus);
  long long bfits = 0;
  for (int B = 2; B <= kBatchedMaxB; ++B) {
    for (long long p = 1; p <= c; ++p) {
      if (!batched_fits(p, b, B, cus)) continue;
      ++bfits;
      const long long r2 = batched_rows2(p, b, B, cus);
      const long long g2 = batched_stage2_blocks(p, b, B, cus);
      if (g2 * r2 < p * b) return fail("batched stage-2 cover", v, c, cus, p);
      if (B + B * g2 + 1 > cus) return fail("batched grid exceeds the CUs", v, c, cus, p);
      if (batched_off_parts(c, B) + 5 * B * g2 > bwords)
        return fail("batched partials overflow", v, c, cus, p);
      for (long long j = 0; j < g2; ++j) {
        const long long lo = j * r2, hi = (lo + r2 < p * b) ? lo + r2 : p * b;
        if (hi <= lo) continue;
        if ((hi - 1) / b - lo / b + 1 > kBatch1MaxProbesPerWg)
          return fail("batched probe list exceeds LDS", v, c, cus, p);
      }
    }
  }
  std::printf("ok g1=%d rows1=%lld fits=%lld maxg2=%lld words=%lld batched_fits=%lld\n", g1, r1,
              fits, maxg2, words, bfits);
  return 0;
}
