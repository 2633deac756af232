// Batch-1 single-launch kernel for fp32 heads with INT4 stage-1 centroids.
#define FH_BATCH1_T float
#define FH_BATCH1_QB 4
#define FH_BATCH1_ENTRY launch_batch1_f32_int4
#include "fh_batch1.inl"
