// Batch-1 single-launch kernel for bf16 heads with INT4 stage-1 centroids.
#define FH_BATCH1_T uint16_t
#define FH_BATCH1_QB 4
#define FH_BATCH1_ENTRY launch_batch1_bf16_int4
#include "fh_batch1.inl"
