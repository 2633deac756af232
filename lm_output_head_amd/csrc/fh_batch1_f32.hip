// Batch-1 single-launch kernel for fp32 heads.
#define FH_BATCH1_T float
#define FH_BATCH1_QB 0
#define FH_BATCH1_ENTRY launch_batch1_f32
#define FH_BATCHED_ENTRY launch_batched_f32
#include "fh_batch1.inl"
