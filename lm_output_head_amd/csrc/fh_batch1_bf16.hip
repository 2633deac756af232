// Batch-1 single-launch kernel for bf16 heads.
#define FH_BATCH1_T uint16_t
#define FH_BATCH1_QB 0
#define FH_BATCH1_ENTRY launch_batch1_bf16
#define FH_BATCHED_ENTRY launch_batched_bf16
#include "fh_batch1.inl"
