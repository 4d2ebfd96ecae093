// Causal-mask instances of the throughput kernel (end-aligned mask within
// the current chunk), built in their own translation unit; the kernel itself
// is in attention_fast.hip.
#define KVQ_FAST_CAUSAL 1
#include "attention_fast.hip"
