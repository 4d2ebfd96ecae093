// Bfloat16-metadata instances of the throughput kernel, built in their own
// translation unit; the kernel itself is in attention_fast.hip.
#define KVQ_FAST_META16 2
#include "attention_fast.hip"
