// Binary16-metadata, paged-cache instances of the throughput kernel,
// built in their own translation unit; the kernel itself is in
// attention_fast.hip.
#define KVQ_FAST_META16 1
#define KVQ_FAST_PAGED 1
#include "attention_fast.hip"
