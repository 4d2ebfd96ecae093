// Bfloat16-metadata, paged-cache instances of the 16-row short-query kernel,
// built in their own translation unit; the kernel itself is in
// attention_short16.hip.
#define KVQ_SHORT16_PAGED 1
#define KVQ_SHORT16_META16 2
#include "attention_short16.hip"
