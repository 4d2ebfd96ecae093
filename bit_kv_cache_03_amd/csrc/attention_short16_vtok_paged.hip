// Instances of the 16-row short-query kernel over paged V caches grouped
// along the tokens (keys either way, fp32 metadata), built in their own
// translation unit; the kernel itself is in attention_short16.hip.
#define KVQ_SHORT16_VTOK 1
#define KVQ_SHORT16_PAGED 1
#include "attention_short16.hip"
