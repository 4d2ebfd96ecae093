// Bfloat16-metadata instances of the short-query kernel, built in their own
// translation unit; the kernel itself is in attention_short.hip.
#define KVQ_SHORT_META16 2
#include "attention_short.hip"
