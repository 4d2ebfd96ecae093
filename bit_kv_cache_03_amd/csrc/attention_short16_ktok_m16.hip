// Instances of the 16-row short-query kernel over binary16-metadata K caches
// grouped along the tokens, built in their own translation unit; the kernel
// itself is in attention_short16.hip.
#define KVQ_SHORT16_KTOK 1
#define KVQ_SHORT16_META16 1
#include "attention_short16.hip"
