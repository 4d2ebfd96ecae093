// Instances of the short-query kernel (32-row tiles) over caches grouped along
// the tokens (K, V or both; fp32 metadata), built in their own translation
// unit; the kernel itself is in attention_short.hip.
#define KVQ_SHORT_TOK 1
#include "attention_short.hip"
