// Instances of the general attention kernel for caches grouped along the
// tokens (per channel), built in their own translation unit; the kernel
// itself is in attention.hip.
#define KVQ_TILE_TOKENS 1
#include "attention.hip"
