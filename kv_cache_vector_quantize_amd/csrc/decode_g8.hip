// Decode and logits kernels for 8 query heads per KV head.
#include "decode_kernels.h"

namespace tq {
TQ_DECODE_G_TU(8)
}  // namespace tq
