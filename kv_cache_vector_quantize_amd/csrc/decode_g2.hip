// Decode and logits kernels for 2 query heads per KV head.
#include "decode_kernels.h"

namespace tq {
TQ_DECODE_G_TU(2)
}  // namespace tq
