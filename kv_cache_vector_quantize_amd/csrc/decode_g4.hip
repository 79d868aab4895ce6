// Decode and logits kernels for 4 query heads per KV head.
#include "decode_kernels.h"

namespace tq {
TQ_DECODE_G_TU(4)
}  // namespace tq
