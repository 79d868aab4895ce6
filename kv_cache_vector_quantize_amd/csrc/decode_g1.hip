// Decode and logits kernels for 1 query head per KV head.
#include "decode_kernels.h"

namespace tq {
TQ_DECODE_G_TU(1)
}  // namespace tq
