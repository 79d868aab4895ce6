// Layout probe for the gfx950 matrix-core and DPP primitives the decode
// kernel relies on; exported for the GPU unit test only (one wave, fixed
// in-bounds sizes).
#include "common.h"

namespace tq {

typedef _Float16 probe_half8 __attribute__((ext_vector_type(8)));
typedef float probe_floatx4 __attribute__((ext_vector_type(4)));

// A: 16x32 row-major fp16, B: 32x16 row-major fp16, D: 16x16 row-major fp32.
// Each lane loads its fragment as the layout under test says.
__global__ __launch_bounds__(64) void probe_mfma_16x16x32_kernel(const _Float16* A, const _Float16* B,
                                                                 float* D, float* dpp_out) {
  const int l = threadIdx.x;
  probe_half8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = A[(l % 16) * 32 + 8 * (l / 16) + i];   // row l%16, k = 8(l/16)+i
    b[i] = B[(8 * (l / 16) + i) * 16 + (l % 16)]; // k = 8(l/16)+i, col l%16
  }
  probe_floatx4 c = {0.f, 0.f, 0.f, 0.f};
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  for (int i = 0; i < 4; ++i) D[(4 * (l / 16) + i) * 16 + (l % 16)] = c[i];  // col l%16, row 4(l/16)+i
  // row_shl:4 (dpp_ctrl 0x104): record which lane's value each lane receives
  const int v = __builtin_amdgcn_update_dpp(-1, l, 0x104, 0xf, 0xf, false);
  dpp_out[l] = static_cast<float>(v);
}

}  // namespace tq

extern "C" int tq_probe_mfma_layout(const void* A, const void* B, void* D, void* dpp_out,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(tq::probe_mfma_16x16x32_kernel, dim3(1), dim3(64), 0, stream,
                     static_cast<const _Float16*>(A), static_cast<const _Float16*>(B),
                     static_cast<float*>(D), static_cast<float*>(dpp_out));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
