// Layout probes for the gfx950 matrix-core and DPP primitives the decode
// and quantize kernels rely on; exported for the GPU unit test only (one wave, fixed
// in-bounds sizes).
#include <hip/hip_runtime.h>

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

typedef float probe_floatx16 __attribute__((ext_vector_type(16)));

// A: 32x16 row-major fp16, B: 16x32 row-major fp16, D: 32x32 row-major fp32.
__global__ __launch_bounds__(64) void probe_mfma_32x32x16_kernel(const _Float16* A, const _Float16* B,
                                                                 float* D) {
  const int l = threadIdx.x;
  probe_half8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = A[(l % 32) * 16 + 8 * (l / 32) + i];   // row l%32, k = 8(l/32)+i
    b[i] = B[(8 * (l / 32) + i) * 32 + (l % 32)]; // k = 8(l/32)+i, col l%32
  }
  probe_floatx16 c;
  for (int i = 0; i < 16; ++i) c[i] = 0.f;
  c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  // col l%32, register v: row 8(v/4) + 4(l/32) + v%4
  for (int v = 0; v < 16; ++v) D[(8 * (v / 4) + 4 * (l / 32) + v % 4) * 32 + (l % 32)] = c[v];
}

}  // namespace tq

extern "C" int tq_probe_mfma_32x32x16(const void* A, const void* B, void* D, hipStream_t stream) {
  hipLaunchKernelGGL(tq::probe_mfma_32x32x16_kernel, dim3(1), dim3(64), 0, stream,
                     static_cast<const _Float16*>(A), static_cast<const _Float16*>(B),
                     static_cast<float*>(D));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int tq_probe_mfma_layout(const void* A, const void* B, void* D, void* dpp_out,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(tq::probe_mfma_16x16x32_kernel, dim3(1), dim3(64), 0, stream,
                     static_cast<const _Float16*>(A), static_cast<const _Float16*>(B),
                     static_cast<float*>(D), static_cast<float*>(dpp_out));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
