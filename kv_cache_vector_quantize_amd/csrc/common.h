// Device-side helpers shared by the libtq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);

template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) {
  return p[i];
}

template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// Store a norm either as float32 or as float16 (round to nearest even).
__device__ __forceinline__ void store_norm(void* base, int norm_dtype, int64_t i, float v) {
  if (norm_dtype == TQ_F16) {
    _Float16 h = static_cast<_Float16>(v);
    reinterpret_cast<_Float16*>(base)[i] = h;
  } else {
    reinterpret_cast<float*>(base)[i] = v;
  }
}

__device__ __forceinline__ float load_norm(const void* base, int norm_dtype, int64_t i) {
  if (norm_dtype == TQ_F16) return static_cast<float>(reinterpret_cast<const _Float16*>(base)[i]);
  return reinterpret_cast<const float*>(base)[i];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace tq
