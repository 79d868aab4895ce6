// Attention straight from packed codes (a2a-mcp.org page, Stage 2 closing
// paragraph and "How to implement", item 1: the query is rotated once and
// dots are taken against the stored indices; nothing dequantizes the cache).
//
//   l_t = ||k_t|| <q', c_K[idx_t]> + sqrt(pi/2)/m ||k_t|| ||r_t|| <u, 2 s_t - 1>
//   q' = Pi q, u = S q'  (the 1-bit JL correction that makes l unbiased)
//
// This file holds the query preparation shared with decode and the logits
// kernel (fp32 dots on the vector ALUs); decode itself is in decode.hip.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace tq {

constexpr int kAD = 128;
constexpr int kAM = 128;

// ------------------------------------------------------------- query prep
// One workgroup per query head: q' = Pi q, then (keys with a sketch) u = S q'.
// Eight threads share a row: thread t takes rows t/8 + 32p (p = 0..3) and of
// each the float4 columns t%8 + 8k (k = 0..3), so that the 8 lanes of a row
// read 128 contiguous bytes per load and a wave touches 8 cache lines per
// load.  All of both matrices' loads are issued up front (the kernel waits
// for memory once); the vectors come from LDS, the same four float4 for
// every row of a thread; three DPP adds sum a row's eighths.
constexpr int kQThreadsP = 2 * kAD;

__device__ __forceinline__ float sum_eighths(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));
  return v;
}

template <typename QT>
__global__ __launch_bounds__(kQThreadsP) void qprep_kernel(const float* __restrict__ rot,
                                                           const float* __restrict__ sketch, int m,
                                                           const QT* __restrict__ q,
                                                           float* __restrict__ qr,
                                                           float* __restrict__ u) {
  __shared__ __align__(16) float xs[kAD], ys[kAD];
  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x, r0 = tid >> 3, j = tid & 7;
  const bool sk = m > 0;                    // m is 0 or kAM (checked on the host)
  float4 pr[4][4], sr[4][4];                // [row p][float4 k]
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float4* prow = reinterpret_cast<const float4*>(rot + (r0 + 32 * p) * kAD);
#pragma unroll
    for (int k = 0; k < 4; ++k) pr[p][k] = prow[j + 8 * k];
  }
  if (sk) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float4* srow = reinterpret_cast<const float4*>(sketch + (r0 + 32 * p) * kAD);
#pragma unroll
      for (int k = 0; k < 4; ++k) sr[p][k] = srow[j + 8 * k];
    }
  }
  if (tid < kAD) xs[tid] = load_elem(q, h * kAD + tid);
  __syncthreads();
  // rows r0 + 32p of W v, every lane of the row's eight holding the sum
  auto dots = [&](const float4 (&w)[4][4], const float* v, float (&out)[4]) {
    float4 vv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) vv[k] = reinterpret_cast<const float4*>(v)[j + 8 * k];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a = fmaf(w[p][k].x, vv[k].x, a);
        a = fmaf(w[p][k].y, vv[k].y, a);
        a = fmaf(w[p][k].z, vv[k].z, a);
        a = fmaf(w[p][k].w, vv[k].w, a);
      }
      out[p] = sum_eighths(a);
    }
  };
  float y[4];
  dots(pr, xs, y);
  if (j == 0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      ys[r0 + 32 * p] = y[p];
      qr[h * kAD + r0 + 32 * p] = y[p];
    }
  }
  if (sk) {
    __syncthreads();
    float z[4];
    dots(sr, ys, z);
    if (j == 0) {
#pragma unroll
      for (int p = 0; p < 4; ++p) u[h * kAM + r0 + 32 * p] = z[p];
    }
  }
}

hipError_t launch_qprep(const tq_tables& tk, const void* q, int q_dtype, int nh, float* qr,
                        float* u, hipStream_t stream) {
  if (nh == 0) return hipSuccess;
  if (q_dtype == TQ_BF16)
    hipLaunchKernelGGL(qprep_kernel<uint16_t>, dim3(nh), dim3(kQThreadsP), 0, stream, tk.rot,
                       tk.sketch, tk.m, static_cast<const uint16_t*>(q), qr, u);
  else
    hipLaunchKernelGGL(qprep_kernel<float>, dim3(nh), dim3(kQThreadsP), 0, stream, tk.rot,
                       tk.sketch, tk.m, static_cast<const float*>(q), qr, u);
  return hipGetLastError();
}

// --------------------------------------------------- one key record's logits
// G logits of token t of sequence s, for the G query heads whose rotated
// queries sit in qs[g][*] (and us[g][*]).  Returns them through l[].
template <int G>
__device__ __forceinline__ void key_logits_one(const uint32_t* __restrict__ codes,
                                               const uint32_t* __restrict__ signs,
                                               const void* norm, const void* rnorm, int nd,
                                               int bits, int m, int64_t rec,
                                               const float (*qs)[kAD], const float (*us)[kAM],
                                               const float* cs, float qjl, float* l) {
  float ac[G], as[G];
#pragma unroll
  for (int g = 0; g < G; ++g) ac[g] = as[g] = 0.f;
  const uint32_t* cw = codes + rec * (kAD / 32) * bits;
  for (int w = 0; w < kAD / 32; ++w) {
    uint32_t pw[4];
    for (int p = 0; p < bits; ++p) pw[p] = cw[w * bits + p];
    for (int k = 0; k < 32; ++k) {
      int idx = 0;
      for (int p = 0; p < bits; ++p) idx |= ((pw[p] >> k) & 1u) << p;
      const float c = cs[idx];
      const int jj = w * 32 + k;
#pragma unroll
      for (int g = 0; g < G; ++g) ac[g] = fmaf(qs[g][jj], c, ac[g]);
    }
  }
  if (m > 0) {
    const uint32_t* sw = signs + rec * (m / 32);
    for (int w = 0; w < m / 32; ++w) {
      const uint32_t word = sw[w];
      for (int k = 0; k < 32; ++k) {
        const float sg = ((word >> k) & 1u) ? 1.f : -1.f;
        const int ii = w * 32 + k;
#pragma unroll
        for (int g = 0; g < G; ++g) as[g] = fmaf(us[g][ii], sg, as[g]);
      }
    }
  }
  const float n = load_norm(norm, nd, rec);
  const float rn = (m > 0) ? load_norm(rnorm, nd, rec) : 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = n * ac[g] + qjl * rn * as[g];
}

// ------------------------------------------------------------------ logits
constexpr int kLThreads = 256;

template <int G>
__global__ __launch_bounds__(kLThreads) void logits_kernel(
    const float* __restrict__ cent, int bits, int m, const float* __restrict__ qr,
    const float* __restrict__ u, int Hq, int Hkv, int64_t T, int64_t Tp,
    const uint32_t* __restrict__ codes,
    const uint32_t* __restrict__ signs, const void* norm, const void* rnorm, int nd,
    float* __restrict__ logits) {
  __shared__ float qs[G][kAD];
  __shared__ float us[G][kAM];
  __shared__ float cs[16];
  const int64_t s = blockIdx.y;  // sequence = b * Hkv + kv head
  const int64_t h0 = s * G;      // first query head (b * Hq + kv * G)
  const int tid = threadIdx.x;
  for (int i = tid; i < G * kAD; i += kLThreads) qs[i / kAD][i % kAD] = qr[h0 * kAD + i];
  if (m > 0)
    for (int i = tid; i < G * m; i += kLThreads) us[i / m][i % m] = u[h0 * m + i];
  if (tid < (1 << bits)) cs[tid] = cent[tid];
  __syncthreads();
  const float qjl = (m > 0) ? sqrtf(static_cast<float>(M_PI) / 2.f) / m : 0.f;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kLThreads + tid;
  if (t >= T) return;
  float l[G];
  key_logits_one<G>(codes, signs, norm, rnorm, nd, bits, m, s * Tp + t, qs, us, cs, qjl, l);
#pragma unroll
  for (int g = 0; g < G; ++g) logits[(h0 + g) * T + t] = l[g];
}

hipError_t launch_logits(const tq_tables& tk, const float* qr, const float* u, int B, int Hq,
                         int Hkv, const tq_packed& k, float* logits, hipStream_t stream) {
  if (k.T == 0 || B == 0) return hipSuccess;
  const int G = Hq / Hkv;
  dim3 grid(static_cast<unsigned>((k.T + kLThreads - 1) / kLThreads),
            static_cast<unsigned>(B * Hkv));
#define TQ_LLAUNCH(GV)                                                                          \
  hipLaunchKernelGGL(logits_kernel<GV>, grid, dim3(kLThreads), 0, stream, tk.centroids,        \
                     tk.bits, tk.m, qr, u, Hq, Hkv, k.T, stream_stride(k), k.codes, k.signs,   \
                     k.norm, k.rnorm,                                                          \
                     k.norm_dtype, logits)
  switch (G) {
    case 1: TQ_LLAUNCH(1); break;
    case 2: TQ_LLAUNCH(2); break;
    case 4: TQ_LLAUNCH(4); break;
    case 8: TQ_LLAUNCH(8); break;
    case 16: TQ_LLAUNCH(16); break;
    default: return hipErrorInvalidValue;
  }
#undef TQ_LLAUNCH
  return hipGetLastError();
}

}  // namespace tq
