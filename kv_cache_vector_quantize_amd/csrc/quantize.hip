// Online quantization of key / value vectors (a2a-mcp.org page, "How it
// works": Stage 1 normalise + rotate + Lloyd-Max per coordinate; Stage 2,
// keys only, 1-bit QJL sketch of the residual).
//
// Layout of the work: one unit = 32 consecutive tokens of one sequence (one
// value-stream record per coordinate).  A persistent workgroup of
// 256 threads keeps Pi^T and S^T in LDS and walks units; per unit it takes
// the 32 tokens 8 at a time.  Thread (j, hv): coordinate j = tid % 128,
// vector half hv = tid / 128 (4 of the 8 vectors).
#include "common.h"
#include "launch.h"

namespace tq {

constexpr int kD = 128;
constexpr int kM = 128;
constexpr int kQThreads = 256;
constexpr int kVec = 8;  // vectors per inner step

template <typename XT, bool KEY>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(
    const float* __restrict__ rot, const float* __restrict__ sketch,
    const float* __restrict__ cent, const float* __restrict__ bnd, int bits,
    const XT* __restrict__ x, int64_t nseq, int64_t T, uint32_t* __restrict__ codes,
    uint32_t* __restrict__ signs, void* __restrict__ norm, void* __restrict__ rnorm,
    int norm_dtype) {
  __shared__ float PiT[kD][kD];                          // PiT[k][j] = Pi[j][k]
  __shared__ float ST[KEY ? kD : 1][KEY ? kM : 1];       // ST[j][i] = S[i][j]
  __shared__ __align__(16) float xs[kD][kVec];
  __shared__ __align__(16) float rs[kD][kVec];
  __shared__ float red[4][4], red2[4][4];
  __shared__ float nrm[kVec], rho[kVec];
  __shared__ float sc[16], sb[16];
  __shared__ uint32_t vw[kD][4];

  const int tid = threadIdx.x;
  const int j = tid & (kD - 1);
  const int hv = tid >> 7;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = 1 << bits;

  for (int i = tid; i < kD * kD; i += kQThreads) PiT[i % kD][i / kD] = rot[i];
  if constexpr (KEY) {
    for (int i = tid; i < kM * kD; i += kQThreads) ST[i % kD][i / kD] = sketch[i];
  }
  if (tid < L) sc[tid] = cent[tid];
  if (tid < L - 1) sb[tid] = bnd[tid];
  __syncthreads();

  const int64_t nblk = (T + 31) / 32;
  const int64_t units = nseq * nblk;
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int64_t s = unit / nblk;
    const int64_t blk = unit % nblk;
    // value record of coordinate j: token k's index at bits [bits*k, bits*k+bits)
    uint64_t vlo = 0, vhi = 0;
    for (int it = 0; it < 32 / kVec; ++it) {
      const int64_t t0 = blk * 32 + it * kVec;
      for (int e = tid; e < kD * kVec; e += kQThreads) {
        const int v = e / kD, k = e % kD;
        const int64_t t = t0 + v;
        xs[k][v] = (t < T) ? load_elem(x, (s * T + t) * kD + k) : 0.0f;
      }
      __syncthreads();
      // ||x||: thread partials over its coordinate, wave sums, then 2 waves
#pragma unroll
      for (int vi = 0; vi < 4; ++vi) {
        const float xv = xs[j][hv * 4 + vi];
        const float sum = wave_sum(xv * xv);
        if (lane == 0) red[wave][vi] = sum;
      }
      __syncthreads();
      if (tid < kVec) nrm[tid] = sqrtf(red[2 * (tid / 4)][tid % 4] + red[2 * (tid / 4) + 1][tid % 4]);
      __syncthreads();

      // y_j = sum_k Pi[j][k] x_k for the 4 vectors of this half
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int k = 0; k < kD; ++k) {
        const float p = PiT[k][j];
        const float4 xv = *reinterpret_cast<const float4*>(&xs[k][hv * 4]);
        acc[0] = fmaf(p, xv.x, acc[0]);
        acc[1] = fmaf(p, xv.y, acc[1]);
        acc[2] = fmaf(p, xv.z, acc[2]);
        acc[3] = fmaf(p, xv.w, acc[3]);
      }

      float rsq[4];
#pragma unroll
      for (int vi = 0; vi < 4; ++vi) {
        const int v = hv * 4 + vi;
        const int64_t t = t0 + v;
        const bool valid = t < T;
        const float n = nrm[v];
        int idx;
        float yh = 0.f;
        if (n > 0.f) {
          yh = acc[vi] / n;
          idx = 0;
          for (int i = 0; i < L - 1; ++i) idx += (yh >= sb[i]) ? 1 : 0;
        } else {
          idx = L / 2;
        }
        if constexpr (KEY) {
          const float r = (n > 0.f) ? yh - sc[idx] : 0.f;
          rs[j][v] = r;
          rsq[vi] = r * r;
          for (int p = 0; p < bits; ++p) {
            const uint64_t mask = __ballot((idx >> p) & 1);
            if (valid && (lane & 31) == 0) {
              const uint32_t word = (lane == 0) ? static_cast<uint32_t>(mask)
                                                : static_cast<uint32_t>(mask >> 32);
              codes[((s * T + t) * (kD / 32) + j / 32) * bits + p] = word;
            }
          }
        } else {
          if (valid) {
            const int pos = bits * (it * kVec + v);
            const uint64_t f = static_cast<uint64_t>(idx);
            if (pos < 64) {
              vlo |= f << pos;
              if (pos + bits > 64) vhi |= f >> (64 - pos);
            } else {
              vhi |= f << (pos - 64);
            }
          }
        }
      }

      if constexpr (KEY) {
#pragma unroll
        for (int vi = 0; vi < 4; ++vi) {
          const float sum = wave_sum(rsq[vi]);
          if (lane == 0) red2[wave][vi] = sum;
        }
        __syncthreads();
        if (tid < kVec) {
          rho[tid] = sqrtf(red2[2 * (tid / 4)][tid % 4] + red2[2 * (tid / 4) + 1][tid % 4]);
          const int64_t t = t0 + tid;
          if (t < T) {
            store_norm(norm, norm_dtype, s * T + t, nrm[tid]);
            store_norm(rnorm, norm_dtype, s * T + t, nrm[tid] * rho[tid]);
          }
        }
        // z_i = sum_j S[i][j] r_j ; sign bit = [z >= 0]
        const int i = j;
        float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int jj = 0; jj < kD; ++jj) {
          const float sv = ST[jj][i];
          const float4 rv = *reinterpret_cast<const float4*>(&rs[jj][hv * 4]);
          z[0] = fmaf(sv, rv.x, z[0]);
          z[1] = fmaf(sv, rv.y, z[1]);
          z[2] = fmaf(sv, rv.z, z[2]);
          z[3] = fmaf(sv, rv.w, z[3]);
        }
#pragma unroll
        for (int vi = 0; vi < 4; ++vi) {
          const int64_t t = t0 + hv * 4 + vi;
          const uint64_t mask = __ballot(z[vi] >= 0.f);
          if (t < T && (lane & 31) == 0) {
            const uint32_t word = (lane == 0) ? static_cast<uint32_t>(mask)
                                              : static_cast<uint32_t>(mask >> 32);
            signs[(s * T + t) * (kM / 32) + i / 32] = word;
          }
        }
      } else {
        if (tid < kVec) {
          const int64_t t = t0 + tid;
          if (t < T) store_norm(norm, norm_dtype, s * T + t, nrm[tid]);
        }
      }
      __syncthreads();
    }
    if constexpr (!KEY) {
      const uint32_t rec[4] = {static_cast<uint32_t>(vlo), static_cast<uint32_t>(vlo >> 32),
                               static_cast<uint32_t>(vhi), static_cast<uint32_t>(vhi >> 32)};
      if (hv == 1) {
#pragma unroll
        for (int p = 0; p < 4; ++p) vw[j][p] = rec[p];
      }
      __syncthreads();
      if (hv == 0) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          if (p < bits) codes[((s * nblk + blk) * kD + j) * bits + p] = rec[p] | vw[j][p];
      }
      __syncthreads();
    }
  }
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

hipError_t launch_quantize(const tq_tables& t, const void* x, int x_dtype, const tq_packed& out,
                           hipStream_t stream) {
  const int64_t nblk = (out.T + 31) / 32;
  const int64_t units = out.nseq * nblk;
  if (units == 0) return hipSuccess;
  const int64_t grid = units < device_cus() ? units : device_cus();
  const bool key = out.role == TQ_KEY;
#define TQ_QLAUNCH(XT, KEYV)                                                                     \
  hipLaunchKernelGGL((quantize_kernel<XT, KEYV>), dim3(static_cast<unsigned>(grid)),             \
                     dim3(kQThreads), 0, stream, t.rot, t.sketch, t.centroids, t.bounds, t.bits, \
                     static_cast<const XT*>(x), out.nseq, out.T, out.codes, out.signs, out.norm, \
                     out.rnorm, out.norm_dtype)
  if (x_dtype == TQ_BF16) {
    if (key) TQ_QLAUNCH(uint16_t, true); else TQ_QLAUNCH(uint16_t, false);
  } else {
    if (key) TQ_QLAUNCH(float, true); else TQ_QLAUNCH(float, false);
  }
#undef TQ_QLAUNCH
  return hipGetLastError();
}

}  // namespace tq
