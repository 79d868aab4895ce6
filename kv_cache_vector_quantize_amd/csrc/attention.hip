// Attention straight from packed codes (a2a-mcp.org page, Stage 2 closing
// paragraph and "How to implement", item 1: the query is rotated once and
// dots are taken against the stored indices; nothing dequantizes the cache).
//
//   l_t = ||k_t|| <q', c_K[idx_t]> + sqrt(pi/2)/m ||k_t|| ||r_t|| <u, 2 s_t - 1>
//   q' = Pi q, u = S q'  (the 1-bit JL correction that makes l unbiased)
//
// Decode: a = softmax(scale * l) per query head; values are summed in the
// rotated domain, acc = sum_t a_t ||v_t|| c_V[idxV_t], and rotated back once,
// out = Pi^T acc.  Split-K over the context: every workgroup reduces one
// chunk of tokens for the G query heads that share a KV head and leaves
// (max, sum, acc) behind; a combine kernel merges the chunks by
// log-sum-exp and applies Pi^T.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace tq {

constexpr int kAD = 128;
constexpr int kAM = 128;
constexpr int kChunk = 1024;  // tokens per decode split (multiple of 32)

// ------------------------------------------------------------- query prep
template <typename QT>
__global__ __launch_bounds__(kAD) void qprep_kernel(const float* __restrict__ rot,
                                                    const float* __restrict__ sketch, int m,
                                                    const QT* __restrict__ q,
                                                    float* __restrict__ qr,
                                                    float* __restrict__ u) {
  __shared__ float qs[kAD], qrs[kAD];
  const int h = blockIdx.x, j = threadIdx.x;
  qs[j] = load_elem(q, static_cast<int64_t>(h) * kAD + j);
  __syncthreads();
  float a = 0.f;
  for (int k = 0; k < kAD; ++k) a = fmaf(rot[j * kAD + k], qs[k], a);
  qrs[j] = a;
  qr[static_cast<int64_t>(h) * kAD + j] = a;
  __syncthreads();
  if (m > 0 && j < m) {
    float b = 0.f;
    for (int k = 0; k < kAD; ++k) b = fmaf(sketch[j * kAD + k], qrs[k], b);
    u[static_cast<int64_t>(h) * m + j] = b;
  }
}

hipError_t launch_qprep(const tq_tables& tk, const void* q, int q_dtype, int nh, float* qr,
                        float* u, hipStream_t stream) {
  if (nh == 0) return hipSuccess;
  if (q_dtype == TQ_BF16)
    hipLaunchKernelGGL(qprep_kernel<uint16_t>, dim3(nh), dim3(kAD), 0, stream, tk.rot, tk.sketch,
                       tk.m, static_cast<const uint16_t*>(q), qr, u);
  else
    hipLaunchKernelGGL(qprep_kernel<float>, dim3(nh), dim3(kAD), 0, stream, tk.rot, tk.sketch,
                       tk.m, static_cast<const float*>(q), qr, u);
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
    const float* __restrict__ u, int Hq, int Hkv, int64_t T, const uint32_t* __restrict__ codes,
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
  key_logits_one<G>(codes, signs, norm, rnorm, nd, bits, m, s * T + t, qs, us, cs, qjl, l);
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
                     tk.bits, tk.m, qr, u, Hq, Hkv, k.T, k.codes, k.signs, k.norm, k.rnorm,    \
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

// ------------------------------------------------------------ decode split
constexpr int kDThreads = 256;

int decode_splits(int64_t T) { return static_cast<int>((T + kChunk - 1) / kChunk); }

template <int G>
__global__ __launch_bounds__(kDThreads) void decode_partial_kernel(
    const float* __restrict__ ck, int kbits, int m, const float* __restrict__ cv, int vbits,
    const float* __restrict__ qr, const float* __restrict__ u, int64_t T,
    const uint32_t* __restrict__ kcodes, const uint32_t* __restrict__ ksigns, const void* knorm,
    const void* krnorm, int knd, const uint32_t* __restrict__ vcodes, const void* vnorm, int vnd,
    float scale, int nsplit, float* __restrict__ partials) {
  __shared__ float qs[G][kAD];
  __shared__ float us[G][kAM];
  __shared__ float cks[16], cvs[16];
  __shared__ float lg[G][kChunk];
  __shared__ float nvs[kChunk];
  __shared__ float red[kDThreads / 64][G];
  __shared__ float mx[G], sm[G];
  __shared__ float accx[G][kAD];

  const int split = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int64_t h0 = s * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < G * kAD; i += kDThreads) qs[i / kAD][i % kAD] = qr[h0 * kAD + i];
  if (m > 0)
    for (int i = tid; i < G * m; i += kDThreads) us[i / m][i % m] = u[h0 * m + i];
  if (tid < (1 << kbits)) cks[tid] = ck[tid];
  if (tid < (1 << vbits)) cvs[tid] = cv[tid];
  __syncthreads();

  const int64_t t0 = static_cast<int64_t>(split) * kChunk;
  const int64_t t1 = (t0 + kChunk < T) ? t0 + kChunk : T;
  const int n = static_cast<int>(t1 - t0);
  const float qjl = (m > 0) ? sqrtf(static_cast<float>(M_PI) / 2.f) / m : 0.f;

  // 1. scaled logits of the chunk, and the value norms
  float lmax[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lmax[g] = -INFINITY;
  for (int i = tid; i < n; i += kDThreads) {
    float l[G];
    key_logits_one<G>(kcodes, ksigns, knorm, krnorm, knd, kbits, m, s * T + t0 + i, qs, us, cks,
                      qjl, l);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float v = scale * l[g];
      lg[g][i] = v;
      lmax[g] = fmaxf(lmax[g], v);
    }
    nvs[i] = load_norm(vnorm, vnd, s * T + t0 + i);
  }
  // 2. chunk max and sum of exp per head
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float v = wave_max(lmax[g]);
    if (lane == 0) red[wave][g] = v;
  }
  __syncthreads();
  if (tid < G) {
    float v = red[0][tid];
    for (int w = 1; w < kDThreads / 64; ++w) v = fmaxf(v, red[w][tid]);
    mx[tid] = v;
  }
  __syncthreads();
  float lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lsum[g] = 0.f;
  for (int i = tid; i < n; i += kDThreads) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = expf(lg[g][i] - mx[g]);
      lg[g][i] = p * nvs[i];  // weight of the value's unit-scale codeword
      lsum[g] += p;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float v = wave_sum(lsum[g]);
    if (lane == 0) red[wave][g] = v;
  }
  __syncthreads();
  if (tid < G) {
    float v = 0.f;
    for (int w = 0; w < kDThreads / 64; ++w) v += red[w][tid];
    sm[tid] = v;
  }

  // 3. rotated-domain value sum: thread (j, half) walks alternate 32-token blocks
  const int j = tid & (kAD - 1), half = tid >> 7;
  float acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.f;
  const int64_t nblk = (T + 31) / 32;
  const int nb = (n + 31) / 32;
  for (int bb = half; bb < nb; bb += 2) {
    const int64_t blk = t0 / 32 + bb;
    const uint32_t* vw = vcodes + ((s * nblk + blk) * kAD + j) * vbits;
    uint32_t pw[4];
    for (int p = 0; p < vbits; ++p) pw[p] = vw[p];
    const int kmax = (n - bb * 32 < 32) ? n - bb * 32 : 32;
    for (int k = 0; k < kmax; ++k) {
      int idx = 0;
      for (int p = 0; p < vbits; ++p) idx |= ((pw[p] >> k) & 1u) << p;
      const float c = cvs[idx];
      const int i = bb * 32 + k;
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = fmaf(lg[g][i], c, acc[g]);
    }
  }
  if (half == 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) accx[g][j] = acc[g];
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* out = partials + ((h0 + g) * nsplit + split) * (kAD + 2);
      out[j] = acc[g] + accx[g][j];
      if (j == 0) {
        out[kAD] = mx[g];
        out[kAD + 1] = sm[g];
      }
    }
  }
}

__global__ __launch_bounds__(kAD) void decode_combine_kernel(const float* __restrict__ rot,
                                                             const float* __restrict__ partials,
                                                             int nsplit, float* __restrict__ out) {
  __shared__ float a[kAD];
  const int64_t h = blockIdx.x;
  const int j = threadIdx.x;
  const float* p = partials + h * nsplit * (kAD + 2);
  float M = -INFINITY;
  for (int sidx = 0; sidx < nsplit; ++sidx) M = fmaxf(M, p[sidx * (kAD + 2) + kAD]);
  float Lsum = 0.f, acc = 0.f;
  for (int sidx = 0; sidx < nsplit; ++sidx) {
    const float* q = p + sidx * (kAD + 2);
    const float w = expf(q[kAD] - M);
    Lsum = fmaf(q[kAD + 1], w, Lsum);
    acc = fmaf(q[j], w, acc);
  }
  a[j] = acc / Lsum;
  __syncthreads();
  // out_k = sum_j Pi[j][k] a_j  (Pi^T a)
  float o = 0.f;
  for (int jj = 0; jj < kAD; ++jj) o = fmaf(rot[jj * kAD + j], a[jj], o);
  out[h * kAD + j] = o;
}

hipError_t launch_decode(const tq_tables& tk, const tq_tables& tv, const float* qr, const float* u,
                         int B, int Hq, int Hkv, const tq_packed& k, const tq_packed& v,
                         float scale, float* partials, float* out, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int nsplit = decode_splits(k.T);
  dim3 grid(static_cast<unsigned>(nsplit), static_cast<unsigned>(B * Hkv));
#define TQ_DLAUNCH(GV)                                                                         \
  hipLaunchKernelGGL(decode_partial_kernel<GV>, grid, dim3(kDThreads), 0, stream,             \
                     tk.centroids, tk.bits, tk.m, tv.centroids, tv.bits, qr, u, k.T, k.codes,  \
                     k.signs, k.norm, k.rnorm, k.norm_dtype, v.codes, v.norm, v.norm_dtype,    \
                     scale, nsplit, partials)
  switch (G) {
    case 1: TQ_DLAUNCH(1); break;
    case 2: TQ_DLAUNCH(2); break;
    case 4: TQ_DLAUNCH(4); break;
    case 8: TQ_DLAUNCH(8); break;
    default: return hipErrorInvalidValue;
  }
#undef TQ_DLAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(B * Hq), dim3(kAD), 0, stream, tk.rot, partials,
                     nsplit, out);
  return hipGetLastError();
}

}  // namespace tq
