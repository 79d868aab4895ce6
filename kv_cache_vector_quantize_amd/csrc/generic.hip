// Quantize, query preparation and (16 query heads per KV head) logits at
// head dimensions other than the matrix-core kernels' 128 (any d <= 256,
// sketch rows m <= 256): the vector search workload of the pages runs at
// d = 200 (a2a-mcp.org page, "Benchmarks": GloVe vectors, judged by the
// top-k recall of the estimated inner products).  Logits for up to 8 query
// heads per KV head run on the matrix-core tiles (logits_wide_kernel).
//
// Same method as the d = 128 kernels (a2a-mcp.org page, "How it works",
// Stages 1 and 2): normalise, rotate, count the codebook boundaries at or
// below each rotated coordinate, and for keys take the signs of the sketch
// of the residual.  These run on the vector ALU with float64 accumulation
// (products of float32 table entries and exact inputs): database
// quantization is set-up for search.
//
// Layout as at d = 128 with d and m padded to whole 32-bit words: key
// codes[s][Tp][ceil(d/32)][bits], signs[s][Tp][ceil(m/32)], value
// codes[s][Tp/32][d][bits]; bits of padding coordinates and sketch rows are
// zero.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace tq {

constexpr int kGMax = 256;        // largest d and m of these kernels
constexpr int kGThreads = 256;
constexpr int kGUnit = 32;        // tokens per block of work (the stream's block)
constexpr int kGRow = kGMax + 1;  // LDS row stride in floats (rows start in different banks)

// One workgroup per 32-token block of one sequence, grid-striding.  Thread
// (tt, part) = (tid / 8, tid % 8) owns token tt: the rows part*4 .. part*4+3
// of every 32-row tile of Pi or S, and (keys) coordinate word `part`.
template <typename XT>
__global__ __launch_bounds__(kGThreads) void quantize_generic_kernel(
    int d, int m, int bits, const float* __restrict__ rot, const float* __restrict__ sketch,
    const float* __restrict__ cent, const float* __restrict__ bnd, const XT* __restrict__ x, int64_t nseq,
    int64_t T, int64_t Tp, uint32_t* __restrict__ codes, uint32_t* __restrict__ signs,
    void* __restrict__ norm, void* __restrict__ rnorm, int norm_dtype) {
  __shared__ float xs[kGUnit][kGRow];      // the block's inputs
  __shared__ double ys[kGUnit][kGMax];     // rotated and normalised; keys: then the residual
  __shared__ float tile[kGUnit][kGRow];    // 32 rows of Pi or S
  __shared__ double nrm_s[kGUnit];
  __shared__ double cb[16], bb[16];

  const int tid = threadIdx.x, tt = tid >> 3, part = tid & 7;
  const int L = 1 << bits;
  if (tid < L) cb[tid] = cent[tid];
  if (tid < L - 1) bb[tid] = bnd[tid];
  const bool key = m > 0;
  const int W = (d + 31) / 32, MW = (m + 31) / 32;
  const int64_t nblk = (T + kGUnit - 1) / kGUnit;
  const int64_t units = nseq * nblk;

  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int64_t s = unit / nblk, blk = unit % nblk, t0 = blk * kGUnit;
    __syncthreads();   // the previous unit's LDS reads are done
    for (int e = tid; e < kGUnit * d; e += kGThreads) {
      const int t = e / d, k = e - t * d;
      xs[t][k] = (t0 + t < T) ? load_elem<XT>(x, (s * T + t0 + t) * d + k) : 0.f;   // padding: zero vectors
    }
    __syncthreads();
    {
      double ss = 0.0;
      for (int k = part; k < d; k += 8) {
        const double v = xs[tt][k];
        ss = fma(v, v, ss);
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) ss += __shfl_xor(ss, o, 64);
      if (part == 0) nrm_s[tt] = sqrt(ss);
    }
    __syncthreads();
    const double nr = nrm_s[tt];
    const double inv = nr > 0.0 ? 1.0 / nr : 0.0;
    // ---- y^ = Pi x / ||x||, 32 rows of Pi at a time
    for (int j0 = 0; j0 < d; j0 += 32) {
      for (int e = tid; e < 32 * d; e += kGThreads) {
        const int r = e / d, k = e - r * d;
        tile[r][k] = (j0 + r < d) ? rot[static_cast<int64_t>(j0 + r) * d + k] : 0.f;
      }
      __syncthreads();
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      for (int k = 0; k < d; ++k) {
        const double xv = xs[tt][k];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fma(static_cast<double>(tile[4 * part + i][k]), xv, acc[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * part + i;
        if (j < d) ys[tt][j] = acc[i] * inv;
      }
      __syncthreads();
    }
    auto index_of = [&](double y) {
      int idx = 0;
      for (int i = 0; i < L - 1; ++i) idx += (y >= bb[i]) ? 1 : 0;
      return idx;
    };
    if (key) {
      // ---- codes of word `part` of token tt, residual in place, ||r||^2
      double rr = 0.0;
      for (int w = part; w < W; w += 8) {
        uint32_t pl[4] = {0u, 0u, 0u, 0u};
        for (int b = 0; b < 32; ++b) {
          const int j = 32 * w + b;
          if (j >= d) break;
          int idx;
          double r;
          if (nr > 0.0) {
            const double y = ys[tt][j];
            idx = index_of(y);
            r = y - cb[idx];
          } else {   // a zero vector: the cell just above 0, no residual
            idx = L / 2;
            r = 0.0;
          }
          ys[tt][j] = r;
          rr = fma(r, r, rr);
          for (int p = 0; p < bits; ++p) pl[p] |= ((static_cast<uint32_t>(idx) >> p) & 1u) << b;
        }
        uint32_t* dst = codes + ((s * Tp + t0 + tt) * W + w) * bits;
        for (int p = 0; p < bits; ++p) dst[p] = pl[p];
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) rr += __shfl_xor(rr, o, 64);
      if (part == 0) {
        store_norm(norm, norm_dtype, s * Tp + t0 + tt, static_cast<float>(nr));
        store_norm(rnorm, norm_dtype, s * Tp + t0 + tt, static_cast<float>(nr * sqrt(rr)));
      }
      __syncthreads();
      // ---- z = S r, 32 sketch rows (one sign word) at a time
      for (int i0 = 0; i0 < m; i0 += 32) {
        for (int e = tid; e < 32 * d; e += kGThreads) {
          const int r = e / d, k = e - r * d;
          tile[r][k] = (i0 + r < m) ? sketch[static_cast<int64_t>(i0 + r) * d + k] : 0.f;
        }
        __syncthreads();
        double z[4] = {0.0, 0.0, 0.0, 0.0};
        for (int k = 0; k < d; ++k) {
          const double rv = ys[tt][k];
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] = fma(static_cast<double>(tile[4 * part + i][k]), rv, z[i]);
        }
        uint32_t word = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i0 + 4 * part + i < m && z[i] >= 0.0) word |= 1u << (4 * part + i);   // sign(0) = +1
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) word |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(word), o, 64));
        if (part == 0) signs[(s * Tp + t0 + tt) * MW + i0 / 32] = word;
        __syncthreads();
      }
    } else {
      // ---- values: the record of coordinate j holds its 32 tokens' fields
      // in token order (field t at record bits [bits t, bits t + bits))
      for (int j = tid; j < d; j += kGThreads) {
        uint32_t rec[4] = {0u, 0u, 0u, 0u};
        for (int t = 0; t < kGUnit; ++t) {
          if (t0 + t >= T) break;   // padding tokens keep fields 0
          const int idx = nrm_s[t] > 0.0 ? index_of(ys[t][j]) : L / 2;
          const int pos = bits * t;
          rec[pos >> 5] |= static_cast<uint32_t>(idx) << (pos & 31);
          if ((pos & 31) + bits > 32) rec[(pos >> 5) + 1] |= static_cast<uint32_t>(idx) >> (32 - (pos & 31));
        }
        uint32_t* dst = codes + ((s * (Tp / kGUnit) + blk) * d + j) * bits;
        for (int q = 0; q < bits; ++q) dst[q] = rec[q];
      }
      if (tid < kGUnit && t0 + tid < Tp)
        store_norm(norm, norm_dtype, s * Tp + t0 + tid, (t0 + tid < T) ? static_cast<float>(nrm_s[tid]) : 0.f);
    }
  }
}

// q' = Pi q and u = S q' (float64 sums).  Workgroup (h, rb) computes the
// whole q' of query head h and rows 64 rb .. 64 rb + 63 of its u: thread
// (r, part) = (tid / 8, tid % 8) takes row r of a group of 64 rows and the
// row's entries part, part + 8, ... (the 8 threads of a row read 32
// consecutive bytes per load), three shuffles sum the eighths.  Two groups
// of 64 rows are loaded per round (two rounds up to d = 256).  Workgroup
// rb = 0 writes q'.
constexpr int kQGThreads = 512;

template <typename QT>
__global__ __launch_bounds__(kQGThreads) void qprep_generic_kernel(int d, int m, const float* __restrict__ rot,
                                                                 const float* __restrict__ sketch,
                                                                 const QT* __restrict__ q, float* __restrict__ qr,
                                                                 float* __restrict__ u) {
  __shared__ double qs[kGMax], qrs[kGMax];
  const int64_t h = blockIdx.x;
  const int rb = blockIdx.y;
  const int tid = threadIdx.x, r = tid >> 3, part = tid & 7;
  for (int k = tid; k < d; k += kQGThreads) qs[k] = load_elem<QT>(q, h * d + k);
  __syncthreads();
  // every load of a row's eighth is issued before the sums (at most 32 per
  // thread), unconditionally from a clamped index and masked afterwards: a
  // load under a condition becomes a branch that waits for it, and the L2
  // latency would be paid once per product
  auto load_part = [&](const float* row, float (&w)[32]) {
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int k = part + 8 * t;
      const float x = row[k < d ? k : d - 1];
      w[t] = k < d ? x : 0.f;
    }
  };
  auto part_dot = [&](const float (&w)[32], const double* v) {
    double a = 0.0;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int k = part + 8 * t;
      a = fma(static_cast<double>(w[t]), v[k < d ? k : 0], a);
    }
    a += __shfl_xor(a, 1, 8);
    a += __shfl_xor(a, 2, 8);
    a += __shfl_xor(a, 4, 8);
    return a;
  };
  for (int j0 = 0; j0 < d; j0 += 128) {   // two groups of 64 rows in flight
    const int ja = j0 + r, jb = j0 + 64 + r;
    float wa[32], wb[32];
    load_part(rot + static_cast<int64_t>(ja < d ? ja : 0) * d, wa);
    load_part(rot + static_cast<int64_t>(jb < d ? jb : 0) * d, wb);
    const double a = part_dot(wa, qs), b = part_dot(wb, qs);
    if (part == 0 && ja < d) {
      qrs[ja] = a;
      if (rb == 0) qr[h * d + ja] = static_cast<float>(a);
    }
    if (part == 0 && jb < d) {
      qrs[jb] = b;
      if (rb == 0) qr[h * d + jb] = static_cast<float>(b);
    }
  }
  if (m == 0) return;   // no sketch (uniform)
  __syncthreads();
  const int i = 64 * rb + r;
  float wi[32];
  load_part(sketch + static_cast<int64_t>(i < m ? i : 0) * d, wi);
  const double a = part_dot(wi, qrs);
  if (part == 0 && i < m) u[h * m + i] = static_cast<float>(a);
}

// Raw logits of the G query heads that share KV head s (blockIdx.y), one
// token per thread:
//   l = ||k|| <q', c[idx]> + sqrt(pi/2)/m ||k|| ||r|| <u, 2 s - 1>.
template <int G, int BITS>
__global__ __launch_bounds__(kGThreads) void logits_generic_kernel(
    int d, int m, const float* __restrict__ qr, const float* __restrict__ u, const float* __restrict__ cent,
    int64_t T, int64_t Tp, const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs,
    const void* knorm, const void* krnorm, int norm_dtype, float fu, float* __restrict__ out) {
  __shared__ float q_s[G][kGMax], u_s[G][kGMax];
  __shared__ float cb[1 << BITS];
  const int64_t s = blockIdx.y;
  const int tid = threadIdx.x;
  for (int e = tid; e < G * d; e += kGThreads) q_s[e / d][e % d] = qr[(s * G + e / d) * d + e % d];
  for (int e = tid; e < G * m; e += kGThreads) u_s[e / m][e % m] = u[(s * G + e / m) * m + e % m];
  if (tid < (1 << BITS)) cb[tid] = cent[tid];
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kGThreads + tid;
  if (t >= T) return;
  const int W = (d + 31) / 32, MW = (m + 31) / 32;
  float cen[G], qj[G];
#pragma unroll
  for (int g = 0; g < G; ++g) cen[g] = qj[g] = 0.f;
  const uint32_t* cw = codes + (s * Tp + t) * W * BITS;
  for (int w = 0; w < W; ++w) {
    uint32_t pl[BITS];
#pragma unroll
    for (int p = 0; p < BITS; ++p) pl[p] = cw[w * BITS + p];
    const int nb = (d - 32 * w) < 32 ? d - 32 * w : 32;
    for (int b = 0; b < nb; ++b) {
      uint32_t idx = 0;
#pragma unroll
      for (int p = 0; p < BITS; ++p) idx |= ((pl[p] >> b) & 1u) << p;
      const float c = cb[idx];
#pragma unroll
      for (int g = 0; g < G; ++g) cen[g] = fmaf(q_s[g][32 * w + b], c, cen[g]);
    }
  }
  const uint32_t* sp = signs + (s * Tp + t) * MW;
  for (int w = 0; w < MW; ++w) {
    const uint32_t sw = sp[w];
    const int nb = (m - 32 * w) < 32 ? m - 32 * w : 32;
    for (int b = 0; b < nb; ++b) {
      const float sg = ((sw >> b) & 1u) ? 1.f : -1.f;
#pragma unroll
      for (int g = 0; g < G; ++g) qj[g] = fmaf(u_s[g][32 * w + b], sg, qj[g]);
    }
  }
  const float nk = load_norm(knorm, norm_dtype, s * Tp + t);
  const float nrr = load_norm(krnorm, norm_dtype, s * Tp + t);
#pragma unroll
  for (int g = 0; g < G; ++g) out[(s * G + g) * T + t] = fmaf(nk, cen[g], fu * nrr * qj[g]);
}

static int generic_grid(int64_t units) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return static_cast<int>(units < cus ? units : cus);   // one 130 KB workgroup per CU
}

hipError_t launch_quantize_generic(const tq_tables& t, const void* x, int x_dtype, const tq_packed& out,
                                   hipStream_t stream) {
  const int64_t units = out.nseq * ((out.T + kGUnit - 1) / kGUnit);
  if (units == 0) return hipSuccess;
  const dim3 grid(generic_grid(units));
  const int m = out.role == TQ_KEY ? t.m : 0;
  if (x_dtype == TQ_BF16)
    hipLaunchKernelGGL(quantize_generic_kernel<uint16_t>, grid, dim3(kGThreads), 0, stream, t.d, m, t.bits,
                       t.rot, t.sketch, t.centroids, t.bounds, static_cast<const uint16_t*>(x), out.nseq, out.T,
                       stream_stride(out), out.codes, out.signs, out.norm, out.rnorm, out.norm_dtype);
  else
    hipLaunchKernelGGL(quantize_generic_kernel<float>, grid, dim3(kGThreads), 0, stream, t.d, m, t.bits, t.rot,
                       t.sketch, t.centroids, t.bounds, static_cast<const float*>(x), out.nseq, out.T,
                       stream_stride(out), out.codes, out.signs, out.norm, out.rnorm, out.norm_dtype);
  return hipGetLastError();
}

hipError_t launch_qprep_generic(const tq_tables& tk, const void* q, int q_dtype, int nh, float* qr, float* u,
                                hipStream_t stream) {
  if (nh == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nh), static_cast<unsigned>(tk.m > 0 ? (tk.m + 63) / 64 : 1));
  if (q_dtype == TQ_BF16)
    hipLaunchKernelGGL(qprep_generic_kernel<uint16_t>, grid, dim3(kQGThreads), 0, stream, tk.d, tk.m, tk.rot,
                       tk.sketch, static_cast<const uint16_t*>(q), qr, u);
  else
    hipLaunchKernelGGL(qprep_generic_kernel<float>, grid, dim3(kQGThreads), 0, stream, tk.d, tk.m, tk.rot,
                       tk.sketch, static_cast<const float*>(q), qr, u);
  return hipGetLastError();
}

template <int G>
static void launch_logits_generic_g(dim3 grid, hipStream_t stream, const tq_tables& tk, const float* qr,
                                    const float* u, const tq_packed& k, float fu, float* out) {
#define TQ_LG(BV)                                                                                      \
  hipLaunchKernelGGL((logits_generic_kernel<G, BV>), grid, dim3(kGThreads), 0, stream, tk.d, tk.m, qr, u,    \
                     tk.centroids, k.T, stream_stride(k), k.codes, k.signs, k.norm, k.rnorm, k.norm_dtype, fu, \
                     out)
  switch (tk.bits) {
    case 1: TQ_LG(1); break;
    case 2: TQ_LG(2); break;
    case 3: TQ_LG(3); break;
    default: TQ_LG(4); break;
  }
#undef TQ_LG
}

hipError_t launch_logits_generic(const tq_tables& tk, const float* qr, const float* u, int B, int Hq, int Hkv,
                                 const tq_packed& k, float* logits, hipStream_t stream) {
  if (B == 0 || k.T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((k.T + kGThreads - 1) / kGThreads), static_cast<unsigned>(k.nseq));
  const float fu = 1.2533141373155003f / static_cast<float>(tk.m);   // sqrt(pi/2) / m
  switch (Hq / Hkv) {
    case 1: launch_logits_generic_g<1>(grid, stream, tk, qr, u, k, fu, logits); break;
    case 2: launch_logits_generic_g<2>(grid, stream, tk, qr, u, k, fu, logits); break;
    case 4: launch_logits_generic_g<4>(grid, stream, tk, qr, u, k, fu, logits); break;
    case 8: launch_logits_generic_g<8>(grid, stream, tk, qr, u, k, fu, logits); break;
    default: launch_logits_generic_g<16>(grid, stream, tk, qr, u, k, fu, logits); break;
  }
  return hipGetLastError();
}

}  // namespace tq
