// Decode attention straight from the packed codes, on the matrix cores.
//
// Method (a2a-mcp.org page, Stage 2 closing paragraph; "How to implement",
// item 1): the query is rotated once (q' = Pi q, u = S q'), every logit is
//   l_t = ||k_t|| <q', c_K[idx_t]> + sqrt(pi/2)/m ||k_t|| ||r_t|| <u, 2 s_t - 1>,
// a = softmax(scale * l), and the values are summed in the rotated domain,
// acc = sum_t a_t ||v_t|| c_V[idxV_t]; out = Pi^T acc happens once, in the
// combine kernel.  No pass dequantizes the cache to memory.
//
// Mapping onto gfx950 (wave64, v_mfma_f32_16x16x32_f16):
//  * one workgroup = 4 waves = one split of up to 1024 tokens of one KV head;
//    every wave owns 32-token blocks blk = wave, wave+4, ... and keeps its
//    own online-softmax state; the 4 states are merged through LDS.
//  * logits, per 16-token tile: A = centroid values of 16 tokens x 32
//    coordinates (looked up from a 16/64/256-entry LDS table by the 2b-bit
//    index of a coordinate pair, as an fp16 hi/lo pair), B = the rotated
//    queries of the G heads, fp16 hi in columns [0,G) and lo in [G,2G).
//    Two MFMAs (A_hi, A_lo) per 32 coordinates give fp32-grade dots.  The
//    1-bit correction is the same contraction with A = +-1 and B = u hi/lo.
//  * tile rows are ordered so that after the two tiles of a block every lane
//    group g4 = lane/16 holds the logits of tokens 8*g4 .. 8*g4+7, which is
//    exactly the K-slice its lanes feed to the value MFMA.
//  * values: A = softmax weights (rows = heads, fp16, p <= 2^8 by a lazily
//    updated reference max), B = value centroids of 32 tokens x 16
//    coordinates from a pair table, times ||v|| (packed fp16 multiply).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kDD = 128;
constexpr int kDecThreads = 256;
constexpr int kSplit = 1024;     // tokens per workgroup
constexpr float kTau = 8.0f;     // rescale when a block max exceeds the reference by 2^8

__device__ __forceinline__ uint32_t h2u(_Float16 lo, _Float16 hi) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
}

__device__ __forceinline__ half8 u4_to_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ uint32_t pk_mul_h2(uint32_t a, uint32_t b) {
  half2_t x = __builtin_bit_cast(half2_t, a), y = __builtin_bit_cast(half2_t, b);
  return __builtin_bit_cast(uint32_t, x * y);
}

// 2b-bit index of the coordinate pair (2m, 2m+1) of one 32-coordinate word:
// bit 2p = plane p of the lower coordinate, bit 2p+1 = plane p of the upper.
template <int KB>
__device__ __forceinline__ uint32_t pair_index(const uint32_t* p, int m) {
  uint32_t x = 0;
#pragma unroll
  for (int q = 0; q < KB; ++q) x |= ((p[q] >> (2 * m)) & 3u) << (2 * q);
  return x;
}

template <int G, int KB, int VB>
__global__ __launch_bounds__(kDecThreads, 2) void decode_mfma_kernel(
    const float* __restrict__ ck, const float* __restrict__ cv, const float* __restrict__ qr,
    const float* __restrict__ u, int64_t T, const uint32_t* __restrict__ kcodes,
    const uint32_t* __restrict__ ksigns, const void* knorm, const void* krnorm, int knd,
    const uint32_t* __restrict__ vcodes, const void* vnorm, int vnd, float scale_log2,
    int nsplit, float* __restrict__ partials) {
  constexpr int KL = 1 << (2 * KB);
  constexpr int VL = 1 << (2 * VB);
  __shared__ uint2 klut[KL];
  __shared__ uint32_t slut[4];
  __shared__ uint32_t vlut[VL];
  __shared__ float nk_s[kSplit], rnq_s[kSplit];
  __shared__ __align__(16) _Float16 nv_s[kSplit];
  __shared__ float m_s[4][16], l_s[4][16];
  __shared__ float o_s[4][G][kDD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int64_t h0 = s * G;
  const int64_t t0 = static_cast<int64_t>(split) * kSplit;
  const int64_t t1 = (t0 + kSplit < T) ? t0 + kSplit : T;
  const int ntok = static_cast<int>(t1 - t0);
  const float qjl = sqrtf(static_cast<float>(M_PI) / 2.f) / 128.f;

  // --- tables and the split's norms
  for (int x = tid; x < KL; x += kDecThreads) {
    int ia = 0, ib = 0;
    for (int q = 0; q < KB; ++q) {
      ia |= ((x >> (2 * q)) & 1) << q;
      ib |= ((x >> (2 * q + 1)) & 1) << q;
    }
    const float ca = ck[ia], cb = ck[ib];
    const _Float16 ha = static_cast<_Float16>(ca), hb = static_cast<_Float16>(cb);
    const _Float16 la = static_cast<_Float16>(ca - static_cast<float>(ha));
    const _Float16 lb = static_cast<_Float16>(cb - static_cast<float>(hb));
    klut[x] = make_uint2(h2u(ha, hb), h2u(la, lb));
  }
  if (tid < 4)
    slut[tid] = h2u(static_cast<_Float16>((tid & 1) ? 1.f : -1.f),
                    static_cast<_Float16>((tid & 2) ? 1.f : -1.f));
  for (int x = tid; x < VL; x += kDecThreads)
    vlut[x] = h2u(static_cast<_Float16>(cv[x & ((1 << VB) - 1)]), static_cast<_Float16>(cv[x >> VB]));
  for (int i = tid; i < kSplit; i += kDecThreads) {
    if (i < ntok) {
      const int64_t rec = s * T + t0 + i;
      nk_s[i] = load_norm(knorm, knd, rec);
      rnq_s[i] = qjl * load_norm(krnorm, knd, rec);
      nv_s[i] = static_cast<_Float16>(load_norm(vnorm, vnd, rec));
    } else {
      nk_s[i] = 0.f;
      rnq_s[i] = 0.f;
      nv_s[i] = static_cast<_Float16>(0.f);
    }
  }

  // --- B operands: rotated queries (and u), fp16 hi in columns [0,G), lo in [G,2G)
  half8 bq[4], bu[4];
  {
    const bool hi_col = n < G, lo_col = (n >= G) && (n < 2 * G);
    const int g = hi_col ? n : (lo_col ? n - G : 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = 32 * g4 + 8 * c + i;
        _Float16 vq = static_cast<_Float16>(0.f), vu = static_cast<_Float16>(0.f);
        if (hi_col || lo_col) {
          const float xq = qr[(h0 + g) * kDD + j], xu = u[(h0 + g) * kDD + j];
          const _Float16 hq = static_cast<_Float16>(xq), hu = static_cast<_Float16>(xu);
          vq = hi_col ? hq : static_cast<_Float16>(xq - static_cast<float>(hq));
          vu = hi_col ? hu : static_cast<_Float16>(xu - static_cast<float>(hu));
        }
        bq[c][i] = vq;
        bu[c][i] = vu;
      }
    }
  }
  __syncthreads();

  floatx4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, lsum = 0.f;
  const int64_t nblk = (T + 31) / 32;
  const int nb_split = (ntok + 31) / 32;

  for (int bb = wave; bb < nb_split; bb += 4) {
    const int64_t blk = t0 / 32 + bb;
    // ---------------- logits of the block's 32 tokens
    float sv[8];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const int tok = 8 * (n >> 2) + (n & 3) + 4 * tile;   // token of A-row n
      const int64_t t = blk * 32 + tok;
      const int64_t tl = (t < T) ? t : T - 1;               // clamped for the loads
      const uint32_t* kw = kcodes + ((s * T + tl) * 4 + g4) * KB;
      uint32_t pw[KB];
#pragma unroll
      for (int q = 0; q < KB; ++q) pw[q] = kw[q];
      const uint32_t sw = ksigns[(s * T + tl) * 4 + g4];
      floatx4 accC = {0.f, 0.f, 0.f, 0.f}, accS = {0.f, 0.f, 0.f, 0.f};
      uint32_t E = 0, Od = 0;
      if constexpr (KB == 2) {
        E = (pw[0] & 0x33333333u) | ((pw[1] << 2) & 0xCCCCCCCCu);
        Od = ((pw[0] >> 2) & 0x33333333u) | (pw[1] & 0xCCCCCCCCu);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t ahi[4], alo[4], as[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t x;
          if constexpr (KB == 2) {
            const uint32_t src = (q & 1) ? Od : E;
            x = (src >> (8 * c + 4 * (q >> 1))) & 15u;
          } else {
            x = pair_index<KB>(pw, 4 * c + q);
          }
          const uint2 e = klut[x];
          ahi[q] = e.x;
          alo[q] = e.y;
          as[q] = slut[(sw >> (8 * c + 2 * q)) & 3u];
        }
        accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(ahi[0], ahi[1], ahi[2], ahi[3]), bq[c], accC, 0, 0, 0);
        accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(alo[0], alo[1], alo[2], alo[3]), bq[c], accC, 0, 0, 0);
        accS = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(as[0], as[1], as[2], as[3]), bu[c], accS, 0, 0, 0);
      }
      // column n < G gets its lo partner from column n + G
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float cen = accC[i] + __shfl_down(accC[i], G, 16);
        const float qj = accS[i] + __shfl_down(accS[i], G, 16);
        const int tk = 8 * g4 + 4 * tile + i;             // token of output row 4*g4 + i
        const int li = static_cast<int>(blk * 32 - t0) + tk;
        const bool ok = (n < G) && (blk * 32 + tk < T);
        const float l = nk_s[ok ? li : 0] * cen + rnq_s[ok ? li : 0] * qj;
        sv[4 * tile + i] = ok ? l * scale_log2 : -INFINITY;
      }
    }
    // ---------------- online softmax (reference max updated lazily)
    float bm = sv[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) bm = fmaxf(bm, sv[k]);
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    if (__ballot(bm > m_ref + kTau)) {
      const float m_new = fmaxf(m_ref, bm);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_ref - m_new);
      lsum *= alpha;
      m_ref = m_new;
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * g4 + i);
        a4[i] = (4 * g4 + i < G) ? ai : 1.f;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) O[nt][i] *= a4[i];
      }
    }
    half8 pa;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = exp2f(sv[k] - m_ref);                // 0 for masked tokens / rows
      lsum += (n < G) ? p : 0.f;
      pa[k] = static_cast<_Float16>((n < G) ? p : 0.f);
    }
    // ---------------- values: B = ||v|| * c_V[idx] for tokens 8*g4 .. 8*g4+7
    const int lbase = static_cast<int>(blk * 32 - t0) + 8 * g4;
    const uint4 nvq = *reinterpret_cast<const uint4*>(&nv_s[lbase]);
    const uint32_t nvp[4] = {nvq.x, nvq.y, nvq.z, nvq.w};
    constexpr int kBitsPerGroup = 8 * VB;
    const int bit0 = kBitsPerGroup * g4;
    const int wlo = bit0 >> 5, sh = bit0 & 31;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int j = 16 * nt + n;
      const uint32_t* vw = vcodes + ((s * nblk + blk) * kDD + j) * VB;
      uint32_t rw[VB];
#pragma unroll
      for (int q = 0; q < VB; ++q) rw[q] = vw[q];
      uint32_t lo = rw[0], hi = (VB > 1) ? rw[VB > 1 ? 1 : 0] : 0u;
#pragma unroll
      for (int q = 1; q < VB; ++q) {
        if (wlo == q) {
          lo = rw[q];
          hi = (q + 1 < VB) ? rw[q + 1 < VB ? q + 1 : q] : 0u;
        }
      }
      const uint32_t X = (sh == 0) ? lo : __builtin_amdgcn_alignbit(hi, lo, sh);
      uint32_t bw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x = (X >> (2 * VB * q)) & (VL - 1);
        bw[q] = pk_mul_h2(vlut[x], nvp[q]);
      }
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, u4_to_h8(bw[0], bw[1], bw[2], bw[3]), O[nt], 0, 0, 0);
    }
  }

  // ---------------- merge the 4 waves' states, write this split's partial
  float ltot = lsum;
  ltot += __shfl_xor(ltot, 16);
  ltot += __shfl_xor(ltot, 32);
  if (g4 == 0) {
    m_s[wave][n] = m_ref;
    l_s[wave][n] = ltot;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * g4 + i;
      if (g < G) o_s[wave][g][16 * nt + n] = O[nt][i];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kDD; e += kDecThreads) {
    const int g = e / kDD, j = e % kDD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, m_s[w][g]);
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (m_s[w][g] == -INFINITY) ? 0.f : exp2f(m_s[w][g] - M);
      acc += f * o_s[w][g][j];
      L += f * l_s[w][g];
    }
    float* out = partials + ((h0 + g) * nsplit + split) * (kDD + 2);
    out[j] = acc;
    if (j == 0) {
      out[kDD] = M;
      out[kDD + 1] = L;
    }
  }
}

// Merge the splits by log-sum-exp (log2 units) and rotate back once.
__global__ __launch_bounds__(kDD) void decode_combine_kernel(const float* __restrict__ rot,
                                                             const float* __restrict__ partials,
                                                             int nsplit, float* __restrict__ out) {
  __shared__ float a[kDD];
  const int64_t h = blockIdx.x;
  const int j = threadIdx.x;
  const float* p = partials + h * nsplit * (kDD + 2);
  float M = -INFINITY;
  for (int sidx = 0; sidx < nsplit; ++sidx) M = fmaxf(M, p[sidx * (kDD + 2) + kDD]);
  float Lsum = 0.f, acc = 0.f;
  for (int sidx = 0; sidx < nsplit; ++sidx) {
    const float* q = p + sidx * (kDD + 2);
    const float w = exp2f(q[kDD] - M);
    Lsum = fmaf(q[kDD + 1], w, Lsum);
    acc = fmaf(q[j], w, acc);
  }
  a[j] = acc / Lsum;
  __syncthreads();
  float o = 0.f;
  for (int jj = 0; jj < kDD; ++jj) o = fmaf(rot[jj * kDD + j], a[jj], o);  // (Pi^T a)_j
  out[h * kDD + j] = o;
}

int decode_splits(int64_t T) { return static_cast<int>((T + kSplit - 1) / kSplit); }

template <int G, int KB>
static void launch_vb(int vb, dim3 grid, hipStream_t stream, const tq_tables& tk,
                      const tq_tables& tv, const float* qr, const float* u, const tq_packed& k,
                      const tq_packed& v, float sl2, int nsplit, float* partials) {
#define TQ_DEC(VBV)                                                                              \
  hipLaunchKernelGGL((decode_mfma_kernel<G, KB, VBV>), grid, dim3(kDecThreads), 0, stream,       \
                     tk.centroids, tv.centroids, qr, u, k.T, k.codes, k.signs, k.norm, k.rnorm, \
                     k.norm_dtype, v.codes, v.norm, v.norm_dtype, sl2, nsplit, partials)
  switch (vb) {
    case 1: TQ_DEC(1); break;
    case 2: TQ_DEC(2); break;
    case 3: TQ_DEC(3); break;
    default: TQ_DEC(4); break;
  }
#undef TQ_DEC
}

template <int G>
static void launch_kb(int kb, int vb, dim3 grid, hipStream_t stream, const tq_tables& tk,
                      const tq_tables& tv, const float* qr, const float* u, const tq_packed& k,
                      const tq_packed& v, float sl2, int nsplit, float* partials) {
  switch (kb) {
    case 1: launch_vb<G, 1>(vb, grid, stream, tk, tv, qr, u, k, v, sl2, nsplit, partials); break;
    case 2: launch_vb<G, 2>(vb, grid, stream, tk, tv, qr, u, k, v, sl2, nsplit, partials); break;
    case 3: launch_vb<G, 3>(vb, grid, stream, tk, tv, qr, u, k, v, sl2, nsplit, partials); break;
    default: launch_vb<G, 4>(vb, grid, stream, tk, tv, qr, u, k, v, sl2, nsplit, partials); break;
  }
}

hipError_t launch_decode(const tq_tables& tk, const tq_tables& tv, const float* qr, const float* u,
                         int B, int Hq, int Hkv, const tq_packed& k, const tq_packed& v,
                         float scale, float* partials, float* out, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int nsplit = decode_splits(k.T);
  const float sl2 = scale * 1.4426950408889634f;  // softmax in base 2
  dim3 grid(static_cast<unsigned>(nsplit), static_cast<unsigned>(B * Hkv));
  switch (G) {
    case 1: launch_kb<1>(tk.bits, tv.bits, grid, stream, tk, tv, qr, u, k, v, sl2, nsplit, partials); break;
    case 2: launch_kb<2>(tk.bits, tv.bits, grid, stream, tk, tv, qr, u, k, v, sl2, nsplit, partials); break;
    case 4: launch_kb<4>(tk.bits, tv.bits, grid, stream, tk, tv, qr, u, k, v, sl2, nsplit, partials); break;
    case 8: launch_kb<8>(tk.bits, tv.bits, grid, stream, tk, tv, qr, u, k, v, sl2, nsplit, partials); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(B * Hq), dim3(kDD), 0, stream, tk.rot, partials,
                     nsplit, out);
  return hipGetLastError();
}

}  // namespace tq
