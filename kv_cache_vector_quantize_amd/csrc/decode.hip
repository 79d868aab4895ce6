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
//  * decode_prep (one wave per KV head) lays the G rotated queries out as
//    matrix-core B fragments -- fp16 hi in columns [0,G), the fp16 residual
//    in [G,2G) -- and builds the code tables once.
//  * one workgroup = 4 waves = one split of the context of one KV head;
//    wave w owns 32-token blocks w, w+4, ... and keeps its own
//    online-softmax state; the 4 states merge through LDS.
//  * logits, per 16-token tile: A = centroid values of 16 tokens x 32
//    coordinates, looked up from an LDS table by the 2b-bit index of a
//    coordinate pair as an fp16 hi/lo pair; two MFMAs (A_hi, A_lo) against
//    the query fragment give fp32-grade dots.  The 1-bit correction is the
//    same contraction with A = +-1 and B = u.  The hi and lo columns are
//    summed with one DPP row shift.
//  * tile rows are ordered so that after the two tiles of a block, lane group
//    g4 = lane/16 holds the logits of tokens 8*g4 .. 8*g4+7: exactly the
//    K-slice those lanes feed to the value MFMA, so softmax weights never
//    leave registers.
//  * values: A = softmax weight times ||v|| / sigma (rows = heads, fp16;
//    p <= 2^8 thanks to a lazily raised reference max, sigma = the split's
//    largest value norm), B = value centroids of 32 tokens x 16 coordinates
//    from a token-pair table; the merge multiplies sigma back in.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kDD = 128;
constexpr int kDecThreads = 256;
constexpr int kMaxSplit = 2048;   // tokens staged per workgroup (LDS)
constexpr float kTau = 8.0f;      // raise the reference max when a block exceeds it by 2^8
constexpr size_t kLutBytes = 4096;
constexpr int kSLutOff = 2048;    // byte offsets inside the table area
constexpr int kVLutOff = 2064;

__device__ __forceinline__ uint32_t h2u(_Float16 lo, _Float16 hi) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
}

__device__ __forceinline__ half8 u4_to_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

// value of lane (i + SH) within the lane's row of 16 (DPP row_shl); lanes
// whose source falls off the row get 0
template <int SH>
__device__ __forceinline__ float row_shl(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x100 + SH, 0xf, 0xf, false));
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

// ------------------------------------------------------------ preparation
// Per KV head s and lane (n = lane%16, g4 = lane/16), 12 B-fragments of 8 fp16:
//  frag[s][0..7][lane]: centroid K-steps c' = 0..7.  The K slots hold the
//    coordinates 32*g4 + 4c' + {0,1,0,1,2,3,2,3}: every coordinate twice, once
//    against the hi and once against the lo half of its centroid.
//  frag[s][8..11][lane]: sign K-steps c = 0..3, coordinates 32*g4 + 8c + i.
// Columns n < G carry the fp16 value, G <= n < 2G its fp16 residual, the
// rest zero.
constexpr int kFragsPerSeq = 12;

template <int G>
__global__ __launch_bounds__(64) void decode_prep_kernel(const float* __restrict__ qr,
                                                         const float* __restrict__ u, int kb, int vb,
                                                         const float* __restrict__ ck,
                                                         const float* __restrict__ cv,
                                                         uint4* __restrict__ frag,
                                                         char* __restrict__ lut) {
  const int lane = threadIdx.x, n = lane & 15, g4 = lane >> 4;
  const int64_t s = blockIdx.x, h0 = s * G;
  const bool hi_col = n < G, lo_col = (n >= G) && (n < 2 * G);
  const int g = hi_col ? n : (lo_col ? n - G : 0);
  auto part = [&](const float* src, int j) -> _Float16 {
    if (!(hi_col || lo_col)) return static_cast<_Float16>(0.f);
    const float x = src[(h0 + g) * kDD + j];
    const _Float16 a = static_cast<_Float16>(x);
    return hi_col ? a : static_cast<_Float16>(x - static_cast<float>(a));
  };
  constexpr int kSlot[8] = {0, 1, 0, 1, 2, 3, 2, 3};
  for (int c = 0; c < 8; ++c) {
    _Float16 h[8];
    for (int i = 0; i < 8; ++i) h[i] = part(qr, 32 * g4 + 4 * c + kSlot[i]);
    frag[(s * kFragsPerSeq + c) * 64 + lane] =
        make_uint4(h2u(h[0], h[1]), h2u(h[2], h[3]), h2u(h[4], h[5]), h2u(h[6], h[7]));
  }
  for (int c = 0; c < 4; ++c) {
    _Float16 h[8];
    for (int i = 0; i < 8; ++i) h[i] = part(u, 32 * g4 + 8 * c + i);
    frag[(s * kFragsPerSeq + 8 + c) * 64 + lane] =
        make_uint4(h2u(h[0], h[1]), h2u(h[2], h[3]), h2u(h[4], h[5]), h2u(h[6], h[7]));
  }
  if (s != 0) return;
  // key pair table: entry x -> (hi pair, lo pair) of the two coordinates' centroids
  uint2* klut = reinterpret_cast<uint2*>(lut);
  for (int x = lane; x < (1 << (2 * kb)); x += 64) {
    int ia = 0, ib = 0;
    for (int q = 0; q < kb; ++q) {
      ia |= ((x >> (2 * q)) & 1) << q;
      ib |= ((x >> (2 * q + 1)) & 1) << q;
    }
    const float ca = ck[ia], cb = ck[ib];
    const _Float16 ha = static_cast<_Float16>(ca), hb = static_cast<_Float16>(cb);
    klut[x] = make_uint2(h2u(ha, hb), h2u(static_cast<_Float16>(ca - static_cast<float>(ha)),
                                          static_cast<_Float16>(cb - static_cast<float>(hb))));
  }
  uint32_t* slut = reinterpret_cast<uint32_t*>(lut + kSLutOff);
  if (lane < 4)
    slut[lane] = h2u(static_cast<_Float16>((lane & 1) ? 1.f : -1.f),
                     static_cast<_Float16>((lane & 2) ? 1.f : -1.f));
  // value pair table: entry x -> (c[x & mask], c[x >> vb]) for tokens (2q, 2q+1)
  uint32_t* vlut = reinterpret_cast<uint32_t*>(lut + kVLutOff);
  for (int x = lane; x < (1 << (2 * vb)); x += 64)
    vlut[x] = h2u(static_cast<_Float16>(cv[x & ((1 << vb) - 1)]), static_cast<_Float16>(cv[x >> vb]));
}

// ------------------------------------------------------------ the kernel
template <int G, int KB, int VB>
__global__ __launch_bounds__(kDecThreads, 2) void decode_mfma_kernel(
    const uint4* __restrict__ frag, const char* __restrict__ lut, int64_t T, int split_len,
    const uint32_t* __restrict__ kcodes, const uint32_t* __restrict__ ksigns, const void* knorm,
    const void* krnorm, int knd, const uint32_t* __restrict__ vcodes, const void* vnorm, int vnd,
    float sl2, int nsplit, float* __restrict__ partials) {
  constexpr int KL = 1 << (2 * KB);
  constexpr int VL = 1 << (2 * VB);
  // One LDS buffer with a fixed layout: the code tables first (small
  // offsets fold into the ds_read instructions; the hi and lo key tables sit
  // 1 KiB apart so that their reads stay separate and land directly in the
  // matrix-core operand registers), then the staged norms of the split.
  // After the main loop the staging bytes hold the four waves' softmax
  // states for the merge.
  constexpr int kKhi = 0, kKlo = 1024, kSlu = 2048, kVlu = 2064, kStage = 3104;
  constexpr int kStageBytes = kMaxSplit * 12;
  constexpr int kMergeBytes = (2 * 4 * 16 + 4 * G * kDD + 4) * 4;
  constexpr int kRed = kStage + (kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes);
  __shared__ __align__(16) char lds[kRed + 16];
  uint32_t* khi = reinterpret_cast<uint32_t*>(lds + kKhi);
  uint32_t* klo = reinterpret_cast<uint32_t*>(lds + kKlo);
  uint32_t* slut = reinterpret_cast<uint32_t*>(lds + kSlu);
  uint32_t* vlut = reinterpret_cast<uint32_t*>(lds + kVlu);
  float* nk_s = reinterpret_cast<float*>(lds + kStage);   // ||k|| * scale * log2(e)
  float* rq_s = nk_s + kMaxSplit;          // sqrt(pi/2)/m ||k|| ||r|| * scale * log2(e)
  float* nv_s = rq_s + kMaxSplit;          // ||v|| / sigma, sigma = the split's largest ||v||
  float (*m_s)[16] = reinterpret_cast<float (*)[16]>(lds + kStage);
  float (*l_s)[16] = reinterpret_cast<float (*)[16]>(lds + kStage + 4 * 16 * 4);
  float (*o_s)[G][kDD] = reinterpret_cast<float (*)[G][kDD]>(lds + kStage + 2 * 4 * 16 * 4);
  float* red_s = reinterpret_cast<float*>(lds + kRed);   // the 4 waves' largest ||v||

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int64_t h0 = s * G;
  const int t0 = split * split_len;                  // T < 2^28 (checked on the host)
  const int Ti = static_cast<int>(T);
  const int t1 = (t0 + split_len < Ti) ? t0 + split_len : Ti;
  const int ntok = t1 - t0;
  const float qjl = sqrtf(static_cast<float>(M_PI) / 2.f) / 128.f;

  for (int x = tid; x < KL; x += kDecThreads) {
    const uint2 e = reinterpret_cast<const uint2*>(lut)[x];
    khi[x] = e.x;
    klo[x] = e.y;
  }  // visible after the staging barrier below
  if (tid < 4) slut[tid] = reinterpret_cast<const uint32_t*>(lut + kSLutOff)[tid];
  for (int x = tid; x < VL; x += kDecThreads) vlut[x] = reinterpret_cast<const uint32_t*>(lut + kVLutOff)[x];
  float sigma;
  {
    const int64_t rec0 = s * T + t0;
    const int nst = (ntok + 31) & ~31;
    float vmax = 0.f;
    for (int i = tid; i < nst; i += kDecThreads) {
      float a = 0.f, b = 0.f, c = 0.f;
      if (i < ntok) {
        a = load_norm(knorm, knd, rec0 + i);
        b = load_norm(krnorm, knd, rec0 + i);
        c = load_norm(vnorm, vnd, rec0 + i);
      }
      nk_s[i] = a * sl2;
      rq_s[i] = qjl * b * sl2;
      nv_s[i] = c;
      vmax = fmaxf(vmax, c);
    }
    vmax = wave_max(vmax);
    if (lane == 0) red_s[wave] = vmax;
    __syncthreads();
    sigma = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
    if (!(sigma > 0.f)) sigma = 1.f;
    const float inv = 1.f / sigma;
    for (int i = tid; i < nst; i += kDecThreads) nv_s[i] *= inv;
  }
  half8 bq[8], bu[4];
#pragma unroll
  for (int c = 0; c < 8; ++c) bq[c] = __builtin_bit_cast(half8, frag[(s * kFragsPerSeq + c) * 64 + lane]);
#pragma unroll
  for (int c = 0; c < 4; ++c) bu[c] = __builtin_bit_cast(half8, frag[(s * kFragsPerSeq + 8 + c) * 64 + lane]);
  __syncthreads();

  floatx4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // lanes outside the G heads never rescale (their reference stays 0)
  float m_ref = (n < G) ? -INFINITY : 0.f, lsum = 0.f;
  const int nblk = (Ti + 31) / 32;
  const int nb_split = (ntok + 31) / 32;
  const uint32_t* kc_seq = kcodes + s * T * 4 * KB;
  const uint32_t* ks_seq = ksigns + s * T * 4;
  const uint32_t* vc_seq = vcodes + s * nblk * kDD * VB;
  const int rowtok = 8 * (n >> 2) + (n & 3);          // token of A-row n (tile 0)
  const int vbit0 = 8 * VB * g4;                       // this lane group's 8 value fields
  const int vwlo = vbit0 >> 5, vsh = vbit0 & 31;
  const int vwhi = (vwlo + 1 < VB) ? vwlo + 1 : VB - 1;
  const char* khi_b = lds + kKhi;
  const char* klo_b = lds + kKlo;
  const char* slut_b = lds + kSlu;

  // this wave's next block: key plane words and the sign word of both tiles
  uint32_t kw_n[2][KB], sw_n[2];
  auto fetch = [&](int bb) {
    const int tb = t0 + 32 * bb;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      int t = tb + rowtok + 4 * tile;
      t = (t < Ti) ? t : Ti - 1;                       // clamped: tail tokens are masked later
      const uint32_t* kw = kc_seq + static_cast<uint32_t>(t * 4 + g4) * KB;
#pragma unroll
      for (int q = 0; q < KB; ++q) kw_n[tile][q] = kw[q];
      sw_n[tile] = ks_seq[static_cast<uint32_t>(t * 4 + g4)];
    }
  };
  if (wave < nb_split) fetch(wave);

  for (int bb = wave; bb < nb_split; bb += 4) {
    uint32_t kw_c[2][KB], sw_c[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
#pragma unroll
      for (int q = 0; q < KB; ++q) kw_c[tile][q] = kw_n[tile][q];
      sw_c[tile] = sw_n[tile];
    }
    // the (lo, hi) record words of this lane group's value fields, for the 8
    // coordinate tiles: issued now, consumed after the logits
    uint32_t vw_c[8][2];
    {
      const uint32_t* vb_blk = vc_seq + static_cast<uint32_t>(((t0 >> 5) + bb) * kDD + n) * VB;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        vw_c[nt][0] = vb_blk[16 * nt * VB + vwlo];
        vw_c[nt][1] = vb_blk[16 * nt * VB + vwhi];
      }
    }
    if (bb + 4 < nb_split) fetch(bb + 4);              // in flight during this block

    const int tb = t0 + 32 * bb;                       // first token of the block
    const bool full = tb + 32 <= Ti;
    const int lb = 32 * bb;                            // block offset in the staged norms
    // ---------------- logits of the block's 32 tokens
    float sv[8];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint32_t* pw = kw_c[tile];
      // nibble q of E / O: the 4-bit index of the coordinate pair (4q, 4q+1) /
      // (4q+2, 4q+3); table entries are 4 bytes, so offset = nibble << 2
      uint32_t E = 0, Od = 0;
      if constexpr (KB == 2) {
        E = (pw[0] & 0x33333333u) | ((pw[1] << 2) & 0xCCCCCCCCu);
        Od = ((pw[0] >> 2) & 0x33333333u) | (pw[1] & 0xCCCCCCCCu);
      }
      const uint32_t sw = sw_c[tile];
      const uint32_t sv0 = sw << 2, sv2 = sw >> 2, sv3 = sw >> 4;
      floatx4 accC = {0.f, 0.f, 0.f, 0.f}, accS = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        // coordinates 4c .. 4c+3 of word g4: A = (hi, lo) of pair (4c, 4c+1), then of (4c+2, 4c+3)
        uint32_t offA, offB;
        if constexpr (KB == 2) {
          offA = (c == 0) ? (E << 2) & 0x3Cu : (E >> (4 * c - 2)) & 0x3Cu;
          offB = (c == 0) ? (Od << 2) & 0x3Cu : (Od >> (4 * c - 2)) & 0x3Cu;
        } else {
          offA = pair_index<KB>(pw, 2 * c) << 2;
          offB = pair_index<KB>(pw, 2 * c + 1) << 2;
        }
        const uint32_t a0 = *reinterpret_cast<const uint32_t*>(khi_b + offA);
        const uint32_t a1 = *reinterpret_cast<const uint32_t*>(klo_b + offA);
        const uint32_t a2 = *reinterpret_cast<const uint32_t*>(khi_b + offB);
        const uint32_t a3 = *reinterpret_cast<const uint32_t*>(klo_b + offB);
        accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(a0, a1, a2, a3), bq[c], accC, 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t as[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t ssrc = (q == 0) ? sv0 : (q == 1) ? sw : (q == 2) ? sv2 : sv3;
          as[q] = *reinterpret_cast<const uint32_t*>(slut_b + ((ssrc >> (8 * c)) & 0xCu));
        }
        accS = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(as[0], as[1], as[2], as[3]), bu[c], accS, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float cen = accC[i] + row_shl<G>(accC[i]);
        const float qj = accS[i] + row_shl<G>(accS[i]);
        const int li = lb + 8 * g4 + 4 * tile + i;
        float v = nk_s[li] * cen + rq_s[li] * qj;
        if (!full && tb + (li - lb) >= Ti) v = -INFINITY;
        sv[4 * tile + i] = v;
      }
    }
    // ---------------- online softmax, base 2
    float bm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    if (__ballot(bm > m_ref + kTau)) {
      const float m_new = fmaxf(m_ref, bm);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 on the first block
      lsum *= alpha;
      m_ref = m_new;
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * g4 + i);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) O[nt][i] *= a4[i];
      }
    }
    // A = p * ||v|| / sigma (fp16, <= 2^8); B = c_V[idx] for tokens 8*g4 .. 8*g4+7
    const float4 nva = *reinterpret_cast<const float4*>(&nv_s[lb + 8 * g4]);
    const float4 nvb = *reinterpret_cast<const float4*>(&nv_s[lb + 8 * g4 + 4]);
    const float nvk[8] = {nva.x, nva.y, nva.z, nva.w, nvb.x, nvb.y, nvb.z, nvb.w};
    half8 pa;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = __builtin_amdgcn_exp2f(sv[k] - m_ref);
      lsum += p;
      pa[k] = static_cast<_Float16>(p * nvk[k]);
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint32_t X = __builtin_amdgcn_alignbit(vw_c[nt][1], vw_c[nt][0], vsh);
      uint32_t bw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) bw[q] = vlut[(X >> (2 * VB * q)) & (VL - 1)];
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, u4_to_h8(bw[0], bw[1], bw[2], bw[3]), O[nt], 0, 0, 0);
    }
  }

  // ---------------- merge the 4 waves' states, write this split's partial
  __syncthreads();  // the staging area is reused below
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
      const float f = (m_s[w][g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_s[w][g] - M);
      acc += f * o_s[w][g][j];
      L += f * l_s[w][g];
    }
    float* out = partials + ((h0 + g) * nsplit + split) * (kDD + 2);
    out[j] = acc * sigma;
    if (j == 0) {
      out[kDD] = M;
      out[kDD + 1] = L;
    }
  }
}

// Merge the splits of one query head by log-sum-exp (base 2), then rotate
// back once: out = Pi^T (acc / L).
constexpr int kCombThreads = 256;

__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(
    const float* __restrict__ rot, const float* __restrict__ partials, int nsplit,
    float* __restrict__ out) {
  __shared__ float red[kCombThreads];
  __shared__ float half_acc[kDD];
  __shared__ float a[kDD];
  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x;
  const float* p = partials + h * nsplit * (kDD + 2);
  float M = -INFINITY;
  for (int sidx = tid; sidx < nsplit; sidx += kCombThreads) M = fmaxf(M, p[sidx * (kDD + 2) + kDD]);
  red[tid] = M;
  __syncthreads();
  for (int o = kCombThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();
  const int j = tid & (kDD - 1), part = tid >> 7;
  float acc = 0.f, L = 0.f;
  int sidx = part;
#pragma unroll 4
  for (; sidx < nsplit; sidx += 2) {
    const float* q = p + sidx * (kDD + 2);
    const float w = __builtin_amdgcn_exp2f(q[kDD] - M);
    acc = fmaf(q[j], w, acc);
    L = fmaf(q[kDD + 1], w, L);
  }
  if (part == 1) half_acc[j] = acc;
  red[tid] = L;
  __syncthreads();
  if (part == 0) a[j] = (acc + half_acc[j]) / (red[j] + red[j + kDD]);
  __syncthreads();
  if (tid < kDD) {
    float o = 0.f;
    for (int jj = 0; jj < kDD; ++jj) o = fmaf(rot[jj * kDD + tid], a[jj], o);
    out[h * kDD + tid] = o;
  }
}

// Split length: enough workgroups for about two rounds of the chip at two
// resident workgroups per CU (two waves per SIMD), in whole 32-token blocks,
// at most kMaxSplit (the staged norms of a split live in LDS).
constexpr int kResidentPerCu = 2;

static int split_length(int64_t nseq, int64_t T) {
  const int64_t target = 2 * kResidentPerCu * 256;
  int64_t per_seq = (target + nseq - 1) / nseq;
  if (per_seq < 1) per_seq = 1;
  int64_t len = (T + per_seq - 1) / per_seq;
  len = ((len + 31) / 32) * 32;
  if (len < 128) len = 128;
  if (len > kMaxSplit) len = kMaxSplit;
  return static_cast<int>(len);
}

static size_t a256(size_t x) { return (x + 255u) & ~static_cast<size_t>(255u); }

DecodeWorkspace decode_workspace_layout(int B, int Hq, int Hkv, int64_t T, int d, int m) {
  DecodeWorkspace w{};
  const size_t nh = static_cast<size_t>(B) * Hq;
  const int64_t nseq = static_cast<int64_t>(B) * Hkv;
  const int64_t len = split_length(nseq > 0 ? nseq : 1, T);
  const size_t nsplit = static_cast<size_t>((T + len - 1) / len);
  w.qr = 0;
  w.u = a256(nh * d * sizeof(float));
  w.frag = w.u + a256(nh * m * sizeof(float));
  w.lut = w.frag + a256(static_cast<size_t>(nseq) * kFragsPerSeq * 64 * sizeof(uint4));
  w.partials = w.lut + kLutBytes;
  w.total = w.partials + a256(nh * nsplit * (d + 2) * sizeof(float));
  return w;
}

template <int G, int KB>
static void launch_vb(int vb, dim3 grid, hipStream_t stream, const uint4* frag, const char* lut,
                      const tq_packed& k, const tq_packed& v, int len, float sl2, int nsplit,
                      float* partials) {
#define TQ_DEC(VBV)                                                                            \
  hipLaunchKernelGGL((decode_mfma_kernel<G, KB, VBV>), grid, dim3(kDecThreads), 0, stream,     \
                     frag, lut, k.T, len, k.codes, k.signs, k.norm, k.rnorm, k.norm_dtype,     \
                     v.codes, v.norm, v.norm_dtype, sl2, nsplit, partials)
  switch (vb) {
    case 1: TQ_DEC(1); break;
    case 2: TQ_DEC(2); break;
    case 3: TQ_DEC(3); break;
    default: TQ_DEC(4); break;
  }
#undef TQ_DEC
}

template <int G>
static hipError_t launch_g(const tq_tables& tk, const tq_tables& tv, const float* qr,
                           const float* u, int64_t nseq, const tq_packed& k, const tq_packed& v,
                           float sl2, char* ws, const DecodeWorkspace& lay, int len, int nsplit,
                           hipStream_t stream) {
  uint4* frag = reinterpret_cast<uint4*>(ws + lay.frag);
  char* lut = ws + lay.lut;
  float* partials = reinterpret_cast<float*>(ws + lay.partials);
  hipLaunchKernelGGL(decode_prep_kernel<G>, dim3(static_cast<unsigned>(nseq)), dim3(64), 0, stream,
                     qr, u, tk.bits, tv.bits, tk.centroids, tv.centroids, frag, lut);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(nsplit), static_cast<unsigned>(nseq));
  switch (tk.bits) {
    case 1: launch_vb<G, 1>(tv.bits, grid, stream, frag, lut, k, v, len, sl2, nsplit, partials); break;
    case 2: launch_vb<G, 2>(tv.bits, grid, stream, frag, lut, k, v, len, sl2, nsplit, partials); break;
    case 3: launch_vb<G, 3>(tv.bits, grid, stream, frag, lut, k, v, len, sl2, nsplit, partials); break;
    default: launch_vb<G, 4>(tv.bits, grid, stream, frag, lut, k, v, len, sl2, nsplit, partials); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const tq_tables& tk, const tq_tables& tv, const float* qr, const float* u,
                         int B, int Hq, int Hkv, const tq_packed& k, const tq_packed& v,
                         float scale, void* ws, const DecodeWorkspace& lay, float* out,
                         hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t nseq = static_cast<int64_t>(B) * Hkv;
  const int len = split_length(nseq, k.T);
  const int nsplit = static_cast<int>((k.T + len - 1) / len);
  const float sl2 = scale * 1.4426950408889634f;  // softmax in base 2
  char* base = static_cast<char*>(ws);
  hipError_t e;
  switch (G) {
    case 1: e = launch_g<1>(tk, tv, qr, u, nseq, k, v, sl2, base, lay, len, nsplit, stream); break;
    case 2: e = launch_g<2>(tk, tv, qr, u, nseq, k, v, sl2, base, lay, len, nsplit, stream); break;
    case 4: e = launch_g<4>(tk, tv, qr, u, nseq, k, v, sl2, base, lay, len, nsplit, stream); break;
    case 8: e = launch_g<8>(tk, tv, qr, u, nseq, k, v, sl2, base, lay, len, nsplit, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(B * Hq), dim3(kCombThreads), 0, stream, tk.rot,
                     reinterpret_cast<const float*>(base + lay.partials), nsplit, out);
  return hipGetLastError();
}

}  // namespace tq
