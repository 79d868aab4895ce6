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
//  * every workgroup lays the G rotated queries of its KV head out as
//    matrix-core B fragments -- fp16 hi in columns [0,G), the fp16 residual
//    in [G,2G) -- and builds its code tables in LDS from the codebooks.
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
// LDS code tables (built by build_tables): key tables at 0, sign table at
// kS8Off, value table at kVluOff
constexpr int kS8Off = 4096, kVluOff = 8192, kTabBytes = 9216;

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

// max over the 4 rows of 16 lanes (lanes n, n+16, n+32, n+48), in every lane:
// v_permlane16_swap / v_permlane32_swap exchange rows without LDS
__device__ __forceinline__ float max_over_rows(float v) {
  auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
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

// ------------------------------------------------------------ query operands
// Per KV head s and lane (n = lane%16, g4 = lane/16), 12 B-fragments of 8 fp16:
//  bq[0..7]: centroid K-steps c' = 0..7.  The K slots hold the coordinates
//    32*g4 + 4c' + {0,1,0,1,2,3,2,3}: every coordinate twice, once against
//    the hi and once against the lo half of its centroid.
//  bu[0..3]: sign K-steps c = 0..3, coordinates 32*g4 + 8c + i.
// Columns n < G carry the fp16 value, G <= n < 2G its fp16 residual, the
// rest zero.

// Centroid and sign dots of one 16-token tile (tile 0 or 1 of a 32-token
// block) for this lane's query-head column: lane (g4, n) gets, for rows
// 4*g4 + i, the centroid dot <q', c[idx]> (cen) and the sign dot
// <u, 2s - 1> (qj) of head n (n < G; the other lanes hold partial sums).
// pw: the tile token's KB plane words of coordinate word g4; sw: its sign
// word; tab: the LDS tables of build_tables.
template <int G, int KB>
__device__ __forceinline__ void tile_logits(const uint32_t* pw, uint32_t sw, const half8 (&bq)[8],
                                            const half8 (&bu)[4], const char* tab, float (&cen)[4],
                                            float (&qj)[4]) {
  floatx4 accC = {0.f, 0.f, 0.f, 0.f}, accS = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KB == 2) {
    // byte k of E / O: the quad-table index of coordinates 8k .. 8k+3 /
    // 8k+4 .. 8k+7 (plane-0 nibble | plane-1 nibble << 4)
    const uint32_t E = (pw[0] & 0x0F0F0F0Fu) | ((pw[1] & 0x0F0F0F0Fu) << 4);
    const uint32_t O = ((pw[0] >> 4) & 0x0F0F0F0Fu) | (pw[1] & 0xF0F0F0F0u);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t x = ((c & 1) ? O : E) >> (8 * (c >> 1)) & 0xFFu;
      const uint4 a = *reinterpret_cast<const uint4*>(tab + 16 * x);
      accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(a.x, a.y, a.z, a.w), bq[c], accC, 0, 0, 0);
    }
  } else {
    const char* khi_b = tab;
    const char* klo_b = tab + 1024;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // coordinates 4c .. 4c+3 of word g4: A = (hi, lo) of pair (4c, 4c+1), then of (4c+2, 4c+3)
      const uint32_t offA = pair_index<KB>(pw, 2 * c) << 2;
      const uint32_t offB = pair_index<KB>(pw, 2 * c + 1) << 2;
      const uint32_t a0 = *reinterpret_cast<const uint32_t*>(khi_b + offA);
      const uint32_t a1 = *reinterpret_cast<const uint32_t*>(klo_b + offA);
      const uint32_t a2 = *reinterpret_cast<const uint32_t*>(khi_b + offB);
      const uint32_t a3 = *reinterpret_cast<const uint32_t*>(klo_b + offB);
      accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(a0, a1, a2, a3), bq[c], accC, 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // sign K-step c: coordinates 8c .. 8c+7 of word g4 = byte c of the sign word
    const uint4 a = *reinterpret_cast<const uint4*>(tab + kS8Off + 16 * ((sw >> (8 * c)) & 0xFFu));
    accS = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(a.x, a.y, a.z, a.w), bu[c], accS, 0, 0, 0);
  }
  // the hi column n plus the lo column G + n
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cen[i] = accC[i] + row_shl<G>(accC[i]);
    qj[i] = accS[i] + row_shl<G>(accS[i]);
  }
}

// This lane's query fragments for KV head s, built from the rotated queries
// (q' = Pi q, u = S q', one row of d floats per query head) in the layout
// described above.
template <int G>
__device__ __forceinline__ void query_frags(const float* __restrict__ qr, const float* __restrict__ u,
                                            int64_t s, int lane, half8 (&bq)[8], half8 (&bu)[4]) {
  const int n = lane & 15, g4 = lane >> 4;
  const bool hi_col = n < G, lo_col = (n >= G) && (n < 2 * G);
  const int g = hi_col ? n : (lo_col ? n - G : 0);
  const float* qg = qr + (s * G + g) * kDD;
  const float* ug = u + (s * G + g) * kDD;
  auto part = [&](float x) -> _Float16 {
    const _Float16 a = static_cast<_Float16>(x);
    if (hi_col) return a;
    if (lo_col) return static_cast<_Float16>(x - static_cast<float>(a));
    return static_cast<_Float16>(0.f);
  };
  constexpr int kSlot[8] = {0, 1, 0, 1, 2, 3, 2, 3};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = part(qg[32 * g4 + 4 * c + kSlot[i]]);
    bq[c] = u4_to_h8(h2u(h[0], h[1]), h2u(h[2], h[3]), h2u(h[4], h[5]), h2u(h[6], h[7]));
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = part(ug[32 * g4 + 8 * c + i]);
    bu[c] = u4_to_h8(h2u(h[0], h[1]), h2u(h[2], h[3]), h2u(h[4], h[5]), h2u(h[6], h[7]));
  }
}

// The workgroup's code tables in LDS (kTabBytes at the start of its LDS),
// built from the codebooks:
//  * 2-bit keys: entry x of the quad table (uint4 at 16x) holds the centroids
//    of 4 consecutive coordinates whose plane-0 bits are x & 15 and plane-1
//    bits x >> 4, as {hi(c0,c1), lo(c0,c1), hi(c2,c3), lo(c2,c3)} -- the
//    order of a centroid K-step's slots;
//  * other widths: pair tables khi[x] / klo[x] (uint32 at 4x and 1024 + 4x)
//    with the fp16 hi / lo halves of the centroids of a coordinate pair whose
//    2*KB-bit index is x (bit 2p: plane p of the lower coordinate, bit 2p+1:
//    plane p of the upper);
//  * at kS8Off, entry x (uint4): the +-1 values of 8 sign bits x, as fp16;
//  * at kVluOff (VB > 0), vlut[x]: the value centroids of the token pair
//    whose fields are x & (2^VB - 1) and x >> VB.
template <int KB, int VB>
__device__ __forceinline__ void build_tables(const float* __restrict__ ck, const float* __restrict__ cv,
                                             char* tab, int tid, int nthreads) {
  auto hilo = [&](float c, _Float16& h, _Float16& l) {
    h = static_cast<_Float16>(c);
    l = static_cast<_Float16>(c - static_cast<float>(h));
  };
  if constexpr (KB == 2) {
    uint4* quad = reinterpret_cast<uint4*>(tab);
    for (int x = tid; x < 256; x += nthreads) {
      _Float16 h[4], l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hilo(ck[((x >> i) & 1) | (((x >> (4 + i)) & 1) << 1)], h[i], l[i]);
      quad[x] = make_uint4(h2u(h[0], h[1]), h2u(l[0], l[1]), h2u(h[2], h[3]), h2u(l[2], l[3]));
    }
  } else {
    uint32_t* khi = reinterpret_cast<uint32_t*>(tab);
    uint32_t* klo = reinterpret_cast<uint32_t*>(tab + 1024);
    for (int x = tid; x < (1 << (2 * KB)); x += nthreads) {
      int ia = 0, ib = 0;
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        ia |= ((x >> (2 * p)) & 1) << p;
        ib |= ((x >> (2 * p + 1)) & 1) << p;
      }
      _Float16 ha, la, hb, lb;
      hilo(ck[ia], ha, la);
      hilo(ck[ib], hb, lb);
      khi[x] = h2u(ha, hb);
      klo[x] = h2u(la, lb);
    }
  }
  uint4* s8 = reinterpret_cast<uint4*>(tab + kS8Off);
  for (int x = tid; x < 256; x += nthreads) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = h2u(static_cast<_Float16>(((x >> (2 * i)) & 1) ? 1.f : -1.f),
                 static_cast<_Float16>(((x >> (2 * i + 1)) & 1) ? 1.f : -1.f));
    s8[x] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if constexpr (VB > 0) {
    uint32_t* vlut = reinterpret_cast<uint32_t*>(tab + kVluOff);
    for (int x = tid; x < (1 << (2 * VB)); x += nthreads)
      vlut[x] = h2u(static_cast<_Float16>(cv[x & ((1 << VB) - 1)]), static_cast<_Float16>(cv[x >> VB]));
  }
}

// ------------------------------------------------------------ the kernel
template <int G, int KB, int VB>
__global__ __launch_bounds__(kDecThreads, 3) void decode_mfma_kernel(
    const float* __restrict__ qr, const float* __restrict__ u, const float* __restrict__ ck,
    const float* __restrict__ cv, int64_t T, int split_len,
    const uint32_t* __restrict__ kcodes, const uint32_t* __restrict__ ksigns, const void* knorm,
    const void* krnorm, int knd, const uint32_t* __restrict__ vcodes, const void* vnorm, int vnd,
    float sl2, int nsplit, float* __restrict__ partials) {
  constexpr int VL = 1 << (2 * VB);
  // One LDS buffer with a fixed layout: the code tables first (small
  // offsets fold into the ds_read instructions; the hi and lo key tables sit
  // 1 KiB apart so that their reads stay separate and land directly in the
  // matrix-core operand registers), then the staged norms of the split.
  // After the main loop the staging bytes hold the four waves' softmax
  // states for the merge.
  constexpr int kStage = kTabBytes;
  constexpr int kStageBytes = kMaxSplit * 12;
  constexpr int kMergeBytes = (2 * 4 * 16 + 4 * G * kDD + 4) * 4;
  constexpr int kRed = kStage + (kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes);
  __shared__ __align__(16) char lds[kRed + 16];
  const uint32_t* vlut = reinterpret_cast<const uint32_t*>(lds + kVluOff);
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
  const int64_t Tp = (T + 31) / 32 * 32;             // padded tokens per sequence (streams)
  const int t1 = (t0 + split_len < Ti) ? t0 + split_len : Ti;
  const int ntok = t1 - t0;
  const float qjl = sqrtf(static_cast<float>(M_PI) / 2.f) / 128.f;

  build_tables<KB, VB>(ck, cv, lds, tid, kDecThreads);  // visible after the barrier below
  float sigma;
  {
    const int64_t rec0 = s * Tp + t0;
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
  query_frags<G>(qr, u, s, lane, bq, bu);
  __syncthreads();

  floatx4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // lanes outside the G heads never rescale (their reference stays 0)
  float m_ref = (n < G) ? -INFINITY : 0.f, lsum = 0.f;
  const int nblk = (Ti + 31) / 32;
  const int nb_split = (ntok + 31) / 32;
  const uint32_t* kc_seq = kcodes + s * Tp * 4 * KB;
  const uint32_t* ks_seq = ksigns + s * Tp * 4;
  const uint32_t* vc_seq = vcodes + s * nblk * kDD * VB;
  const int rowtok = 8 * (n >> 2) + (n & 3);          // token of A-row n (tile 0)
  const int vbit0 = 8 * VB * g4;                       // this lane group's 8 value fields
  // the lane group's fields span at most two record words: load the pair
  // (vw0, vw0 + 1) that holds them (one 8-byte load; vw0 <= VB - 2 keeps it
  // inside the record) and funnel-shift them out
  const int vwlo = vbit0 >> 5, vsh = vbit0 & 31;
  const int vw0 = (VB >= 2 && vwlo > VB - 2) ? VB - 2 : vwlo;
  const bool vhi_only = vwlo > vw0;                    // fields lie in the upper word

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
        if constexpr (VB >= 2) {
          typedef uint2 __attribute__((aligned(4))) uint2_a4;  // record words are 4-byte aligned
          const uint2 w2 = *reinterpret_cast<const uint2_a4*>(vb_blk + 16 * nt * VB + vw0);
          vw_c[nt][0] = w2.x;
          vw_c[nt][1] = w2.y;
        } else {
          vw_c[nt][0] = vb_blk[16 * nt * VB];
          vw_c[nt][1] = 0u;
        }
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
      float cen[4], qj[4];
      tile_logits<G, KB>(kw_c[tile], sw_c[tile], bq, bu, lds, cen, qj);
      const int l0 = lb + 8 * g4 + 4 * tile;
      const float4 nk4 = *reinterpret_cast<const float4*>(&nk_s[l0]);
      const float4 rq4 = *reinterpret_cast<const float4*>(&rq_s[l0]);
      const float nk[4] = {nk4.x, nk4.y, nk4.z, nk4.w}, rq[4] = {rq4.x, rq4.y, rq4.z, rq4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * tile + i] = nk[i] * cen[i] + rq[i] * qj[i];
      if (!full) {  // the context's last, partial block: tokens past T get no weight
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tb + (l0 + i - lb) >= Ti) sv[4 * tile + i] = -INFINITY;
      }
    }
    // ---------------- online softmax, base 2
    float bm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    bm = max_over_rows(bm);
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
      const uint32_t X = vhi_only ? (vw_c[nt][1] >> vsh)
                                  : __builtin_amdgcn_alignbit(vw_c[nt][1], vw_c[nt][0], vsh);
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

// ------------------------------------------------------------ logits only
// Raw logits of the G query heads sharing KV head s (same page, Stage 2
// closing paragraph): l_t = ||k_t|| <q', c[idx_t]> + sqrt(pi/2)/m ||r_t|| <u, 2 s_t - 1>
// with ||r_t|| the stored ||k|| ||r^||.  One workgroup per (split, KV head),
// the same tiles as decode; out[(s*G + g) * T + t].
template <int G, int KB>
__global__ __launch_bounds__(kDecThreads, 2) void logits_mfma_kernel(
    const float* __restrict__ qr, const float* __restrict__ u, const float* __restrict__ ck,
    int64_t T, int split_len, const uint32_t* __restrict__ kcodes,
    const uint32_t* __restrict__ ksigns, const void* knorm, const void* krnorm, int knd,
    float* __restrict__ out) {
  constexpr int kStage = kTabBytes;
  __shared__ __align__(16) char lds[kStage + 2 * kMaxSplit * 4];
  float* nk_s = reinterpret_cast<float*>(lds + kStage);   // ||k||
  float* rq_s = nk_s + kMaxSplit;                          // sqrt(pi/2)/m ||k|| ||r||

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int t0 = split * split_len;                  // T < 2^28 (checked on the host)
  const int Ti = static_cast<int>(T);
  const int64_t Tp = (T + 31) / 32 * 32;             // padded tokens per sequence (streams)
  const int t1 = (t0 + split_len < Ti) ? t0 + split_len : Ti;
  const int ntok = t1 - t0;
  const float qjl = sqrtf(static_cast<float>(M_PI) / 2.f) / 128.f;

  build_tables<KB, 0>(ck, nullptr, lds, tid, kDecThreads);
  {
    const int64_t rec0 = s * Tp + t0;
    const int nst = (ntok + 31) & ~31;
    for (int i = tid; i < nst; i += kDecThreads) {
      float a = 0.f, b = 0.f;
      if (i < ntok) {
        a = load_norm(knorm, knd, rec0 + i);
        b = load_norm(krnorm, knd, rec0 + i);
      }
      nk_s[i] = a;
      rq_s[i] = qjl * b;
    }
  }
  half8 bq[8], bu[4];
  query_frags<G>(qr, u, s, lane, bq, bu);
  __syncthreads();

  const int nb_split = (ntok + 31) / 32;
  const uint32_t* kc_seq = kcodes + s * Tp * 4 * KB;
  const uint32_t* ks_seq = ksigns + s * Tp * 4;
  const int rowtok = 8 * (n >> 2) + (n & 3);          // token of A-row n (tile 0)
  float* out_h = out + (s * G + (n < G ? n : 0)) * T;
  const bool vec_ok = (Ti & 3) == 0;                  // 16-byte aligned output rows

  uint32_t kw_n[2][KB], sw_n[2];
  auto fetch = [&](int bb) {
    const int tb = t0 + 32 * bb;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      int t = tb + rowtok + 4 * tile;
      t = (t < Ti) ? t : Ti - 1;                       // clamped: tail tokens are not stored
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
    if (bb + 4 < nb_split) fetch(bb + 4);              // in flight during this block
    const int lb = 32 * bb;
    const int tb = t0 + lb;
    float lv[8];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      float cen[4], qj[4];
      tile_logits<G, KB>(kw_c[tile], sw_c[tile], bq, bu, lds, cen, qj);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int li = lb + 8 * g4 + 4 * tile + i;
        lv[4 * tile + i] = nk_s[li] * cen[i] + rq_s[li] * qj[i];
      }
    }
    // lane (g4, n < G): tokens tb + 8*g4 .. tb + 8*g4 + 7 of head n
    if (n < G) {
      const int tt = tb + 8 * g4;
      if (vec_ok && tt + 8 <= Ti) {
        float4* o4 = reinterpret_cast<float4*>(out_h + tt);
        o4[0] = make_float4(lv[0], lv[1], lv[2], lv[3]);
        o4[1] = make_float4(lv[4], lv[5], lv[6], lv[7]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (tt + k < Ti) out_h[tt + k] = lv[k];
      }
    }
  }
}

// Merge the splits of one query head by log-sum-exp (base 2), then rotate
// back once: out = Pi^T (acc / L).  512 threads: 4 groups of splits x 128
// coordinates, then 4 groups of rows of Pi^T.
constexpr int kCombThreads = 512;

__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(
    const float* __restrict__ rot, const float* __restrict__ partials, int nsplit,
    float* __restrict__ out) {
  __shared__ float red[kCombThreads];
  __shared__ float part_acc[4][kDD];
  __shared__ float part_l[4];
  __shared__ float a[kDD];
  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x;
  const float* p = partials + h * nsplit * (kDD + 2);
  float M = -INFINITY;
  for (int sidx = tid; sidx < nsplit; sidx += kCombThreads) M = fmaxf(M, p[sidx * (kDD + 2) + kDD]);
  M = wave_max(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) M = fmaxf(M, red[w]);
  const int j = tid & (kDD - 1), part = tid >> 7;
  float acc = 0.f, L = 0.f;
#pragma unroll 8
  for (int sidx = part; sidx < nsplit; sidx += 4) {
    const float* q = p + sidx * (kDD + 2);
    const float w = __builtin_amdgcn_exp2f(q[kDD] - M);
    acc = fmaf(q[j], w, acc);
    L = fmaf(q[kDD + 1], w, L);
  }
  part_acc[part][j] = acc;
  if (j == 0) part_l[part] = L;
  __syncthreads();
  if (tid < kDD) {
    const float Lt = part_l[0] + part_l[1] + part_l[2] + part_l[3];
    a[tid] = (part_acc[0][tid] + part_acc[1][tid] + part_acc[2][tid] + part_acc[3][tid]) / Lt;
  }
  __syncthreads();
  // out[j] = sum_jj Pi[jj][j] a[jj]; group `part` takes rows jj = 32 part .. 32 part + 31
  float o = 0.f;
#pragma unroll 8
  for (int jj = 32 * part; jj < 32 * part + 32; ++jj) o = fmaf(rot[jj * kDD + j], a[jj], o);
  part_acc[part][j] = o;  // every thread read a[] only after the barrier above
  __syncthreads();
  if (tid < kDD) out[h * kDD + tid] = part_acc[0][tid] + part_acc[1][tid] + part_acc[2][tid] + part_acc[3][tid];
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
  w.partials = w.u + a256(nh * m * sizeof(float));
  w.total = w.partials + a256(nh * nsplit * (d + 2) * sizeof(float));
  return w;
}

template <int G, int KB>
static void launch_vb(int vb, dim3 grid, hipStream_t stream, const tq_tables& tk,
                      const tq_tables& tv, const float* qr, const float* u, const tq_packed& k,
                      const tq_packed& v, int len, float sl2, int nsplit, float* partials) {
#define TQ_DEC(VBV)                                                                            \
  hipLaunchKernelGGL((decode_mfma_kernel<G, KB, VBV>), grid, dim3(kDecThreads), 0, stream,     \
                     qr, u, tk.centroids, tv.centroids, k.T, len, k.codes, k.signs, k.norm,    \
                     k.rnorm, k.norm_dtype, v.codes, v.norm, v.norm_dtype, sl2, nsplit, partials)
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
                           float sl2, float* partials, int len, int nsplit, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(nsplit), static_cast<unsigned>(nseq));
  switch (tk.bits) {
    case 1: launch_vb<G, 1>(tv.bits, grid, stream, tk, tv, qr, u, k, v, len, sl2, nsplit, partials); break;
    case 2: launch_vb<G, 2>(tv.bits, grid, stream, tk, tv, qr, u, k, v, len, sl2, nsplit, partials); break;
    case 3: launch_vb<G, 3>(tv.bits, grid, stream, tk, tv, qr, u, k, v, len, sl2, nsplit, partials); break;
    default: launch_vb<G, 4>(tv.bits, grid, stream, tk, tv, qr, u, k, v, len, sl2, nsplit, partials); break;
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
  float* partials = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.partials);
  hipError_t e;
  switch (G) {
    case 1: e = launch_g<1>(tk, tv, qr, u, nseq, k, v, sl2, partials, len, nsplit, stream); break;
    case 2: e = launch_g<2>(tk, tv, qr, u, nseq, k, v, sl2, partials, len, nsplit, stream); break;
    case 4: e = launch_g<4>(tk, tv, qr, u, nseq, k, v, sl2, partials, len, nsplit, stream); break;
    case 8: e = launch_g<8>(tk, tv, qr, u, nseq, k, v, sl2, partials, len, nsplit, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(B * Hq), dim3(kCombThreads), 0, stream, tk.rot,
                     partials, nsplit, out);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_logits_g(const tq_tables& tk, const float* qr, const float* u,
                                  int64_t nseq, const tq_packed& k, int len, int nsplit, float* out,
                                  hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(nsplit), static_cast<unsigned>(nseq));
#define TQ_LOG(KBV)                                                                                \
  hipLaunchKernelGGL((logits_mfma_kernel<G, KBV>), grid, dim3(kDecThreads), 0, stream, qr, u,     \
                     tk.centroids, k.T, len, k.codes, k.signs, k.norm, k.rnorm, k.norm_dtype, out)
  switch (tk.bits) {
    case 1: TQ_LOG(1); break;
    case 2: TQ_LOG(2); break;
    case 3: TQ_LOG(3); break;
    default: TQ_LOG(4); break;
  }
#undef TQ_LOG
  return hipGetLastError();
}

hipError_t launch_logits_mfma(const tq_tables& tk, const float* qr, const float* u, int B, int Hq,
                              int Hkv, const tq_packed& k, float* logits, hipStream_t stream) {
  if (B == 0 || k.T == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t nseq = static_cast<int64_t>(B) * Hkv;
  const int len = split_length(nseq, k.T);
  const int nsplit = static_cast<int>((k.T + len - 1) / len);
  switch (G) {
    case 1: return launch_logits_g<1>(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 2: return launch_logits_g<2>(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 4: return launch_logits_g<4>(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 8: return launch_logits_g<8>(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
