// Online quantization of key / value vectors on the matrix cores.
//
// Method (a2a-mcp.org page, "How it works"): Stage 1 normalises the vector,
// rotates it with Pi and maps every rotated coordinate to a b-bit Lloyd-Max
// index; Stage 2 (keys only) takes the residual r = Pi x/||x|| - c[idx] and
// stores the signs of z = S r, one bit per sketch row.
//
// Mapping onto gfx950 (wave64, v_mfma_f32_32x32x16_f16):
//  * a unit of work is 32 consecutive tokens of one sequence.  The 4 waves of
//    a workgroup share it; wave w owns the 32 rotated coordinates
//    [32w, 32w+32) and, for keys, the 32 sketch rows [32w, 32w+32), so one
//    32x32 output tile per product.  Its slices of Pi^T and S^T live in
//    registers as fp16 hi + lo pairs for the whole kernel.
//  * the 32 input vectors are staged in LDS as fp16.  Each vector is first
//    scaled by a power of two that puts its norm just below 2^15: a bf16
//    input is then exact in fp16, an fp32 input is split into fp16 hi + lo.
//    Pi is held x16 so that its lo half stays a normal fp16 number.  The
//    rotation X Pi^T carries about 22 significant bits, fp32-grade.
//  * result layout: lane l holds coordinate 32w + l%32 of the 16 tokens
//    16*(l/32) + v, v = 0..15 (A-row r of a tile is token
//    16*((r/4)%2) + 4*(r/8) + r%4).  A wave-wide compare of register v is then
//    two finished 32-bit words: the low half is word w of token v, the high
//    half word w of token 16 + v.  Code planes and sign words are moved from
//    those masks into lanes with v_writelane and stored lane by lane.
//  * keys: the residual (x256, fp16 hi + lo) goes through LDS; the sketch is
//    Z = R S^T with three products (hi*hi, hi*lo, lo*hi) and ||r||^2 is the
//    diagonal of R R^T, each wave summing the 32 coordinates it owns.
//  * values: every lane packs the b-bit fields of its 16 consecutive tokens
//    of one coordinate; the 32-token record is the two lane halves' fields in
//    token order.
#include <math.h>

#include "common.h"
#include "launch.h"

// v_writelane_b32: set lane `lane` of `old` to the wave-uniform `value`.
extern "C" __device__ int tq_writelane_i32(int value, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

namespace tq {

typedef _Float16 qhalf8 __attribute__((ext_vector_type(8)));
typedef _Float16 qhalf2 __attribute__((ext_vector_type(2)));
typedef float qfloatx4 __attribute__((ext_vector_type(4)));
typedef float qfloatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t qu32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kQThreads = 256;
constexpr int kUnit = 32;          // tokens per unit
constexpr int kRowH = 136;         // LDS row stride in halves (272 B, a multiple of 16 B)
constexpr float kPiScale = 16.f;   // Pi is held x16 so that its lo half stays normal
constexpr float kResScale = 256.f; // rotated coordinates are handled x256 (exact)

__device__ __forceinline__ uint32_t writelane(uint32_t value, int lane, uint32_t old) {
  return static_cast<uint32_t>(tq_writelane_i32(static_cast<int>(value), lane, static_cast<int>(old)));
}

__device__ __forceinline__ uint32_t h2u(qhalf2 h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ qhalf8 qu4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  qu32x4 v = {a, b, c, d};
  return __builtin_bit_cast(qhalf8, v);
}

__device__ __forceinline__ float pow2f(int e) {  // 2^e for -126 <= e <= 127
  return __uint_as_float(static_cast<uint32_t>(127 + e) << 23);
}

// fp16 hi + lo fragment of 8 consecutive fp32 values scaled by `sc`.
__device__ __forceinline__ void split_frag(const float* p, float sc, qhalf8& hi, qhalf8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = p[2 * i] * sc, b = p[2 * i + 1] * sc;
    const qhalf2 hh = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    const qhalf2 ll = {static_cast<_Float16>(a - static_cast<float>(hh[0])),
                       static_cast<_Float16>(b - static_cast<float>(hh[1]))};
    h[i] = h2u(hh);
    l[i] = h2u(ll);
  }
  hi = qu4(h[0], h[1], h[2], h[3]);
  lo = qu4(l[0], l[1], l[2], l[3]);
}

// B fragment of a Walsh-Hadamard rotation: the signs of 8 entries of Pi_H
// (+-1/sqrt(d)) as fp16 +-1, exact, so one product replaces the hi + lo pair
__device__ __forceinline__ void sign_frag(const float* p, qhalf8& hi) {
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = (__float_as_uint(p[2 * i]) >> 16) & 0x8000u;
    const uint32_t b = (__float_as_uint(p[2 * i + 1]) >> 16) & 0x8000u;
    h[i] = (a | 0x3C00u) | ((b | 0x3C00u) << 16);   // fp16 1.0 = 0x3C00
  }
  hi = qu4(h[0], h[1], h[2], h[3]);
}

// fp16(a - hi.x), fp16(b - hi.y): the lo halves of an fp16 hi + lo split,
// each from one mixed-precision fma (hi read as fp16, a and b as fp32)
__device__ __forceinline__ qhalf2 split_lo(qhalf2 hi, float a, float b) {
  uint32_t lo = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t h = h2u(hi);
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(lo) : "v"(h), "v"(a));
  asm("v_fma_mixhi_f16 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(lo)
      : "v"(h), "v"(b));
#else
  (void)hi;
  (void)a;
  (void)b;
#endif
  return __builtin_bit_cast(qhalf2, lo);
}

// Code table of one stream at the x256 scale: positive decision boundaries
// bounds[L/2 .. L-2] and centroid magnitudes centroids[L/2 .. L-1].  The
// codebooks are symmetric about 0.
template <int BITS>
struct QTab {
  float tpos[(1 << BITS) / 2 > 1 ? (1 << BITS) / 2 - 1 : 1];
  float cpos[(1 << BITS) / 2];
};

// c ? a : b on values (a conditional over two array elements would select
// an address and keep the table out of registers)
__device__ __forceinline__ float sel(bool c, float a, float b) { return c ? a : b; }

// Index of y (x256 scale) = number of boundaries <= y.  Writes the lane masks
// of the index bits into P (bit BITS-1 is the sign test: y's sign bit clear;
// the lower bits are the magnitude cell, complemented for y < 0), returns the
// signed centroid through C and the index through idx.  The sign test reads
// the sign bit, so a -0.0 (only from a negative product that underflowed)
// counts as negative, like the value it rounds.
template <int BITS>
__device__ __forceinline__ void quant_one(float y, const QTab<BITS>& tab, uint64_t* P, float& C,
                                          int& idx) {
  const int sgn = static_cast<int>(__float_as_uint(y)) >> 31;   // 0, or -1 for a set sign bit
  const bool ms = sgn == 0;
  const float a = fabsf(y);
  const uint64_t Ms = __ballot(ms);
  float mag;
  int cnt;
  P[BITS - 1] = Ms;
  if constexpr (BITS == 1) {
    mag = tab.cpos[0];
    cnt = 0;
  } else if constexpr (BITS == 2) {
    const bool m1 = a >= tab.tpos[0];
    P[0] = ~(Ms ^ __ballot(m1));
    mag = sel(m1, tab.cpos[1], tab.cpos[0]);
    cnt = m1 ? 1 : 0;
  } else if constexpr (BITS == 3) {
    const bool m1 = a >= tab.tpos[1];
    const bool m2 = a >= sel(m1, tab.tpos[2], tab.tpos[0]);
    P[1] = ~(Ms ^ __ballot(m1));
    P[0] = ~(Ms ^ __ballot(m2));
    mag = sel(m1, sel(m2, tab.cpos[3], tab.cpos[2]), sel(m2, tab.cpos[1], tab.cpos[0]));
    cnt = (m1 ? 2 : 0) + (m2 ? 1 : 0);
  } else {
    const bool m1 = a >= tab.tpos[3];
    const bool m2 = a >= sel(m1, tab.tpos[5], tab.tpos[1]);
    const float t3 = sel(m1, sel(m2, tab.tpos[6], tab.tpos[4]), sel(m2, tab.tpos[2], tab.tpos[0]));
    const bool m3 = a >= t3;
    P[2] = ~(Ms ^ __ballot(m1));
    P[1] = ~(Ms ^ __ballot(m2));
    P[0] = ~(Ms ^ __ballot(m3));
    const float lo4 = sel(m2, sel(m3, tab.cpos[3], tab.cpos[2]), sel(m3, tab.cpos[1], tab.cpos[0]));
    const float hi4 = sel(m2, sel(m3, tab.cpos[7], tab.cpos[6]), sel(m3, tab.cpos[5], tab.cpos[4]));
    mag = sel(m1, hi4, lo4);
    cnt = (m1 ? 4 : 0) + (m2 ? 2 : 0) + (m3 ? 1 : 0);
  }
  constexpr int half = 1 << (BITS - 1);
  C = ms ? mag : -mag;
  idx = (cnt ^ sgn) + half;  // half + cnt, or half - 1 - cnt
}

template <typename XT>
struct RawX {
  static constexpr int kWords = sizeof(XT) == 4 ? 4 : 2;  // uint4 per thread (16 elements)
  uint4 w[kWords];
};

template <typename XT>
__device__ __forceinline__ void unpack_raw(const RawX<XT>& r, float* xv) {
  if constexpr (sizeof(XT) == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[4 * i + 0] = __uint_as_float(r.w[i].x);
      xv[4 * i + 1] = __uint_as_float(r.w[i].y);
      xv[4 * i + 2] = __uint_as_float(r.w[i].z);
      xv[4 * i + 3] = __uint_as_float(r.w[i].w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t u[4] = {r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[8 * i + 2 * e] = __uint_as_float(u[e] << 16);
        xv[8 * i + 2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
      }
    }
  }
}

// DPP lane permutations within rows of 16 lanes: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1] and row_half_mirror (lane i <-> 7 - i within 8 lanes)
constexpr int kDppSwap1 = 0xB1, kDppSwap2 = 0x4E, kDppHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// sum / max over the 8 lanes that stage one token (lanes 8k .. 8k+7)
__device__ __forceinline__ float sum8(float v) {
  v += dpp<kDppSwap1>(v);
  v += dpp<kDppSwap2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v;
}

__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp<kDppSwap1>(v));
  v = fmaxf(v, dpp<kDppSwap2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return v;
}

// sum of squares of the 16 staged elements; bf16 pairs go through v_dot2
template <typename XT>
__device__ __forceinline__ float sumsq16(const RawX<XT>& r, const float* xv) {
  float ss = 0.f;
  if constexpr (sizeof(XT) == 2) {
    typedef __bf16 qbf2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t u[4] = {r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const qbf2 b = __builtin_bit_cast(qbf2, u[e]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(b, b, ss, false);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) ss = fmaf(xv[i], xv[i], ss);
  }
  return ss;
}

// APPEND: the stream already holds tokens below pos (a separate instance, so
// that the whole-stream launches carry none of the merge code).  HAD: Pi is
// a randomized Walsh-Hadamard rotation, whose sqrt(d) Pi has entries +-1:
// one fp16 product rotates exactly, where a general Pi needs hi + lo.
template <typename XT, bool KEY, int BITS, bool APPEND, bool HAD>
__global__ __launch_bounds__(kQThreads, KEY ? 2 : 3) void quantize_mfma_kernel(
    const float* __restrict__ rot, const float* __restrict__ sketch,
    const float* __restrict__ cent, const float* __restrict__ bnd, const XT* __restrict__ x,
    int64_t nseq, int64_t pos_arg, int64_t T, int64_t Tp, uint32_t* __restrict__ codes,
    uint32_t* __restrict__ signs,
    void* __restrict__ norm, void* __restrict__ rnorm, int norm_dtype) {
  constexpr bool kSplitX = sizeof(XT) == 4;  // fp32 input: stage hi and lo
  constexpr int kXP = kSplitX ? 2 : 1;
  // keys: one staging buffer (the sketch barrier separates its reads from the
  // next unit's writes); values: two, so that one barrier per unit suffices
  constexpr int kXB = KEY ? 1 : 2;
  __shared__ __align__(16) _Float16 xs[kXB][kXP][kUnit][kRowH];
  __shared__ __align__(16) _Float16 rs[KEY ? 2 : 1][KEY ? kUnit : 1][KEY ? kRowH : 8];
  __shared__ __align__(16) float rinv_s[2][kUnit];  // kResScale / (rotation scale * ||scaled x||); 0 for x = 0
  __shared__ float n_s[2][kUnit];                 // ||x||, by unit parity
  __shared__ float rho_s[2][4][KEY ? kUnit : 1];  // per-wave sums of the residual squares (x256^2)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, h = lane >> 5;

  QTab<BITS> tab;
  constexpr int kHalf = (1 << BITS) / 2;
#pragma unroll
  for (int i = 0; i < kHalf; ++i) tab.cpos[i] = cent[kHalf + i] * kResScale;
#pragma unroll
  for (int i = 0; i + 1 < kHalf; ++i) tab.tpos[i] = bnd[kHalf + i] * kResScale;
  if constexpr (BITS == 1) tab.tpos[0] = 0.f;

  // B fragments: Pi^T for coordinates j = 32*wave + c32 and (keys) S^T for
  // sketch rows i = 32*wave + c32; K-step c covers input index 16c + 8h + e.
  qhalf8 bph[8], bpl[HAD ? 1 : 8];
  qhalf8 bsh[KEY ? 8 : 1], bsl[KEY ? 8 : 1];
  {
    const int j = 32 * wave + c32;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (HAD) sign_frag(rot + j * kD + 16 * c + 8 * h, bph[c]);
      else split_frag(rot + j * kD + 16 * c + 8 * h, kPiScale, bph[c], bpl[c]);
    }
    if constexpr (KEY) {
#pragma unroll
      for (int c = 0; c < 8; ++c) split_frag(sketch + j * kD + 16 * c + 8 * h, 1.f, bsh[c], bsl[c]);
    }
  }

  // x holds tokens pos .. T-1 of every sequence; the blocks that hold them are
  // blk0 .. blk0+nblk-1 (Tp: tokens stored per sequence).  Tokens below pos
  // keep their records, tokens from T to the block's end become padding.
  const int64_t pos = APPEND ? pos_arg : 0;
  const int64_t nx = T - pos;
  const int64_t blk0 = pos / kUnit;
  const int64_t nblk = (T + kUnit - 1) / kUnit - blk0;
  const int64_t units = nseq * nblk;
  // A-row c32 of a 32x32 tile holds token atok
  const int atok = 16 * ((c32 >> 2) & 1) + 4 * (c32 >> 3) + (c32 & 3);
  // staging role: token sv, elements 16*sq .. 16*sq+15
  const int sv = tid >> 3, sq = tid & 7;
  // (sequence, block) of the first unit and the per-iteration step
  const int64_t step_s = gridDim.x / nblk, step_b = gridDim.x % nblk;
  int64_t s = blockIdx.x / nblk, blk = blockIdx.x % nblk;

  auto load_raw = [&](int64_t us, int64_t ub, RawX<XT>& raw) {
    const int64_t t = (blk0 + ub) * kUnit + sv;
    if (us < nseq && t >= pos && t < T) {
      const uint4* src = reinterpret_cast<const uint4*>(x + ((us * nx + t - pos) * kD + 16 * sq));
#pragma unroll
      for (int r = 0; r < RawX<XT>::kWords; ++r) raw.w[r] = src[r];
    } else {
#pragma unroll
      for (int r = 0; r < RawX<XT>::kWords; ++r) raw.w[r] = make_uint4(0u, 0u, 0u, 0u);
    }
  };

  auto advance = [&](int64_t& us, int64_t& ub) {
    us += step_s;
    ub += step_b;
    if (ub >= nblk) {
      ub -= nblk;
      ++us;
    }
  };

  // input of the current unit and (bf16) of the next one: two units of
  // loads in flight; fp32 input keeps one (its registers are twice as many)
  constexpr bool kAhead2 = !kSplitX;
  RawX<XT> raw, raw_next;
  int64_t s1 = s, b1 = blk;
  advance(s1, b1);
  int64_t s2 = s1, b2 = b1;
  advance(s2, b2);
  load_raw(s, blk, raw);
  if constexpr (kAhead2) load_raw(s1, b1, raw_next);

  // keys: the norms of a unit are stored after the next unit's first barrier
  // (they need every wave's share of ||r||^2)
  int64_t pend_base = 0;
  int pend_lo = 0, pend_n = 0;
  auto store_key_norms = [&](int pp) {
    if (tid >= pend_lo && tid < pend_n) {  // the unit's new tokens, padding included
      const float rho2 = rho_s[pp][0][tid] + rho_s[pp][1][tid] + rho_s[pp][2][tid] + rho_s[pp][3][tid];
      const float nx = n_s[pp][tid];
      store_norm(norm, norm_dtype, pend_base + tid, nx);
      store_norm(rnorm, norm_dtype, pend_base + tid, nx * (sqrtf(rho2) / kResScale));
    }
  };

  int par = 0;
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x, par ^= 1) {
    const int xb = KEY ? 0 : par;
    const int64_t t0 = (blk0 + blk) * kUnit;
    const int nvalid = static_cast<int>((T - t0 < kUnit) ? T - t0 : kUnit);
    const int lo = pos > t0 ? static_cast<int>(pos - t0) : 0;  // tokens t0 .. t0+lo-1 are kept

    // ---------------- stage: norms, power-of-two range scale, fp16 copy
    {
      float xv[16];
      unpack_raw<XT>(raw, xv);
      float ss = sum8(sumsq16<XT>(raw, xv));
      int sh;
      if (ss >= 1.f && ss < 0x1p28f) {
        // ||x|| in [1, 2^14): every element is below 2^14 and those that are
        // not exact in fp16 (below 2^-17) are negligible against the norm
        sh = 0;
      } else if (ss >= 0x1p-100f && ss <= 0x1p100f) {
        int e;
        (void)frexpf(ss, &e);      // ss in [2^(e-1), 2^e): ||x|| < 2^ceil(e/2)
        sh = 15 - ((e + 1) >> 1);  // ||x|| * 2^sh < 2^15
        const float f = pow2f(sh);
#pragma unroll
        for (int i = 0; i < 16; ++i) xv[i] *= f;
        ss *= f * f;
      } else {
        // far outside the usual range (or zero): scale from the largest element
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(xv[i]));
        mx = max8(mx);
        int e = 0;
        if (mx > 0.f) (void)frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
        sh = 11 - e;                         // ||x|| * 2^sh < 2^14.5
        ss = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          xv[i] = ldexpf(xv[i], sh);
          ss = fmaf(xv[i], xv[i], ss);
        }
        ss = sum8(ss);
      }
      if (sq == 0) {
        const float nr = sqrtf(ss);
        n_s[par][sv] = ldexpf(nr, -sh);
        // the rotation product is kPiScale Pi x (dense) or sqrt(d) Pi_H x (HAD)
        static_assert(kD == 128, "sqrt(kD) below");
        constexpr float kRotScale = HAD ? 11.313708498984761f : kPiScale;
        rinv_s[par][sv] = (ss > 0.f) ? (kResScale / kRotScale) * __builtin_amdgcn_rcpf(nr) : 0.f;
      }
      uint32_t wh[8], wl[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const qhalf2 hh = {static_cast<_Float16>(xv[2 * i]), static_cast<_Float16>(xv[2 * i + 1])};
        wh[i] = h2u(hh);
        if constexpr (kSplitX) {
          const qhalf2 ll = {static_cast<_Float16>(xv[2 * i] - static_cast<float>(hh[0])),
                             static_cast<_Float16>(xv[2 * i + 1] - static_cast<float>(hh[1]))};
          wl[i] = h2u(ll);
        }
      }
      uint4* dh = reinterpret_cast<uint4*>(&xs[xb][0][sv][16 * sq]);
      dh[0] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
      dh[1] = make_uint4(wh[4], wh[5], wh[6], wh[7]);
      if constexpr (kSplitX) {
        uint4* dl = reinterpret_cast<uint4*>(&xs[xb][kXP - 1][sv][16 * sq]);
        dl[0] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
        dl[1] = make_uint4(wl[4], wl[5], wl[6], wl[7]);
      }
    }
    __syncthreads();
    if constexpr (KEY) store_key_norms(par ^ 1);  // the previous unit's
    if constexpr (kAhead2) {
      raw = raw_next;
      load_raw(s2, b2, raw_next);  // the unit after next, in flight during two units' compute
    } else {
      load_raw(s1, b1, raw);  // the next unit, in flight during this unit's compute
    }

    // ---------------- rotation: acc = X Pi^T (x kPiScale, inputs scaled)
    qfloatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const qhalf8 ah = *reinterpret_cast<const qhalf8*>(&xs[xb][0][atok][16 * c + 8 * h]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bph[c], acc, 0, 0, 0);
      if constexpr (!HAD) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bpl[c], acc, 0, 0, 0);
      if constexpr (kSplitX) {
        const qhalf8 al = *reinterpret_cast<const qhalf8*>(&xs[xb][kXP - 1][atok][16 * c + 8 * h]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bph[c], acc, 0, 0, 0);
      }
    }

    // ---------------- quantize: acc[v] is token 16h + v, coordinate 32*wave + c32
    float rv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 r4 = *reinterpret_cast<const float4*>(&rinv_s[par][16 * h + 4 * q]);
      rv[4 * q] = r4.x;
      rv[4 * q + 1] = r4.y;
      rv[4 * q + 2] = r4.z;
      rv[4 * q + 3] = r4.w;
    }
    uint32_t cw0 = 0, cw1 = 0;  // key code words: lane = token + 32 * (plane & 1)
    uint32_t vlo = 0, vhi = 0;  // value fields of tokens 16h .. 16h+15 (bits BITS*v ..)
    float rprev = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float y = acc[v] * rv[v];
      uint64_t P[BITS];
      float C;
      int idx;
      quant_one<BITS>(y, tab, P, C, idx);
      if constexpr (KEY) {
#pragma unroll
        for (int p = 0; p < BITS; ++p) {
          const uint32_t lo = static_cast<uint32_t>(P[p]), hi = static_cast<uint32_t>(P[p] >> 32);
          const int base = 32 * (p & 1);
          if (p < 2) {
            cw0 = writelane(lo, base + v, cw0);
            cw0 = writelane(hi, base + 16 + v, cw0);
          } else {
            cw1 = writelane(lo, base + v, cw1);
            cw1 = writelane(hi, base + 16 + v, cw1);
          }
        }
        // residual x256 (for a zero vector y = 0 and the residual is unused:
        // its signs and rnorm are fixed at the store)
        const float r = y - C;
        if (v & 1) {
          // tokens (v-1, v) of coordinate 32*wave + c32: fp16 hi + lo
          const qhalf2 hh = {static_cast<_Float16>(rprev), static_cast<_Float16>(r)};
          const qhalf2 ll = split_lo(hh, rprev, r);
          const int tk = 16 * h + v - 1, j = 32 * wave + c32;
          rs[0][tk][j] = hh[0];
          rs[0][tk + 1][j] = hh[1];
          rs[1][tk][j] = ll[0];
          rs[1][tk + 1][j] = ll[1];
        }
        rprev = r;
      } else {
        const int sh = BITS * v;
        const uint32_t u = static_cast<uint32_t>(idx);
        if (sh < 32) vlo |= u << sh;
        if (sh + BITS > 32) vhi |= (sh < 32) ? (u >> (32 - sh)) : (u << (sh - 32));
      }
    }

    if constexpr (KEY) {
      {
        const int tk = lane & 31, p = lane >> 5;
        if (p < BITS && tk >= lo) {  // padding tokens get the zero-vector encoding
          uint32_t* dst = codes + ((s * Tp + t0 + tk) * 4 + wave) * BITS;
          dst[p] = cw0;
          if (p + 2 < BITS) dst[p + 2] = cw1;
        }
      }
      __syncthreads();
      // ---------------- sketch Z = R S^T (this wave's 32 sketch rows)
      qfloatx16 z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const qhalf8 ah = *reinterpret_cast<const qhalf8*>(&rs[0][atok][16 * c + 8 * h]);
        const qhalf8 al = *reinterpret_cast<const qhalf8*>(&rs[1][atok][16 * c + 8 * h]);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bsh[c], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bsl[c], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bsh[c], z, 0, 0, 0);
      }
      // ---------------- ||r||^2 over this wave's coordinates: diagonal of R R^T
      // (16x16 tiles: A-row n of tile mt is token 16mt + n; k = 32*wave + 8*(lane/16) + e)
      {
        const int n = lane & 15, g = lane >> 4;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const qhalf8 gh = *reinterpret_cast<const qhalf8*>(&rs[0][16 * mt + n][32 * wave + 8 * g]);
          const qhalf8 gl = *reinterpret_cast<const qhalf8*>(&rs[1][16 * mt + n][32 * wave + 8 * g]);
          qfloatx4 d = {0.f, 0.f, 0.f, 0.f};
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(gh, gh, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(gh, gl, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(gl, gh, d, 0, 0, 0);
          // lane (g, n) holds rows 4g .. 4g+3 of column n: the diagonal when g = n/4
          const int ii = n & 3;
          const float dg = sel(ii & 2, sel(ii & 1, d[3], d[2]), sel(ii & 1, d[1], d[0]));
          if (g == (n >> 2)) rho_s[par][wave][16 * mt + n] = dg;
        }
      }
      uint32_t sw = 0;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint64_t Z = __ballot(z[v] >= 0.f);
        sw = writelane(static_cast<uint32_t>(Z), v, sw);
        sw = writelane(static_cast<uint32_t>(Z >> 32), 16 + v, sw);
      }
      if (lane >= lo && lane < kUnit) {
        // a zero vector (padding included) has every sign bit set
        if (n_s[par][lane] == 0.f) sw = 0xFFFFFFFFu;
        signs[(s * Tp + t0 + lane) * 4 + wave] = sw;
      }
    } else {
      // mask off the fields of padded tokens (zero vectors past the end of T)
      const int nv = nvalid - 16 * h;  // valid tokens of this lane half
      if (nv < 16) {
        const int nbits = nv > 0 ? BITS * nv : 0;
        const uint32_t mlo = nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
        const uint32_t mhi = nbits <= 32 ? 0u : ((1u << (nbits - 32)) - 1u);
        vlo &= mlo;
        vhi &= mhi;
      }
      // lane half h holds record bits [16*BITS*h, 16*BITS*(h+1))
      const int j = 32 * wave + c32;
      uint32_t* dst = codes + ((s * (Tp / kUnit) + blk0 + blk) * kD + j) * BITS;
      // record word q; its bits below BITS*lo belong to kept tokens and are
      // merged from the stored record (only in a block that an append resumes)
      auto put = [&](int q, uint32_t w) {
        const int kb = BITS * lo - 32 * q;
        if (kb > 0) {
          const uint32_t keep = kb >= 32 ? 0xFFFFFFFFu : (1u << kb) - 1u;
          w = (dst[q] & keep) | (w & ~keep);
        }
        dst[q] = w;
      };
      if constexpr (BITS == 1) {
        const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(vlo), 32, 64));
        if (h == 0) put(0, vlo | (other << 16));
      } else if constexpr (BITS == 2) {
        put(h, vlo);
      } else if constexpr (BITS == 3) {
        const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(vlo), 32, 64));
        if (h == 0) {
          put(0, vlo);
          put(1, vhi | (other << 16));
        } else {
          put(2, (vlo >> 16) | (vhi << 16));
        }
      } else {
        put(2 * h, vlo);
        put(2 * h + 1, vhi);
      }
      if (tid >= lo && tid < kUnit) store_norm(norm, norm_dtype, s * Tp + t0 + tid, n_s[par][tid]);
    }
    if constexpr (KEY) {
      pend_base = s * Tp + t0;
      pend_lo = lo;
      pend_n = kUnit;
    }
    s = s1;
    blk = b1;
    s1 = s2;
    b1 = b2;
    advance(s2, b2);
  }
  if constexpr (KEY) {
    __syncthreads();
    store_key_norms(par ^ 1);
  }
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

template <typename XT, bool KEY, bool APPEND, bool HAD>
static void launch_bits(dim3 grid, hipStream_t stream, const tq_tables& t, const void* x,
                        const tq_packed& out, int64_t pos, int64_t n) {
#define TQ_QL(B)                                                                                    \
  hipLaunchKernelGGL((quantize_mfma_kernel<XT, KEY, B, APPEND, HAD>), grid, dim3(kQThreads), 0, stream, t.rot,  \
                     t.sketch, t.centroids, t.bounds, static_cast<const XT*>(x), out.nseq, pos,    \
                     pos + n, stream_stride(out), out.codes, out.signs, out.norm, out.rnorm,       \
                     out.norm_dtype)
  switch (t.bits) {
    case 1: TQ_QL(1); break;
    case 2: TQ_QL(2); break;
    case 3: TQ_QL(3); break;
    default: TQ_QL(4); break;
  }
#undef TQ_QL
}

template <bool APPEND, bool HAD>
static void launch_dtypes(dim3 grid, hipStream_t stream, const tq_tables& t, const void* x, int x_dtype,
                          const tq_packed& out, int64_t pos, int64_t n) {
  const bool key = out.role == TQ_KEY;
  if (x_dtype == TQ_BF16) {
    if (key) launch_bits<uint16_t, true, APPEND, HAD>(grid, stream, t, x, out, pos, n);
    else launch_bits<uint16_t, false, APPEND, HAD>(grid, stream, t, x, out, pos, n);
  } else {
    if (key) launch_bits<float, true, APPEND, HAD>(grid, stream, t, x, out, pos, n);
    else launch_bits<float, false, APPEND, HAD>(grid, stream, t, x, out, pos, n);
  }
}

hipError_t launch_quantize(const tq_tables& t, const void* x, int x_dtype, const tq_packed& out,
                           int64_t pos, int64_t n, bool append, hipStream_t stream) {
  const int64_t nblk = (pos + n + kUnit - 1) / kUnit - pos / kUnit;
  const int64_t units = out.nseq * nblk;
  if (units == 0) return hipSuccess;
  const int64_t cap = (out.role == TQ_KEY ? 2 : 3) * static_cast<int64_t>(device_cus());
  const dim3 grid(static_cast<unsigned>(units < cap ? units : cap));
  const bool had = t.rot_kind == TQ_ROT_HADAMARD;
  if (append) {
    if (had) launch_dtypes<true, true>(grid, stream, t, x, x_dtype, out, pos, n);
    else launch_dtypes<true, false>(grid, stream, t, x, x_dtype, out, pos, n);
  } else {
    if (had) launch_dtypes<false, true>(grid, stream, t, x, x_dtype, out, 0, n);
    else launch_dtypes<false, false>(grid, stream, t, x, x_dtype, out, 0, n);
  }
  return hipGetLastError();
}

}  // namespace tq
