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
//    32x32 output tile per product.  Its slices of Pi and S live in
//    registers as fp16 hi + lo pairs for the whole kernel.
//  * the 32 input vectors are staged in LDS as fp16.  Each vector is first
//    scaled by a power of two that puts its norm just below 2^15: a bf16
//    input is then exact in fp16, an fp32 input is split into fp16 hi + lo.
//    Pi is held x16 so that its lo half stays a normal fp16 number.  The
//    rotation X Pi^T carries about 22 significant bits, fp32-grade.
//  * values: lane l holds coordinate 32w + l%32 of the 16 tokens
//    16*(l/32) + v, v = 0..15 (X Pi^T with A-row r of a tile token
//    16*((r/4)%2) + 4*(r/8) + r%4); every lane packs the b-bit fields of its
//    16 tokens, and the 32-token record of a coordinate is the two lane
//    halves' fields in token order.
//  * keys are computed transposed (Pi X^T, S R^T, the A rows permuted the
//    same way): lane l holds coordinates 32w + 16*(l/32) + v of token l%32,
//    so each lane builds its token's code-plane and sign words itself, one
//    v_alignbit per bit from float sign bits, and sums its residual squares
//    for ||r||^2.  The residual (x256, fp16 hi + lo) goes through LDS, one
//    row per token; the sketch has three products (hi*hi, hi*lo, lo*hi), or
//    two (R_hi S + R_lo S) when S is exact in fp16 (the tables' flag).
//  * kernels: quantize_keys_pipe_kernel and quantize_values_pipe_kernel take
//    whole streams as software pipelines (the vector work of one unit beside
//    the matrix work of another); quantize_mfma_kernel takes appends and
//    split-width value streams unit by unit, with the same arithmetic, so
//    that appended records equal the bulk ones bit for bit.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

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
// Fourth word of a buffer resource for untyped dword loads (DATA_FORMAT 32,
// bits 18:15 = 4): with stride 0 the unit checks each byte offset against
// num_records and returns zeros at or past it.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ uint32_t h2u(qhalf2 h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ qhalf8 qu4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  qu32x4 v = {a, b, c, d};
  return __builtin_bit_cast(qhalf8, v);
}

// v_sqrt_f32: within 1 ulp (6e-8 relative), where sqrtf's correctly rounded
// expansion costs ~15 instructions.  Norms need 1e-6 relative (fp32) or the
// fp16 rounding of the exact value except within 1e-6 of a midpoint, and the
// arguments here are 0 or at least 1 (sums of squares of scaled vectors).
__device__ __forceinline__ float hw_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }

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

// Index of y (x256 scale) = number of boundaries <= y.  With the codebook
// symmetric about 0, the index of a y with its sign bit clear is L/2 + m and
// of one with it set L/2 - 1 - m, m the cell of |y| among the positive
// boundaries: in bits, the top bit is the inverted sign bit and the lower
// bits are m, each XOR the sign bit.  (A -0.0, only from a negative product
// that underflowed, counts as negative like the value it rounds.)
//
// Values: appends the raw bits of one token's field below the bits already
// in w, top bit first -- the sign bit of x, then for each step of the
// magnitude search the sign bit of a rt - t, a = |x|, t the boundary the
// step tests (set for |y| < t: the inverted bit of m).  value_fields turns
// whole words of raw fields into indices.  As in quant_append below, each
// a rt - t is one fma whose sign bit is exactly the compare.
template <int BITS>
__device__ __forceinline__ void value_append(float x, float rt, const QTab<BITS>& tab, uint32_t& w) {
  auto push = [&](float v) { w = __builtin_amdgcn_alignbit(w, __float_as_uint(v), 31); };
  const float a = fabsf(x);
  push(x);
  if constexpr (BITS == 2) {
    push(fmaf(a, rt, -tab.tpos[0]));
  } else if constexpr (BITS == 3) {
    const float d1 = fmaf(a, rt, -tab.tpos[1]);
    const float d2 = fmaf(a, rt, -sel(d1 >= 0.f, tab.tpos[2], tab.tpos[0]));
    push(d1);
    push(d2);
  } else if constexpr (BITS == 4) {
    const float d1 = fmaf(a, rt, -tab.tpos[3]);
    const bool m1 = d1 >= 0.f;
    const float d2 = fmaf(a, rt, -sel(m1, tab.tpos[5], tab.tpos[1]));
    const bool m2 = d2 >= 0.f;
    const float d3 = fmaf(a, rt, -sel(m1, sel(m2, tab.tpos[6], tab.tpos[4]), sel(m2, tab.tpos[2], tab.tpos[0])));
    push(d1);
    push(d2);
    push(d3);
  }
}

// the top bit of each of n fields of `bits` bits
constexpr uint32_t field_tops(int bits, int n) {
  uint32_t m = 0u;
  for (int f = 0; f < n; ++f) m |= 1u << (bits * f + bits - 1);
  return m;
}

// Indices from N raw fields of BITS bits at the bottom of r: each field's
// lower bits XOR its top bit (t - (t >> (BITS-1)) copies every top bit of t
// into the bits below it in its field), then every field bit inverted.
template <int BITS, int N>
__device__ __forceinline__ uint32_t value_fields(uint32_t r) {
  static_assert(BITS * N <= 32, "one word");
  constexpr uint32_t kValid = BITS * N == 32 ? 0xFFFFFFFFu : (1u << (BITS * N % 32)) - 1u;
  if constexpr (BITS == 1) {
    return r ^ kValid;
  } else {
    const uint32_t t = r & field_tops(BITS, N);
    return r ^ (t - (t >> (BITS - 1))) ^ kValid;
  }
}

// The same index for keys in the transposed layout (one token per lane),
// of y = x rt (x the rotation output, rt > 0 its token's scale, or 0 for a
// zero vector, whose x is +0): appends one bit per plane below the bits
// already in pw[] -- pw[BITS-1] <- the sign bit of x, which is y's (the
// sign plane, inverted: set for y's sign bit clear), pw[p] <- the sign bit
// of a rt - t, a = |x|, for the boundary t the magnitude search tested for
// plane p.  The inverted plane bit is that XOR the sign bit of x (set for
// [|y| >= t] XNOR [y's sign bit clear]); code_words applies the XOR to
// whole words.  Each a rt - t is one fma, never -0 or NaN for finite inputs
// (the exact difference is 0 or far above the smallest denormal), so its
// sign bit is exactly |y| < t, the compare the index is defined by.  Returns the
// signed centroid through C (x's sign, so -0.0 gives -mag).
template <int BITS>
__device__ __forceinline__ void quant_append(float x, float rt, const QTab<BITS>& tab, uint32_t* pw, float& C) {
  const uint32_t yb = __float_as_uint(x);
  const float a = fabsf(x);
  auto push = [&](int p, uint32_t bits) { pw[p] = __builtin_amdgcn_alignbit(pw[p], bits, 31); };
  push(BITS - 1, yb);
  float mag;
  if constexpr (BITS == 1) {
    mag = tab.cpos[0];
  } else if constexpr (BITS == 2) {
    const float d1 = fmaf(a, rt, -tab.tpos[0]);
    push(0, __float_as_uint(d1));
    mag = sel(d1 >= 0.f, tab.cpos[1], tab.cpos[0]);
  } else if constexpr (BITS == 3) {
    const float d1 = fmaf(a, rt, -tab.tpos[1]);
    const bool m1 = d1 >= 0.f;
    const float d2 = fmaf(a, rt, -sel(m1, tab.tpos[2], tab.tpos[0]));
    const bool m2 = d2 >= 0.f;
    push(1, __float_as_uint(d1));
    push(0, __float_as_uint(d2));
    mag = sel(m1, sel(m2, tab.cpos[3], tab.cpos[2]), sel(m2, tab.cpos[1], tab.cpos[0]));
  } else {
    const float d1 = fmaf(a, rt, -tab.tpos[3]);
    const bool m1 = d1 >= 0.f;
    const float d2 = fmaf(a, rt, -sel(m1, tab.tpos[5], tab.tpos[1]));
    const bool m2 = d2 >= 0.f;
    const float d3 = fmaf(a, rt, -sel(m1, sel(m2, tab.tpos[6], tab.tpos[4]), sel(m2, tab.tpos[2], tab.tpos[0])));
    const bool m3 = d3 >= 0.f;
    push(2, __float_as_uint(d1));
    push(1, __float_as_uint(d2));
    push(0, __float_as_uint(d3));
    const float lo4 = sel(m2, sel(m3, tab.cpos[3], tab.cpos[2]), sel(m3, tab.cpos[1], tab.cpos[0]));
    const float hi4 = sel(m2, sel(m3, tab.cpos[7], tab.cpos[6]), sel(m3, tab.cpos[5], tab.cpos[4]));
    mag = sel(m1, hi4, lo4);
  }
  C = copysignf(mag, x);
}

// y - C for y = x rt, one v_fma_f32 with the addend negated by a source
// modifier (the compiler would otherwise negate C with a separate XOR to
// use the accumulating form); the result is a value of its own, so that its
// fp16 rounding is one v_cvt_pk_f16_f32 per pair rather than a fused
// fma_mix per value
__device__ __forceinline__ float residual(float x, float rt, float C) {
#if defined(__HIP_DEVICE_COMPILE__)
  float r;
  asm("v_fma_f32 %0, %1, %2, -%3" : "=v"(r) : "v"(x), "v"(rt), "v"(C));
  return r;
#else
  return fmaf(x, rt, -C);
#endif
}

// The code-plane words of the lane's token from quant_append's bits (16
// coordinates per lane half): each lower plane XOR the sign plane, lane half
// 0 taking half 1's 16 bits on top, the inversion undone.
template <int B>
__device__ __forceinline__ void code_words(const uint32_t (&pw)[B], uint32_t (&cw)[B]) {
#pragma unroll
  for (int p = 0; p < B; ++p) {
    const uint32_t w = p + 1 < B ? pw[p] ^ pw[B - 1] : pw[p];
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(w), 32, 64));
    cw[p] = ~((w & 0xFFFFu) | (o << 16));
  }
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

template <int W>
using Width = std::integral_constant<int, W>;

// APPEND: the stream already holds tokens below pos (a separate instance, so
// that the whole-stream launches carry none of the merge code).  HAD: Pi is
// a randomized Walsh-Hadamard rotation, whose sqrt(d) Pi has entries +-1:
// one fp16 product rotates exactly, where a general Pi needs hi + lo.
// MIX: a split (fractional-width) stream -- coordinates 0..63, the words of
// waves 0 and 1, take BITS + 1 bits from the second codebook (cent_hi,
// bnd_hi), coordinates 64..127 BITS bits; each word (keys) or coordinate
// (values) keeps its own width in the records.
template <typename XT, bool KEY, int BITS, bool APPEND, bool HAD, bool MIX = false>
__global__ __launch_bounds__(kQThreads, KEY ? 2 : 3) void quantize_mfma_kernel(
    const float* __restrict__ rot, const float* __restrict__ sketch,
    const float* __restrict__ cent, const float* __restrict__ bnd, const XT* __restrict__ x,
    int64_t nseq, int64_t pos_arg, int64_t T, int64_t Tp, uint32_t* __restrict__ codes,
    uint32_t* __restrict__ signs,
    void* __restrict__ norm, void* __restrict__ rnorm, int norm_dtype,
    const float* __restrict__ cent_hi = nullptr, const float* __restrict__ bnd_hi = nullptr) {
  static_assert(!MIX || BITS + 1 <= 4, "split streams widen BITS by one, up to 4");
  constexpr int BW = MIX ? BITS + 1 : BITS;   // width of the leading coordinates
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
  QTab<BW> tabw;   // the leading coordinates' table (MIX only)
  if constexpr (MIX) {
    constexpr int kHalfW = (1 << BW) / 2;
#pragma unroll
    for (int i = 0; i < kHalfW; ++i) tabw.cpos[i] = cent_hi[kHalfW + i] * kResScale;
#pragma unroll
    for (int i = 0; i + 1 < kHalfW; ++i) tabw.tpos[i] = bnd_hi[kHalfW + i] * kResScale;
  }
  // record words per token (keys) / per block (values), and where this
  // wave's word (keys) or coordinate c32 (values) starts in the record
  constexpr int kKeyRec = MIX ? 4 * BITS + 2 : 4 * BITS;
  constexpr int kValRec = MIX ? kD * BITS + kD / 2 : kD * BITS;
  const bool wide = MIX && wave < 2;

  // 32x32 tile row / column c32 <-> token or coordinate atok: output register
  // v of lane half h is tile row 8(v/4) + 4h + v%4, and atok of that row is
  // 16h + v
  const int atok = 16 * ((c32 >> 2) & 1) + 4 * (c32 >> 3) + (c32 & 3);
  // Pi fragments for coordinates j and (keys) S fragments for sketch rows
  // i = j; K-step c covers input index 16c + 8h + e.  Values: B = Pi^T with
  // j = 32*wave + c32 (output column = coordinate).  Keys: A = Pi with
  // j = 32*wave + atok (output row = coordinate, permuted so that register v
  // of lane half h is coordinate 32*wave + 16h + v).
  qhalf8 bph[8], bpl[HAD ? 1 : 8];
  qhalf8 bsh[KEY ? 8 : 1], bsl[KEY ? 8 : 1];
  {
    const int j = 32 * wave + (KEY ? atok : c32);
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
  // staging role: token sv, elements 16*sq .. 16*sq+15
  const int sv = tid >> 3, sq = tid & 7;
  // (sequence, block) of the first unit and the per-iteration step
  const int64_t step_s = gridDim.x / nblk, step_b = gridDim.x % nblk;
  int64_t s = blockIdx.x / nblk, blk = blockIdx.x % nblk;

  const uint32_t voff = static_cast<uint32_t>((sv * kD + 16 * sq) * static_cast<int>(sizeof(XT)));
  auto load_raw = [&](int64_t us, int64_t ub, RawX<XT>& raw) {
    const int64_t tb = (blk0 + ub) * kUnit;
    if (us < nseq && tb >= pos && tb + kUnit <= T) {
      // the whole unit is input (the condition is the same for every thread):
      // buffer loads from one resource for the workgroup (a form of their
      // own, which keeps the per-thread checks and zero fill below off this
      // path)
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<XT*>(x + (us * nx + tb - pos) * kD), 0, kUnit * kD * static_cast<int>(sizeof(XT)),
          kBufferWord3);
#pragma unroll
      for (int r = 0; r < RawX<XT>::kWords; ++r)
        raw.w[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + 16 * r, 0, 0));
      return;
    }
    // a unit at the ends of the input: each thread loads its own token if
    // it is input, else zeros
    const int64_t t = tb + sv;
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
      store_norm(rnorm, norm_dtype, pend_base + tid, nx * (hw_sqrt(rho2) / kResScale));
    }
  };

  // One unit of work.  par, the unit's parity (a constant per call), picks
  // the LDS buffers; cur holds the unit's input.  The loop below takes two
  // units per iteration, so that with two units of input in flight the two
  // register buffers trade roles rather than being copied.
  auto unit_step = [&](auto pc, RawX<XT>& cur) {
    constexpr int par = decltype(pc)::value;
    const int xb = KEY ? 0 : par;
    const int64_t t0 = (blk0 + blk) * kUnit;
    const int nvalid = static_cast<int>((T - t0 < kUnit) ? T - t0 : kUnit);
    const int lo = pos > t0 ? static_cast<int>(pos - t0) : 0;  // tokens t0 .. t0+lo-1 are kept

    // ---------------- stage: norms, power-of-two range scale, fp16 copy
    {
      float xv[16];
      unpack_raw<XT>(cur, xv);
      float ss = sum8(sumsq16<XT>(cur, xv));
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
        const float nr = hw_sqrt(ss);
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
    // cur is free once staged: it takes the unit after next (bf16: in flight
    // during two units' compute) or the next unit (fp32: during this one's)
    if constexpr (kAhead2) load_raw(s2, b2, cur);
    else load_raw(s1, b1, cur);

    // ---------------- rotation (x kPiScale, inputs scaled).  Values:
    // acc = X Pi^T, acc[v] = token 16h + v of coordinate 32*wave + c32.
    // Keys: acc = Pi X^T, acc[v] = coordinate 32*wave + 16h + v of token c32.
    qfloatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const qhalf8 xh = *reinterpret_cast<const qhalf8*>(&xs[xb][0][KEY ? c32 : atok][16 * c + 8 * h]);
      if constexpr (KEY) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bph[c], xh, acc, 0, 0, 0);
        if constexpr (!HAD) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bpl[c], xh, acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, bph[c], acc, 0, 0, 0);
        if constexpr (!HAD) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, bpl[c], acc, 0, 0, 0);
      }
      if constexpr (kSplitX) {
        const qhalf8 xl = *reinterpret_cast<const qhalf8*>(&xs[xb][kXP - 1][KEY ? c32 : atok][16 * c + 8 * h]);
        if constexpr (KEY) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bph[c], xl, acc, 0, 0, 0);
        else acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl, bph[c], acc, 0, 0, 0);
      }
    }

    if constexpr (KEY) {
      // ---------------- quantize (keys): acc[v] is coordinate 32*wave + 16h + v
      // of token c32.  Descending v appends each plane bit below the ones
      // before it, so after 16 steps coordinate 16h + v sits at bit v.
      const float rt = rinv_s[par][c32];
      auto quantize_key_word = [&](auto wc, const auto& tb) {
      constexpr int WB = decltype(wc)::value;
      uint32_t pw[WB];   // code planes, inverted, coordinates 16h .. 16h+15
#pragma unroll
      for (int p = 0; p < WB; ++p) pw[p] = 0u;
      uint32_t hw[8], lw[8];   // residual (x256) as fp16 hi / lo pairs of coordinates (2i, 2i+1)
      float rr = 0.f;          // sum of the residual squares (x256^2)
      float rodd = 0.f;
#pragma unroll
      for (int v = 15; v >= 0; --v) {
        float C;
        quant_append<WB>(acc[v], rt, tb, pw, C);
        // residual x256 (for a zero vector y = 0 and the residual is unused:
        // its signs and rnorm are fixed at the store)
        const float r = residual(acc[v], rt, C);
        rr = fmaf(r, r, rr);
        if (v & 1) {
          rodd = r;
        } else {
          const qhalf2 hh = {static_cast<_Float16>(r), static_cast<_Float16>(rodd)};
          hw[v / 2] = h2u(hh);
          lw[v / 2] = h2u(split_lo(hh, r, rodd));
        }
      }
      // residual rows rs[hi / lo][token c32][coordinates 32*wave + 16h ..]
      {
        uint4* dh = reinterpret_cast<uint4*>(&rs[0][c32][32 * wave + 16 * h]);
        uint4* dl = reinterpret_cast<uint4*>(&rs[1][c32][32 * wave + 16 * h]);
        dh[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        dh[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        dl[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        dl[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
      }
      // code words of token c32
      uint32_t cw[WB];
      code_words<WB>(pw, cw);
      // ||r||^2 over this wave's 32 coordinates
      const float rr32 = rr + __shfl_xor(rr, 32, 64);
      if (h == 0) {
        rho_s[par][wave][c32] = rr32;
        if (c32 >= lo) {  // padding tokens get the zero-vector encoding
          // this wave's word: after the planes of the words before it
          const int woff = wave * BITS + (MIX ? (wave < 2 ? wave : 2) : 0);
          uint32_t* dst = codes + (s * Tp + t0 + c32) * kKeyRec + woff;
#pragma unroll
          for (int p = 0; p < WB; ++p) dst[p] = cw[p];
        }
      }
      };
      if (wide) quantize_key_word(Width<BW>{}, tabw);
      else quantize_key_word(Width<BITS>{}, tab);
      __syncthreads();
      // ---------------- sketch Z^T = S R^T: z[v] is sketch row 32*wave + 16h + v
      // of token c32
      qfloatx16 z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const qhalf8 rh = *reinterpret_cast<const qhalf8*>(&rs[0][c32][16 * c + 8 * h]);
        const qhalf8 rl = *reinterpret_cast<const qhalf8*>(&rs[1][c32][16 * c + 8 * h]);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsh[c], rh, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsl[c], rh, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsh[c], rl, z, 0, 0, 0);
      }
      // sign bits, appended inverted from the float sign bits (z = -0.0, which
      // only an all-zero residual can give, reads as negative; it lies in the
      // parity band |z| <= 1e-5 either way)
      uint32_t sw = 0u;
#pragma unroll
      for (int v = 15; v >= 0; --v) sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(z[v]), 31);
      const uint32_t so = static_cast<uint32_t>(__shfl_xor(static_cast<int>(sw), 32, 64));
      if (h == 0 && c32 >= lo) {
        uint32_t word = ~((sw & 0xFFFFu) | (so << 16));
        // a zero vector (padding included) has every sign bit set
        if (n_s[par][c32] == 0.f) word = 0xFFFFFFFFu;
        signs[(s * Tp + t0 + c32) * 4 + wave] = word;
      }
    } else {
      // ---------------- quantize (values): acc[v] is token 16h + v of
      // coordinate 32*wave + c32
      // the record of coordinate j = 32*wave + c32: WB words, after the
      // records of the coordinates before it
      auto quantize_value_coord = [&](auto wc, const auto& tb) {
      constexpr int WB = decltype(wc)::value;
      // value fields of tokens 16h .. 16h+15 at bits WB*v of (vhi:vlo).  The
      // raw fields are appended top token first, so token v ends at bit WB*v
      // of its word: one word for WB <= 2; tokens 0..9 and 10..15 for WB = 3
      // (the word boundary splits token 10), 0..7 and 8..15 for WB = 4.
      constexpr int kLo = WB <= 2 ? 16 : (WB == 3 ? 10 : 8);
      // (the tokens' scales are read four at a time as they are needed)
      uint32_t wl = 0u, wh = 0u;
      float4 r4;
#pragma unroll
      for (int v = 15; v >= 0; --v) {
        if (v % 4 == 3) r4 = *reinterpret_cast<const float4*>(&rinv_s[par][16 * h + v - 3]);
        const float rt = v % 4 == 0 ? r4.x : v % 4 == 1 ? r4.y : v % 4 == 2 ? r4.z : r4.w;
        value_append<WB>(acc[v], rt, tb, v >= kLo ? wh : wl);
      }
      uint32_t vlo = value_fields<WB, kLo>(wl), vhi = 0u;
      if constexpr (WB == 3) {
        wh = value_fields<WB, 16 - kLo>(wh);
        vlo |= wh << 30;
        vhi = wh >> 2;
      } else if constexpr (WB == 4) {
        vhi = value_fields<WB, 16 - kLo>(wh);
      }
      // mask off the fields of padded tokens (zero vectors past the end of T)
      const int nv = nvalid - 16 * h;  // valid tokens of this lane half
      if (nv < 16) {
        const int nbits = nv > 0 ? WB * nv : 0;
        const uint32_t mlo = nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
        const uint32_t mhi = nbits <= 32 ? 0u : ((1u << (nbits - 32)) - 1u);
        vlo &= mlo;
        vhi &= mhi;
      }
      // lane half h holds record bits [16*WB*h, 16*WB*(h+1))
      const int j = 32 * wave + c32;
      const int joff = MIX ? (j < kD / 2 ? j * BW : (kD / 2) * BW + (j - kD / 2) * BITS) : j * BITS;
      uint32_t* dst = codes + (s * (Tp / kUnit) + blk0 + blk) * kValRec + joff;
      // record word q; its bits below WB*lo belong to kept tokens and are
      // merged from the stored record (only in a block that an append resumes)
      auto put = [&](int q, uint32_t w) {
        const int kb = WB * lo - 32 * q;
        if (kb > 0) {
          const uint32_t keep = kb >= 32 ? 0xFFFFFFFFu : (1u << kb) - 1u;
          w = (dst[q] & keep) | (w & ~keep);
        }
        dst[q] = w;
      };
      if constexpr (WB == 1) {
        const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(vlo), 32, 64));
        if (h == 0) put(0, vlo | (other << 16));
      } else if constexpr (WB == 2) {
        put(h, vlo);
      } else if constexpr (WB == 3) {
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
      };
      if (wide) quantize_value_coord(Width<BW>{}, tabw);
      else quantize_value_coord(Width<BITS>{}, tab);
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
  };

  RawX<XT>& raw_odd = kAhead2 ? raw_next : raw;
  int last = 1;  // parity of the last unit taken (none: 1, whose norms are pending for no token)
  for (int64_t unit = blockIdx.x; unit < units; unit += 2 * static_cast<int64_t>(gridDim.x)) {
    unit_step(Width<0>{}, raw);
    last = 0;
    if (unit + gridDim.x >= units) break;
    unit_step(Width<1>{}, raw_odd);
    last = 1;
  }
  if constexpr (KEY) {
    __syncthreads();
    store_key_norms(last);
  }
}

// ---------------------------------------------------------------------------
// Staging of the pipelined kernels: the 8 threads of a token each take 16
// of its elements (raw), write the fp16 copy (fp32 input: hi and lo) to
// LDS rows xh / xl at their elements, and the token's norm and rotation
// scale to n_dst / rinv_dst (every thread of the token writes the same
// values, so that no branch splits the block).
//
// Common path (||x|| in [1, 2^14): no rescaling): returns whether the token
// needs rescaling.
template <typename XT, bool HAD>
__device__ __forceinline__ bool stage_share_common(const RawX<XT>& raw, _Float16* xh, _Float16* xl,
                                                   float* n_dst, float* rinv_dst) {
  constexpr bool kSplitX = sizeof(XT) == 4;
  static_assert(kD == 128, "sqrt(kD) below");
  constexpr float kRotScale = HAD ? 11.313708498984761f : kPiScale;   // sqrt(128) or 16
  float xv[16];
  unpack_raw<XT>(raw, xv);
  const float ss = sum8(sumsq16<XT>(raw, xv));
  const float nr = hw_sqrt(ss);
  *n_dst = nr;
  *rinv_dst = (ss > 0.f) ? (kResScale / kRotScale) * __builtin_amdgcn_rcpf(nr) : 0.f;
  uint32_t wh[8], wl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const qhalf2 hh = {static_cast<_Float16>(xv[2 * e]), static_cast<_Float16>(xv[2 * e + 1])};
    wh[e] = h2u(hh);
    if constexpr (kSplitX) {
      const qhalf2 ll = {static_cast<_Float16>(xv[2 * e] - static_cast<float>(hh[0])),
                         static_cast<_Float16>(xv[2 * e + 1] - static_cast<float>(hh[1]))};
      wl[e] = h2u(ll);
    }
  }
  uint4* dh = reinterpret_cast<uint4*>(xh);
  dh[0] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
  dh[1] = make_uint4(wh[4], wh[5], wh[6], wh[7]);
  if constexpr (kSplitX) {
    uint4* dl = reinterpret_cast<uint4*>(xl);
    dl[0] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    dl[1] = make_uint4(wl[4], wl[5], wl[6], wl[7]);
  }
  return !(ss >= 1.f && ss < 0x1p28f);
}

// Staging of a unit with at least one token outside that range: the general
// path of quantize_mfma_kernel, for every token (the tokens in range take
// sh = 0 and rewrite what stage_share_common wrote).
template <typename XT, bool HAD>
__device__ __forceinline__ void stage_share_general(const RawX<XT>& raw, _Float16* xh, _Float16* xl,
                                                    float* n_dst, float* rinv_dst) {
  constexpr bool kSplitX = sizeof(XT) == 4;
  constexpr float kRotScale = HAD ? 11.313708498984761f : kPiScale;
  float xv[16];
  unpack_raw<XT>(raw, xv);
  float ss = sum8(sumsq16<XT>(raw, xv));
  int sh;
  if (ss >= 1.f && ss < 0x1p28f) {
    sh = 0;
  } else if (ss >= 0x1p-100f && ss <= 0x1p100f) {
    int e;
    (void)frexpf(ss, &e);
    sh = 15 - ((e + 1) >> 1);
    const float f = pow2f(sh);
#pragma unroll
    for (int i = 0; i < 16; ++i) xv[i] *= f;
    ss *= f * f;
  } else {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(xv[i]));
    mx = max8(mx);
    int e = 0;
    if (mx > 0.f) (void)frexpf(mx, &e);
    sh = 11 - e;
    ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xv[i] = ldexpf(xv[i], sh);
      ss = fmaf(xv[i], xv[i], ss);
    }
    ss = sum8(ss);
  }
  const float nr = hw_sqrt(ss);
  *n_dst = ldexpf(nr, -sh);
  *rinv_dst = (ss > 0.f) ? (kResScale / kRotScale) * __builtin_amdgcn_rcpf(nr) : 0.f;
  uint32_t wh[8], wl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const qhalf2 hh = {static_cast<_Float16>(xv[2 * e]), static_cast<_Float16>(xv[2 * e + 1])};
    wh[e] = h2u(hh);
    if constexpr (kSplitX) {
      const qhalf2 ll = {static_cast<_Float16>(xv[2 * e] - static_cast<float>(hh[0])),
                         static_cast<_Float16>(xv[2 * e + 1] - static_cast<float>(hh[1]))};
      wl[e] = h2u(ll);
    }
  }
  uint4* dh = reinterpret_cast<uint4*>(xh);
  dh[0] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
  dh[1] = make_uint4(wh[4], wh[5], wh[6], wh[7]);
  if constexpr (kSplitX) {
    uint4* dl = reinterpret_cast<uint4*>(xl);
    dl[0] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    dl[1] = make_uint4(wl[4], wl[5], wl[6], wl[7]);
  }
}

// Keys, whole stream: the same arithmetic as quantize_mfma_kernel, arranged
// as a software pipeline so that each wave issues matrix-core and vector
// work of different units side by side.  Iteration i of a workgroup, one
// barrier at its end:
//   phase 1: sketch of unit i-1 (24 MFMAs on the residual staged in LDS; 16
//            when S is exact in fp16, SLO = false) with the quantization of
//            unit i (the vector ALU on the rotation computed in iteration
//            i-1: plane bits, residual into LDS);
//   phase 2: rotation of unit i+1 (16 MFMAs on its staged input) with the
//            sign bits of unit i-1 and the staging of unit i+2 (norm, range
//            test, float16 copy into LDS).
// Residual and input staging are double-buffered by unit parity, the
// per-token scales ring over 4 units, so one barrier per unit orders every
// LDS reuse.  Stores and the (rare) out-of-range rescaling happen between
// the phases, so that each phase is one straight block of code.
// MIX: a split stream, as in quantize_mfma_kernel: waves 0 and 1
// (coordinates 0..63) quantize with BITS + 1 planes from the second
// codebook, and every word keeps its own width in the record.
template <typename XT, int BITS, bool HAD, bool MIX = false, bool SLO = true>
__global__ __launch_bounds__(kQThreads, 2) void quantize_keys_pipe_kernel(
    const float* __restrict__ rot, const float* __restrict__ sketch,
    const float* __restrict__ cent, const float* __restrict__ bnd, const XT* __restrict__ x,
    uint32_t nblk, uint32_t units, int64_t T, int64_t Tp, uint32_t* __restrict__ codes,
    uint32_t* __restrict__ signs, void* __restrict__ norm, void* __restrict__ rnorm,
    int norm_dtype, const float* __restrict__ cent_hi = nullptr, const float* __restrict__ bnd_hi = nullptr) {
  static_assert(!MIX || (BITS + 1 <= 4 && !HAD), "split streams: dense rotation, BITS + 1 up to 4");
  constexpr int BW = MIX ? BITS + 1 : BITS;   // width of the leading coordinates' words
  constexpr int kKeyRec = MIX ? 4 * BITS + 2 : 4 * BITS;   // record words per token
  constexpr bool kSplitX = sizeof(XT) == 4;
  constexpr int kXP = kSplitX ? 2 : 1;
  __shared__ __align__(16) _Float16 xs[2][kXP][kUnit][kRowH];   // staged input, by unit parity
  __shared__ __align__(16) _Float16 rs[2][2][kUnit][kRowH];     // residual hi / lo, by unit parity
  __shared__ __align__(16) float rinv_s[4][kUnit];              // per-token scale, ring of 4 units
  __shared__ float n_s[4][kUnit];                               // ||x||, ring of 4 units
  __shared__ float rho_s[2][4][kUnit];                          // per-wave ||r||^2 (x256^2), by parity

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, h = lane >> 5;
  const int sv = tid >> 3, sq = tid & 7;   // staging role: token sv, elements 16 sq ..

  QTab<BITS> tab;
  constexpr int kHalf = (1 << BITS) / 2;
#pragma unroll
  for (int i = 0; i < kHalf; ++i) tab.cpos[i] = cent[kHalf + i] * kResScale;
#pragma unroll
  for (int i = 0; i + 1 < kHalf; ++i) tab.tpos[i] = bnd[kHalf + i] * kResScale;
  if constexpr (BITS == 1) tab.tpos[0] = 0.f;
  QTab<BW> tabw;   // the leading coordinates' table (MIX only)
  if constexpr (MIX) {
    constexpr int kHalfW = (1 << BW) / 2;
#pragma unroll
    for (int i = 0; i < kHalfW; ++i) tabw.cpos[i] = cent_hi[kHalfW + i] * kResScale;
#pragma unroll
    for (int i = 0; i + 1 < kHalfW; ++i) tabw.tpos[i] = bnd_hi[kHalfW + i] * kResScale;
  }
  const int woff = wave * BITS + (MIX ? (wave < 2 ? wave : 2) : 0);   // this wave's word in a record

  // A = Pi rows / S rows, permuted as in quantize_mfma_kernel (keys)
  const int atok = 16 * ((c32 >> 2) & 1) + 4 * (c32 >> 3) + (c32 & 3);
  qhalf8 bph[8], bpl[HAD ? 1 : 8], bsh[8], bsl[8];
  {
    const int j = 32 * wave + atok;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (HAD) sign_frag(rot + j * kD + 16 * c + 8 * h, bph[c]);
      else split_frag(rot + j * kD + 16 * c + 8 * h, kPiScale, bph[c], bpl[c]);
      split_frag(sketch + j * kD + 16 * c + 8 * h, 1.f, bsh[c], bsl[c]);
    }
  }

  const uint32_t g0 = blockIdx.x, gstep = gridDim.x;
  const int n_units = static_cast<int>((units - g0 + gstep - 1) / gstep);   // >= 1 (grid <= units)
  // first token (sequence * Tp + token) of the workgroup's unit i
  auto unit_base = [&](int i) -> int64_t {
    const uint32_t g = g0 + static_cast<uint32_t>(i) * gstep;
    const uint32_t s = g / nblk, b = g - s * nblk;
    return static_cast<int64_t>(s) * Tp + static_cast<int64_t>(b) * kUnit;
  };
  // loads of unit i's staging share, through a buffer resource over the
  // unit's rows that exist (none for a unit past the workgroup's last): the
  // hardware returns zeros for the rows at or past T, the padding tokens,
  // which then stage as zero vectors.  Every lane issues the same loads, so
  // the waits count a fixed number of them.
  auto load_unit = [&](int i, RawX<XT>& raw) {
    const bool unit_ok = i < n_units;
    const uint32_t g = g0 + static_cast<uint32_t>(unit_ok ? i : 0) * gstep;
    const uint32_t s = g / nblk, b = g - s * nblk;
    const int64_t r0 = static_cast<int64_t>(b) * kUnit;
    const int nrows = !unit_ok ? 0 : (T - r0 < kUnit ? static_cast<int>(T - r0) : kUnit);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<XT*>(x + (static_cast<int64_t>(s) * T + r0) * kD), 0,
        nrows * kD * static_cast<int>(sizeof(XT)), kBufferWord3);
    const uint32_t voff = static_cast<uint32_t>((sv * kD + 16 * sq) * static_cast<int>(sizeof(XT)));
#pragma unroll
    for (int r = 0; r < RawX<XT>::kWords; ++r)
      raw.w[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + 16 * r, 0, 0));
  };
  auto stage_common = [&](const RawX<XT>& raw, int slot, int buf) -> bool {
    return stage_share_common<XT, HAD>(raw, &xs[buf][0][sv][16 * sq], &xs[buf][kXP - 1][sv][16 * sq],
                                       &n_s[slot][sv], &rinv_s[slot][sv]);
  };
  auto stage_general = [&](const RawX<XT>& raw, int slot, int buf) {
    stage_share_general<XT, HAD>(raw, &xs[buf][0][sv][16 * sq], &xs[buf][kXP - 1][sv][16 * sq],
                                 &n_s[slot][sv], &rinv_s[slot][sv]);
  };
  auto stage = [&](const RawX<XT>& raw, int slot, int buf) {
    const bool rare = stage_common(raw, slot, buf);
    if (__builtin_amdgcn_ballot_w64(rare) != 0) stage_general(raw, slot, buf);
  };
  // rotation of the unit staged in xs[buf]: acc[v] = coordinate 32 wave + 16 h + v of token c32
  auto rotate = [&](int buf, qfloatx16& acc) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const qhalf8 xh = *reinterpret_cast<const qhalf8*>(&xs[buf][0][c32][16 * c + 8 * h]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bph[c], xh, acc, 0, 0, 0);
      if constexpr (!HAD) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bpl[c], xh, acc, 0, 0, 0);
      if constexpr (kSplitX) {
        const qhalf8 xl = *reinterpret_cast<const qhalf8*>(&xs[buf][kXP - 1][c32][16 * c + 8 * h]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bph[c], xl, acc, 0, 0, 0);
      }
    }
  };
  // norms of unit i (rho_s holds every wave's share of ||r||^2)
  auto store_norms = [&](int i) {
    if (tid < kUnit) {
      const int pp = i & 1, slot = i & 3;
      const float rho2 = rho_s[pp][0][tid] + rho_s[pp][1][tid] + rho_s[pp][2][tid] + rho_s[pp][3][tid];
      const float nx = n_s[slot][tid];
      const int64_t base = unit_base(i);
      store_norm(norm, norm_dtype, base + tid, nx);
      store_norm(rnorm, norm_dtype, base + tid, nx * (hw_sqrt(rho2) / kResScale));
    }
  };

  constexpr bool kTwoSets = !kSplitX;   // bf16: loads two units ahead
  RawX<XT> rawA, rawB;
  // ---- prologue: stage units 0 and 1, loads of units 2 and 3 in flight,
  // rotation of unit 0
  load_unit(0, rawA);
  load_unit(1, rawB);
  stage(rawA, 0, 0);
  stage(rawB, 1, 1);
  load_unit(2, rawA);
  if constexpr (kTwoSets) load_unit(3, rawB);
  __syncthreads();
  qfloatx16 acc, z;
  rotate(0, acc);
  __syncthreads();   // iteration 0 stages unit 2 into the buffer just read
#pragma unroll
  for (int k = 0; k < 16; ++k) z[k] = 0.f;

  auto iteration = [&](int i, RawX<XT>& raw) {
    const int pb = i & 1;
    // ---------------- phase 1: sketch of unit i-1 with the quantization of unit i
    const float rt = rinv_s[i & 3][c32];
#pragma unroll
    for (int k = 0; k < 16; ++k) z[k] = 0.f;
    auto phase1 = [&](auto wc, const auto& tb) {
    constexpr int WB = decltype(wc)::value;
    uint32_t pw[WB];
#pragma unroll
    for (int p = 0; p < WB; ++p) pw[p] = 0u;
    uint32_t hw[8], lw[8];
    float rr = 0.f, rodd = 0.f;
    auto qstep = [&](int v) {
      float C;
      quant_append<WB>(acc[v], rt, tb, pw, C);
      const float r = residual(acc[v], rt, C);
      rr = fmaf(r, r, rr);
      if (v & 1) {
        rodd = r;
      } else {
        const qhalf2 hh = {static_cast<_Float16>(r), static_cast<_Float16>(rodd)};
        hw[v / 2] = h2u(hh);
        lw[v / 2] = h2u(split_lo(hh, r, rodd));
      }
    };
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const qhalf8 rh = *reinterpret_cast<const qhalf8*>(&rs[pb ^ 1][0][c32][16 * c + 8 * h]);
      const qhalf8 rl = *reinterpret_cast<const qhalf8*>(&rs[pb ^ 1][1][c32][16 * c + 8 * h]);
      z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsh[c], rh, z, 0, 0, 0);
      qstep(15 - 2 * c);
      if constexpr (SLO) z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsl[c], rh, z, 0, 0, 0);
      qstep(14 - 2 * c);
      z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsh[c], rl, z, 0, 0, 0);
    }
    {
      uint4* dh = reinterpret_cast<uint4*>(&rs[pb][0][c32][32 * wave + 16 * h]);
      uint4* dl = reinterpret_cast<uint4*>(&rs[pb][1][c32][32 * wave + 16 * h]);
      dh[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      dh[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
      dl[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      dl[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
    }
    uint32_t cw[WB];
    code_words<WB>(pw, cw);
    const float rr32 = rr + __shfl_xor(rr, 32, 64);
    // codes and ||r||^2 share of unit i
    if (h == 0) {
      rho_s[pb][wave][c32] = rr32;
      uint32_t* dst = codes + (unit_base(i) + c32) * kKeyRec + woff;
#pragma unroll
      for (int p = 0; p < WB; ++p) dst[p] = cw[p];
    }
    };
    if constexpr (MIX) {
      if (wave < 2) phase1(Width<BW>{}, tabw);   // uniform
      else phase1(Width<BITS>{}, tab);
    } else {
      phase1(Width<BITS>{}, tab);
    }
    // ---------------- phase 2: rotation of unit i+1 with the sign bits of
    // unit i-1 and the staging of unit i+2
    uint32_t sw = 0u;
#pragma unroll
    for (int v = 15; v >= 0; --v) sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(z[v]), 31);
    const uint32_t so = static_cast<uint32_t>(__shfl_xor(static_cast<int>(sw), 32, 64));
    rotate(pb ^ 1, acc);
    const bool rare = stage_common(raw, (i + 2) & 3, pb);
    if (__builtin_amdgcn_ballot_w64(rare) != 0) stage_general(raw, (i + 2) & 3, pb);
    if (i > 0) {
      if (h == 0) {
        uint32_t word = ~((sw & 0xFFFFu) | (so << 16));
        if (n_s[(i - 1) & 3][c32] == 0.f) word = 0xFFFFFFFFu;   // a zero vector: every sign bit set
        signs[(unit_base(i - 1) + c32) * 4 + wave] = word;
      }
      store_norms(i - 1);
    }
    if constexpr (kTwoSets) load_unit(i + 4, raw);
    else load_unit(i + 3, raw);
    __syncthreads();
  };

  int i = 0;
  if constexpr (kTwoSets) {
    for (; i + 1 < n_units; i += 2) {
      iteration(i, rawA);
      iteration(i + 1, rawB);
    }
    if (i < n_units) {
      iteration(i, rawA);
      ++i;
    }
  } else {
    for (; i < n_units; ++i) iteration(i, rawA);
  }
  // ---- epilogue: sketch and signs of the last unit
  {
    const int last = n_units - 1, pb = last & 1;
#pragma unroll
    for (int k = 0; k < 16; ++k) z[k] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const qhalf8 rh = *reinterpret_cast<const qhalf8*>(&rs[pb][0][c32][16 * c + 8 * h]);
      const qhalf8 rl = *reinterpret_cast<const qhalf8*>(&rs[pb][1][c32][16 * c + 8 * h]);
      z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsh[c], rh, z, 0, 0, 0);
      if constexpr (SLO) z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsl[c], rh, z, 0, 0, 0);
      z = __builtin_amdgcn_mfma_f32_32x32x16_f16(bsh[c], rl, z, 0, 0, 0);
    }
    uint32_t sw = 0u;
#pragma unroll
    for (int v = 15; v >= 0; --v) sw = __builtin_amdgcn_alignbit(sw, __float_as_uint(z[v]), 31);
    const uint32_t so = static_cast<uint32_t>(__shfl_xor(static_cast<int>(sw), 32, 64));
    if (h == 0) {
      uint32_t word = ~((sw & 0xFFFFu) | (so << 16));
      if (n_s[last & 3][c32] == 0.f) word = 0xFFFFFFFFu;
      signs[(unit_base(last) + c32) * 4 + wave] = word;
    }
    store_norms(last);
  }
}

// Values, whole stream: the arithmetic of quantize_mfma_kernel (values) as a
// software pipeline, in the manner of quantize_keys_pipe_kernel.  Iteration
// i of a workgroup, one barrier at its end, is one straight block of code:
// the rotation of unit i+1 (16 MFMAs on its staged input; 8 with the
// Walsh-Hadamard rotation, 24 for fp32 input) beside the quantization of
// unit i (the vector ALU on the rotation computed in iteration i-1) and the
// staging of unit i+2; then the unit's stores, the (rare) out-of-range
// rescaling and the loads of unit i+4 (fp32: i+3).  Staging is
// double-buffered by unit parity and the per-token scales ring over 4
// units, so that one barrier per unit orders every LDS reuse.  It takes
// about 160 VGPRs: 3 workgroups per CU.  (A split stream keeps the
// unit-by-unit kernel: with two widths in one workgroup this one would
// exceed that budget.)
template <typename XT, int BITS, bool HAD>
__global__ __launch_bounds__(kQThreads, 3) void quantize_values_pipe_kernel(
    const float* __restrict__ rot, const float* __restrict__ bnd, const XT* __restrict__ x,
    uint32_t nblk, uint32_t units, int64_t T, int64_t Tp, uint32_t* __restrict__ codes,
    void* __restrict__ norm, int norm_dtype) {
  constexpr int kValRec = kD * BITS;   // record words per block
  constexpr bool kSplitX = sizeof(XT) == 4;
  constexpr int kXP = kSplitX ? 2 : 1;
  __shared__ __align__(16) _Float16 xs[2][kXP][kUnit][kRowH];   // staged input, by unit parity
  __shared__ __align__(16) float rinv_s[4][kUnit];              // per-token scale, ring of 4 units
  __shared__ float n_s[4][kUnit];                               // ||x||, ring of 4 units

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, h = lane >> 5;
  const int sv = tid >> 3, sq = tid & 7;   // staging role: token sv, elements 16 sq ..

  // decision boundaries (x256 scale); values use no centroids
  QTab<BITS> tab;
  constexpr int kHalf = (1 << BITS) / 2;
#pragma unroll
  for (int i = 0; i + 1 < kHalf; ++i) tab.tpos[i] = bnd[kHalf + i] * kResScale;
  if constexpr (BITS == 1) tab.tpos[0] = 0.f;

  // acc = X Pi^T: the A rows are tokens, permuted so that output register v
  // of lane half h is token 16h + v; B = Pi^T, column c32 = coordinate
  // j = 32*wave + c32, as fp16 hi + lo (or the exact +-1 signs of Pi_H)
  const int atok = 16 * ((c32 >> 2) & 1) + 4 * (c32 >> 3) + (c32 & 3);
  const int j = 32 * wave + c32;
  qhalf8 bph[8], bpl[HAD ? 1 : 8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if constexpr (HAD) sign_frag(rot + j * kD + 16 * c + 8 * h, bph[c]);
    else split_frag(rot + j * kD + 16 * c + 8 * h, kPiScale, bph[c], bpl[c]);
  }
  const int joff = j * BITS;   // the record of coordinate j, after those of the coordinates before it

  const uint32_t g0 = blockIdx.x, gstep = gridDim.x;
  const int n_units = static_cast<int>((units - g0 + gstep - 1) / gstep);   // >= 1 (grid <= units)
  // sequence and block of the workgroup's unit i
  auto unit_sb = [&](int i, uint32_t& s, uint32_t& b) {
    const uint32_t g = g0 + static_cast<uint32_t>(i) * gstep;
    s = g / nblk;
    b = g - s * nblk;
  };
  // loads of unit i's staging share through a buffer resource over the
  // unit's rows that exist (none past the workgroup's last unit): the rows
  // at or past T read as zeros and stage as zero vectors
  const uint32_t voff = static_cast<uint32_t>((sv * kD + 16 * sq) * static_cast<int>(sizeof(XT)));
  auto load_unit = [&](int i, RawX<XT>& raw) {
    const bool unit_ok = i < n_units;
    uint32_t s, b;
    unit_sb(unit_ok ? i : 0, s, b);
    const int64_t r0 = static_cast<int64_t>(b) * kUnit;
    const int nrows = !unit_ok ? 0 : (T - r0 < kUnit ? static_cast<int>(T - r0) : kUnit);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<XT*>(x + (static_cast<int64_t>(s) * T + r0) * kD), 0,
        nrows * kD * static_cast<int>(sizeof(XT)), kBufferWord3);
#pragma unroll
    for (int r = 0; r < RawX<XT>::kWords; ++r)
      raw.w[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + 16 * r, 0, 0));
  };
  auto stage_common = [&](const RawX<XT>& raw, int slot, int buf) -> bool {
    return stage_share_common<XT, HAD>(raw, &xs[buf][0][sv][16 * sq], &xs[buf][kXP - 1][sv][16 * sq],
                                       &n_s[slot][sv], &rinv_s[slot][sv]);
  };
  auto stage_general = [&](const RawX<XT>& raw, int slot, int buf) {
    stage_share_general<XT, HAD>(raw, &xs[buf][0][sv][16 * sq], &xs[buf][kXP - 1][sv][16 * sq],
                                 &n_s[slot][sv], &rinv_s[slot][sv]);
  };
  // rotation of the unit staged in xs[buf], with hook(c) after K-step c
  auto rotate = [&](int buf, qfloatx16& acc, auto&& hook) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const qhalf8 xh = *reinterpret_cast<const qhalf8*>(&xs[buf][0][atok][16 * c + 8 * h]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, bph[c], acc, 0, 0, 0);
      if constexpr (!HAD) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, bpl[c], acc, 0, 0, 0);
      if constexpr (kSplitX) {
        const qhalf8 xl = *reinterpret_cast<const qhalf8*>(&xs[buf][kXP - 1][atok][16 * c + 8 * h]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl, bph[c], acc, 0, 0, 0);
      }
      hook(c);
    }
  };

  constexpr bool kTwoSets = !kSplitX;   // bf16: loads two units ahead
  RawX<XT> rawA, rawB;
  // ---- prologue: stage units 0 and 1, loads of units 2 and 3 in flight,
  // rotation of unit 0
  auto stage = [&](const RawX<XT>& raw, int slot, int buf) {
    const bool rare = stage_common(raw, slot, buf);
    if (__builtin_amdgcn_ballot_w64(rare) != 0) stage_general(raw, slot, buf);
  };
  load_unit(0, rawA);
  load_unit(1, rawB);
  stage(rawA, 0, 0);
  stage(rawB, 1, 1);
  load_unit(2, rawA);
  if constexpr (kTwoSets) load_unit(3, rawB);
  __syncthreads();
  qfloatx16 accA, accB;
  rotate(0, accA, [](int) {});
  __syncthreads();   // iteration 0 stages unit 2 into the buffer just read

  // iteration i: quantize unit i from accq, rotate unit i+1 into accr
  auto iteration = [&](int i, RawX<XT>& raw, const qfloatx16& accq, qfloatx16& accr) {
    const int pb = i & 1, slot = i & 3;
    bool rare = false;
    auto block = [&](auto wc, const auto& tb, uint32_t& vlo, uint32_t& vhi) {
      constexpr int WB = decltype(wc)::value;
      // fields of tokens 16h .. 16h+15 at bits WB*v of (vhi:vlo), appended
      // top token first: one word for WB <= 2; tokens 0..9 and 10..15 for
      // WB = 3 (the word boundary splits token 10), 0..7 and 8..15 for WB = 4
      constexpr int kLo = WB <= 2 ? 16 : (WB == 3 ? 10 : 8);
      uint32_t wl = 0u, wh = 0u;
      float4 r4;
      auto qtoken = [&](int v) {
        if (v % 4 == 3) r4 = *reinterpret_cast<const float4*>(&rinv_s[slot][16 * h + v - 3]);
        const float rt = v % 4 == 0 ? r4.x : v % 4 == 1 ? r4.y : v % 4 == 2 ? r4.z : r4.w;
        value_append<WB>(accq[v], rt, tb, v >= kLo ? wh : wl);
      };
      rotate(pb ^ 1, accr, [&](int c) {
        qtoken(15 - 2 * c);
        qtoken(14 - 2 * c);
      });
      rare = stage_common(raw, (i + 2) & 3, pb);
      vlo = value_fields<WB, kLo>(wl);
      vhi = 0u;
      if constexpr (WB == 3) {
        wh = value_fields<WB, 16 - kLo>(wh);
        vlo |= wh << 30;
        vhi = wh >> 2;
      } else if constexpr (WB == 4) {
        vhi = value_fields<WB, 16 - kLo>(wh);
      }
    };
    uint32_t vlo, vhi;
    block(Width<BITS>{}, tab, vlo, vhi);
    // stores of unit i: the record words of coordinate j (lane half h holds
    // record bits [16*WB*h, 16*WB*(h+1))) and the tokens' norms
    uint32_t s, b;
    unit_sb(i, s, b);
    const int64_t r0 = static_cast<int64_t>(b) * kUnit;
    const int nv = (T - r0 < kUnit ? static_cast<int>(T - r0) : kUnit) - 16 * h;   // valid tokens of the half
    auto put = [&](auto wc) {
      constexpr int WB = decltype(wc)::value;
      if (nv < 16) {   // padding past T: zero fields
        const int nbits = nv > 0 ? WB * nv : 0;
        vlo &= nbits >= 32 ? 0xFFFFFFFFu : ((1u << nbits) - 1u);
        vhi &= nbits <= 32 ? 0u : ((1u << (nbits - 32)) - 1u);
      }
      uint32_t* dst = codes + (static_cast<int64_t>(s) * (Tp / kUnit) + b) * kValRec + joff;
      if constexpr (WB == 1) {
        const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(vlo), 32, 64));
        if (h == 0) dst[0] = vlo | (other << 16);
      } else if constexpr (WB == 2) {
        dst[h] = vlo;
      } else if constexpr (WB == 3) {
        const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(vlo), 32, 64));
        if (h == 0) {
          dst[0] = vlo;
          dst[1] = vhi | (other << 16);
        } else {
          dst[2] = (vlo >> 16) | (vhi << 16);
        }
      } else {
        dst[2 * h] = vlo;
        dst[2 * h + 1] = vhi;
      }
    };
    put(Width<BITS>{});
    if (tid < kUnit) store_norm(norm, norm_dtype, static_cast<int64_t>(s) * Tp + r0 + tid, n_s[slot][tid]);
    if (__builtin_amdgcn_ballot_w64(rare) != 0) stage_general(raw, (i + 2) & 3, pb);
    if constexpr (kTwoSets) load_unit(i + 4, raw);
    else load_unit(i + 3, raw);
    __syncthreads();
  };

  // two units per loop iteration: the accumulators (and, bf16, the input
  // buffers) trade roles
  int i = 0;
  for (; i + 1 < n_units; i += 2) {
    iteration(i, rawA, accA, accB);
    iteration(i + 1, kTwoSets ? rawB : rawA, accB, accA);
  }
  if (i < n_units) iteration(i, rawA, accA, accB);
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
#define TQ_QL(B, MX)                                                                                \
  hipLaunchKernelGGL((quantize_mfma_kernel<XT, KEY, B, APPEND, HAD, MX>), grid, dim3(kQThreads), 0, stream,  \
                     t.rot, t.sketch, t.centroids, t.bounds, static_cast<const XT*>(x), out.nseq, pos, \
                     pos + n, stream_stride(out), out.codes, out.signs, out.norm, out.rnorm,       \
                     out.norm_dtype, t.centroids_hi, t.bounds_hi)
  if (t.hi_coords != 0) {   // split stream (validated: d/2 leading coordinates, bits 1..3)
    if constexpr (!HAD) {
      switch (t.bits) {
        case 1: TQ_QL(1, true); break;
        case 2: TQ_QL(2, true); break;
        default: TQ_QL(3, true); break;
      }
    }
    return;
  }
  switch (t.bits) {
    case 1: TQ_QL(1, false); break;
    case 2: TQ_QL(2, false); break;
    case 3: TQ_QL(3, false); break;
    default: TQ_QL(4, false); break;
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

template <typename XT, bool HAD>
static void launch_keys_pipe(unsigned grid, hipStream_t stream, const tq_tables& t, const void* x,
                             const tq_packed& out, uint32_t nblk, uint32_t units) {
#define TQ_QK_S(B, MX, SL)                                                                                   \
  hipLaunchKernelGGL((quantize_keys_pipe_kernel<XT, B, HAD, MX, SL>), dim3(grid), dim3(kQThreads), 0, stream, \
                     t.rot, t.sketch, t.centroids, t.bounds, static_cast<const XT*>(x), nblk, units,          \
                     out.T, stream_stride(out), out.codes, out.signs, out.norm, out.rnorm,                   \
                     out.norm_dtype, t.centroids_hi, t.bounds_hi)
  // a sketch exact in float16 (the caller's promise) drops the S lo product
#define TQ_QK(B, MX)                \
  do {                              \
    if (t.sketch_f16)               \
      TQ_QK_S(B, MX, false);        \
    else                            \
      TQ_QK_S(B, MX, true);         \
  } while (0)
  if (t.hi_coords != 0) {   // split stream (validated: d/2 leading coordinates, bits 1..3, dense)
    if constexpr (!HAD) {
      switch (t.bits) {
        case 1: TQ_QK(1, true); break;
        case 2: TQ_QK(2, true); break;
        default: TQ_QK(3, true); break;
      }
    }
    return;
  }
  switch (t.bits) {
    case 1: TQ_QK(1, false); break;
    case 2: TQ_QK(2, false); break;
    case 3: TQ_QK(3, false); break;
    default: TQ_QK(4, false); break;
  }
#undef TQ_QK
#undef TQ_QK_S
}

template <typename XT, bool HAD>
static void launch_values_pipe(unsigned grid, hipStream_t stream, const tq_tables& t, const void* x,
                               const tq_packed& out, uint32_t nblk, uint32_t units) {
#define TQ_QV(B)                                                                                        \
  hipLaunchKernelGGL((quantize_values_pipe_kernel<XT, B, HAD>), dim3(grid), dim3(kQThreads), 0, stream,  \
                     t.rot, t.bounds, static_cast<const XT*>(x), nblk, units, out.T, stream_stride(out), \
                     out.codes, out.norm, out.norm_dtype)
  switch (t.bits) {
    case 1: TQ_QV(1); break;
    case 2: TQ_QV(2); break;
    case 3: TQ_QV(3); break;
    default: TQ_QV(4); break;
  }
#undef TQ_QV
}

hipError_t launch_quantize(const tq_tables& t, const void* x, int x_dtype, const tq_packed& out,
                           int64_t pos, int64_t n, bool append, hipStream_t stream) {
  const int64_t nblk = (pos + n + kUnit - 1) / kUnit - pos / kUnit;
  const int64_t units = out.nseq * nblk;
  if (units == 0) return hipSuccess;
  if (!append && out.role == TQ_KEY && units < (static_cast<int64_t>(1) << 31)) {
    // whole key streams: the software-pipelined kernel (2 workgroups per CU)
    const int64_t cap = 2 * static_cast<int64_t>(device_cus());
    const unsigned grid = static_cast<unsigned>(units < cap ? units : cap);
    const bool had = t.rot_kind == TQ_ROT_HADAMARD;
    const uint32_t nb = static_cast<uint32_t>(nblk), nu = static_cast<uint32_t>(units);
    if (x_dtype == TQ_BF16) {
      if (had) launch_keys_pipe<uint16_t, true>(grid, stream, t, x, out, nb, nu);
      else launch_keys_pipe<uint16_t, false>(grid, stream, t, x, out, nb, nu);
    } else {
      if (had) launch_keys_pipe<float, true>(grid, stream, t, x, out, nb, nu);
      else launch_keys_pipe<float, false>(grid, stream, t, x, out, nb, nu);
    }
    return hipGetLastError();
  }
  if (!append && out.role == TQ_VALUE && t.hi_coords == 0 && units < (static_cast<int64_t>(1) << 31)) {
    // whole value streams of one width: the software-pipelined kernel (3 workgroups per CU)
    const int64_t cap = 3 * static_cast<int64_t>(device_cus());
    const unsigned grid = static_cast<unsigned>(units < cap ? units : cap);
    const bool had = t.rot_kind == TQ_ROT_HADAMARD;
    const uint32_t nb = static_cast<uint32_t>(nblk), nu = static_cast<uint32_t>(units);
    if (x_dtype == TQ_BF16) {
      if (had) launch_values_pipe<uint16_t, true>(grid, stream, t, x, out, nb, nu);
      else launch_values_pipe<uint16_t, false>(grid, stream, t, x, out, nb, nu);
    } else {
      if (had) launch_values_pipe<float, true>(grid, stream, t, x, out, nb, nu);
      else launch_values_pipe<float, false>(grid, stream, t, x, out, nb, nu);
    }
    return hipGetLastError();
  }
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
