// Decode attention straight from the packed codes, on the matrix cores:
// the kernels and their per-width dispatch (decode_kernels.h).  Each
// decode_g<G>.hip instantiates one head-group size G; decode.hip holds the
// split-K combine, the workspace layout and the entry launchers.
//
// Method (a2a-mcp.org page, Stage 2 closing paragraph; "How to implement",
// item 1): the query is rotated once (q' = Pi q, u = S q'), every logit is
//   l_t = ||k_t|| <q', c_K[idx_t]> + sqrt(pi/2)/m ||k_t|| ||r_t|| <u, 2 s_t - 1>,
// a = softmax(scale * l), and the values are summed in the rotated domain,
// acc = sum_t a_t ||v_t|| c_V[idxV_t]; out = Pi^T acc happens once, in the
// combine kernel.  No pass dequantizes the cache to memory.
//
// Mapping onto gfx950 (wave64, v_mfma_f32_16x16x32_f16):
//  * one workgroup = 4 waves = one split of the context of one KV head;
//    wave w owns 32-token blocks w, w+4, ..., streams each whole block
//    (key planes, signs, value records, norms) into its LDS ring by LDS DMA,
//    and keeps its own online-softmax state; the 4 states merge through LDS.
//  * every workgroup lays the G rotated queries of its KV head out as
//    matrix-core B fragments -- fp16 hi in columns [0,G), the fp16 residual
//    in [G,2G) -- and builds its code tables in LDS from the codebooks.
//  * logits, per 16-token tile: A = centroid values of 16 tokens x 4
//    coordinates per K-step as fp16 hi/lo pairs, looked up from an LDS table
//    by the index of a coordinate pair, against the query fragment: fp32-grade
//    dots.  Decode with 2-bit keys uses exact float16 levels instead (one
//    K-slot per coordinate, 8 coordinates per K-step; exact_levels2).  The
//    1-bit correction is the same contraction with A = +-1 (a table of sign
//    nibbles) and B = u.  The hi and lo columns are summed with
//    one DPP row shift.
//  * tile rows are ordered so that after the two tiles of a block, lane group
//    g4 = lane/16 holds the logits of tokens 8*g4 .. 8*g4+7: exactly the
//    K-slice those lanes feed to the value MFMA, so softmax weights never
//    leave registers.
//  * values: A = softmax weight times ||v|| (rows = heads, fp16, at most 2^8
//    thanks to a reference that tracks both the running logit max and the
//    running largest ||v||), B = value centroids of 32 tokens x 16
//    coordinates from a token-pair table.
#pragma once

#include <math.h>

#include "common.h"
#include "launch.h"

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kDD = 128;
constexpr int kDecThreads = 256;
constexpr int kLogMaxSplit = 2048;   // logits: tokens per workgroup
constexpr int kDecMaxSplit = 8192;   // decode: tokens per workgroup (longer splits amortise its set-up)
constexpr float kTau = 8.0f;      // raise the reference max when a block exceeds it by 2^8
// LDS code tables (built by build_tables): key tables at 0, value table at
// kVluOff.  Random lookups by 64 lanes are free of LDS bank conflicts only
// while a table fits in the 64 banks (256 bytes; 128 for 4-byte reads): the
// 2-bit key table is therefore indexed by coordinate pairs (16 entries)
// rather than quads.
constexpr int kSgnOff = 2048, kVluOff = 4096, kTabBytes = kVluOff + 1024;
// Split streams (MX, fractional widths): coordinates 0..63 take one bit more
// than 64..127.  The wide key pair table sits at 0 and the wide value table
// at kVluOff as above; the narrow ones follow the sign table (keys; right
// after the wide table for 3-plane wide words, below) and the wide value
// table.
constexpr int kNarrowKeyOff = kSgnOff + 256, kNarrowVluOff = kVluOff + 1024;
constexpr int kTabBytesMix = kNarrowVluOff + 256;
// With 3-plane wide words (2.5-bit keys) the wide table is 64 entries and
// the narrow one sits right after it, at entry 64: a narrow lane sets bit 6
// of its byte indices (kNarrowIndexBit per byte) and reads from the common
// base, so no lookup adds a per-lane table address.
template <int KBW>
constexpr int narrow_key_off() { return KBW == 3 ? 64 * 8 : kNarrowKeyOff; }
constexpr uint32_t kNarrowIndexBit = 0x40404040u;
template <bool MX>
constexpr int tab_bytes() { return MX ? kTabBytesMix : kTabBytes; }


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
//    the hi and once against the lo half of its centroid.  With exact
//    float16 levels (X2, 2-bit keys in decode) only bq[0..3] are used, slot
//    i of K-step c' holding coordinate 32*g4 + 8c' + i once.
//  bu[0..3]: sign K-steps c = 0..3, coordinates 32*g4 + 8c + i.
// Columns n < G carry the fp16 value, G <= n < 2G its fp16 residual, the
// rest zero.


// (x >> 8K) & 0xF0: the high nibble of byte K of x, as a 16-byte-stride
// table offset, in one instruction (a byte-select operand for K > 0)
template <int K>
__device__ __forceinline__ uint32_t high_nibble16(uint32_t x) {
  if constexpr (K == 0) {
    return x & 0xF0u;
  } else {
    uint32_t r = 0;
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (K == 1)
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
          : "=v"(r) : "v"(x), "s"(0xF0u));
    else if constexpr (K == 2)
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
          : "=v"(r) : "v"(x), "s"(0xF0u));
    else
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
          : "=v"(r) : "v"(x), "s"(0xF0u));
#endif
    return r;
  }
}

// centroid K-step C of a 2-bit tile (coordinates 4C .. 4C+3 = the pairs
// (4C, 4C+1) and (4C+2, 4C+3)) from the pair table at `tab`
template <int C>
__device__ __forceinline__ floatx4 key2_kstep(uint32_t Q, uint32_t Q2, uint32_t Qs, uint32_t Q2s,
                                              const char* tab, const half8& b, floatx4 acc) {
  const uint32_t oa = high_nibble16<C / 2>((C & 1) ? Q : Qs);
  const uint32_t ob = high_nibble16<C / 2>((C & 1) ? Q2 : Q2s);
  const uint2 x = *reinterpret_cast<const uint2*>(tab + oa);
  const uint2 y = *reinterpret_cast<const uint2*>(tab + ob);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(x.x, x.y, y.x, y.y), b, acc, 0, 0, 0);
}

// (x >> 8K) & 0x78 in one instruction: with x = Q << 3 it is the low nibble
// of byte K of Q times 8, with x = Q >> 1 its high nibble times 8
template <int K>
__device__ __forceinline__ uint32_t byte_x8(uint32_t x) {
  if constexpr (K == 0) {
    return x & 0x78u;
  } else {
    uint32_t r = 0;
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (K == 1)
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
          : "=v"(r) : "v"(x), "s"(0x78u));
    else if constexpr (K == 2)
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
          : "=v"(r) : "v"(x), "s"(0x78u));
    else
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
          : "=v"(r) : "v"(x), "s"(0x78u));
#endif
    return r;
  }
}

// centroid K-step C of a 2-bit tile on exact float16 levels (build_tables
// with X2): coordinates 8C .. 8C+7 are the pairs (8C, 8C+1) = nibble 2C of
// Q, (8C+2, 8C+3) = nibble 2C of Q2, (8C+4, 8C+5) = nibble 2C+1 of Q and
// (8C+6, 8C+7) = nibble 2C+1 of Q2.  Each pair entry is 4 bytes at an
// 8-byte stride: 4-byte reads by 64 lanes stay free of bank conflicts only
// within a 128-byte table.  Ql / Q2l = Q / Q2 << 3, Qh / Q2h = Q / Q2 >> 1.
template <int C>
__device__ __forceinline__ floatx4 key2x_kstep(uint32_t Ql, uint32_t Q2l, uint32_t Qh, uint32_t Q2h,
                                               const char* tab, const half8& b, floatx4 acc) {
  const uint32_t x0 = *reinterpret_cast<const uint32_t*>(tab + byte_x8<C>(Ql));
  const uint32_t x1 = *reinterpret_cast<const uint32_t*>(tab + byte_x8<C>(Q2l));
  const uint32_t x2 = *reinterpret_cast<const uint32_t*>(tab + byte_x8<C>(Qh));
  const uint32_t x3 = *reinterpret_cast<const uint32_t*>(tab + byte_x8<C>(Q2h));
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(x0, x1, x2, x3), b, acc, 0, 0, 0);
}

// byte K of x times 8, in one instruction (a byte-select operand shifted)
template <int K>
__device__ __forceinline__ uint32_t byte_shl3(uint32_t x) {
  uint32_t r = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (K == 0)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "s"(3u), "v"(x));
  else if constexpr (K == 1)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "s"(3u), "v"(x));
  else if constexpr (K == 2)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "s"(3u), "v"(x));
  else
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "s"(3u), "v"(x));
#else
  r = ((x >> (8 * K)) & 0xFFu) << 3;
#endif
  return r;
}

// centroid K-step C of a 3- or 4-bit tile from the pair table (entry x:
// uint2 at 8x): byte C/2 of E / O is the pair index of coordinates
// (4C, 4C+1) / (4C+2, 4C+3) -- E and O are the words of the low nibbles for
// even C, of the high nibbles for odd C (tile_accumulate)
template <int C>
__device__ __forceinline__ floatx4 key3_kstep(uint32_t E, uint32_t O, const char* tab, const half8& b,
                                              floatx4 acc) {
  const uint2 x = *reinterpret_cast<const uint2*>(tab + byte_shl3<C / 2>(E));
  const uint2 y = *reinterpret_cast<const uint2*>(tab + byte_shl3<C / 2>(O));
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(x.x, x.y, y.x, y.y), b, acc, 0, 0, 0);
}

// sign K-step C: byte C of the sign word sw; sws = sw << 4
template <int C>
__device__ __forceinline__ floatx4 sign_kstep(uint32_t sw, uint32_t sws, const char* tab, const half8& b,
                                              floatx4 acc) {
  const uint2 x = *reinterpret_cast<const uint2*>(tab + high_nibble16<C>(sws));
  const uint2 y = *reinterpret_cast<const uint2*>(tab + high_nibble16<C>(sw));
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(x.x, x.y, y.x, y.y), b, acc, 0, 0, 0);
}

// Centroid and sign dots of one 16-token tile (tile 0 or 1 of a 32-token
// block) for this lane's query-head column: lane (g4, n) gets, for rows
// 4*g4 + i, the centroid dot <q', c[idx]> (cen) and the sign dot
// <u, 2s - 1> (qj) of head n (n < G; the other lanes hold partial sums).
// pw: the tile token's KB plane words of coordinate word g4; sw: its sign
// word; tab: the LDS tables of build_tables.
// MX (split streams): pw holds KB planes, the narrow words' top plane zero,
// and ktab is the lane's own pair table (wide or narrow).  Both tables
// index a pair exactly as the 3- and 4-bit table does (entry x at 8x, the
// coordinates' plane-p bits at bits 2p and 2p + 1 of x), so 3 and 4 planes
// take the repacked byte indices below; a narrow lane's zero top plane
// leaves its indices inside the narrow table.
// tile_accumulate adds one group of 4 coordinate words to the two
// accumulators (head dimensions above 128 take two groups), tile_finish
// folds their hi and lo columns into cen and qj.
template <int G, int KB, bool X2, bool MX = false>
__device__ __forceinline__ void tile_accumulate(const uint32_t* pw, uint32_t sw, const half8 (&bq)[8],
                                                const half8 (&bu)[4], const char* tab, floatx4& accC,
                                                floatx4& accS, const char* ktab = nullptr,
                                                uint32_t kbias = 0u) {
  // the key pair table of this lane: 3-plane split keys index both tables
  // from tab (the narrow lanes' kbias sets bit 6 of each byte index)
  const char* kt = (MX && KB != 3) ? ktab : tab;
  if constexpr (MX && KB == 2) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint2 x = *reinterpret_cast<const uint2*>(ktab + (pair_index<KB>(pw, 2 * c) << 3));
      const uint2 y = *reinterpret_cast<const uint2*>(ktab + (pair_index<KB>(pw, 2 * c + 1) << 3));
      accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(x.x, x.y, y.x, y.y), bq[c], accC, 0, 0, 0);
    }
  } else if constexpr (X2) {
    static_assert(KB == 2, "exact float16 levels exist for 2-bit keys only");
    // same pair-index words as below; one float16 level per coordinate
    const uint32_t Q = ((pw[1] << 2) & 0xCCCCCCCCu) | (pw[0] & 0x33333333u);
    const uint32_t Q2 = (pw[1] & 0xCCCCCCCCu) | ((pw[0] >> 2) & 0x33333333u);
    const uint32_t Ql = Q << 3, Q2l = Q2 << 3, Qh = Q >> 1, Q2h = Q2 >> 1;
    accC = key2x_kstep<0>(Ql, Q2l, Qh, Q2h, tab, bq[0], accC);
    accC = key2x_kstep<1>(Ql, Q2l, Qh, Q2h, tab, bq[1], accC);
    accC = key2x_kstep<2>(Ql, Q2l, Qh, Q2h, tab, bq[2], accC);
    accC = key2x_kstep<3>(Ql, Q2l, Qh, Q2h, tab, bq[3], accC);
  } else if constexpr (KB == 2) {
    // nibble j of Q / Q2: the pair-table index of coordinates (4j, 4j+1) /
    // (4j+2, 4j+3): bits 0, 1 = plane 0 of the two, bits 2, 3 = plane 1.
    // Qs / Q2s hold the same shifted up by 4, so that every nibble is the
    // high nibble of some byte: x16 table offsets with one masked byte read.
    const uint32_t Q = ((pw[1] << 2) & 0xCCCCCCCCu) | (pw[0] & 0x33333333u);
    const uint32_t Q2 = (pw[1] & 0xCCCCCCCCu) | ((pw[0] >> 2) & 0x33333333u);
    const uint32_t Qs = Q << 4, Q2s = Q2 << 4;
    accC = key2_kstep<0>(Q, Q2, Qs, Q2s, tab, bq[0], accC);
    accC = key2_kstep<1>(Q, Q2, Qs, Q2s, tab, bq[1], accC);
    accC = key2_kstep<2>(Q, Q2, Qs, Q2s, tab, bq[2], accC);
    accC = key2_kstep<3>(Q, Q2, Qs, Q2s, tab, bq[3], accC);
    accC = key2_kstep<4>(Q, Q2, Qs, Q2s, tab, bq[4], accC);
    accC = key2_kstep<5>(Q, Q2, Qs, Q2s, tab, bq[5], accC);
    accC = key2_kstep<6>(Q, Q2, Qs, Q2s, tab, bq[6], accC);
    accC = key2_kstep<7>(Q, Q2, Qs, Q2s, tab, bq[7], accC);
  } else if constexpr (KB == 4) {
    // pair indices (8 bits: 2 per plane) one per byte: the nibbles of planes
    // 0-1 (A, B) below those of planes 2-3 (C, D), as for 3-bit keys below
    const uint32_t A = ((pw[1] << 2) & 0xCCCCCCCCu) | (pw[0] & 0x33333333u);
    const uint32_t B = (pw[1] & 0xCCCCCCCCu) | ((pw[0] >> 2) & 0x33333333u);
    const uint32_t C = ((pw[3] << 2) & 0xCCCCCCCCu) | (pw[2] & 0x33333333u);
    const uint32_t D = (pw[3] & 0xCCCCCCCCu) | ((pw[2] >> 2) & 0x33333333u);
    const uint32_t E0 = (A & 0x0F0F0F0Fu) | ((C << 4) & 0xF0F0F0F0u);
    const uint32_t E1 = ((A >> 4) & 0x0F0F0F0Fu) | (C & 0xF0F0F0F0u);
    const uint32_t O0 = (B & 0x0F0F0F0Fu) | ((D << 4) & 0xF0F0F0F0u);
    const uint32_t O1 = ((B >> 4) & 0x0F0F0F0Fu) | (D & 0xF0F0F0F0u);
    accC = key3_kstep<0>(E0, O0, kt, bq[0], accC);
    accC = key3_kstep<1>(E1, O1, kt, bq[1], accC);
    accC = key3_kstep<2>(E0, O0, kt, bq[2], accC);
    accC = key3_kstep<3>(E1, O1, kt, bq[3], accC);
    accC = key3_kstep<4>(E0, O0, kt, bq[4], accC);
    accC = key3_kstep<5>(E1, O1, kt, bq[5], accC);
    accC = key3_kstep<6>(E0, O0, kt, bq[6], accC);
    accC = key3_kstep<7>(E1, O1, kt, bq[7], accC);
  } else if constexpr (KB == 3) {
    // pair indices (6 bits: 2 per plane) repacked one per byte.  Nibble c of
    // A / B holds planes 0 and 1 of the pair (4c, 4c+1) / (4c+2, 4c+3) (as
    // for 2-bit keys); the 4 words below put each pair's plane-2 bits above
    // its nibble, so that byte K of E0 / E1 is the index of pair 4c (c = 2K /
    // 2K+1) and byte K of O0 / O1 that of pair 4c+2.
    const uint32_t A = ((pw[1] << 2) & 0xCCCCCCCCu) | (pw[0] & 0x33333333u);
    const uint32_t B = (pw[1] & 0xCCCCCCCCu) | ((pw[0] >> 2) & 0x33333333u);
    const uint32_t E0 = (A & 0x0F0F0F0Fu) | ((pw[2] << 4) & 0x30303030u) | kbias;
    const uint32_t E1 = ((A >> 4) & 0x0F0F0F0Fu) | (pw[2] & 0x30303030u) | kbias;
    const uint32_t O0 = (B & 0x0F0F0F0Fu) | ((pw[2] << 2) & 0x30303030u) | kbias;
    const uint32_t O1 = ((B >> 4) & 0x0F0F0F0Fu) | ((pw[2] >> 2) & 0x30303030u) | kbias;
    accC = key3_kstep<0>(E0, O0, kt, bq[0], accC);
    accC = key3_kstep<1>(E1, O1, kt, bq[1], accC);
    accC = key3_kstep<2>(E0, O0, kt, bq[2], accC);
    accC = key3_kstep<3>(E1, O1, kt, bq[3], accC);
    accC = key3_kstep<4>(E0, O0, kt, bq[4], accC);
    accC = key3_kstep<5>(E1, O1, kt, bq[5], accC);
    accC = key3_kstep<6>(E0, O0, kt, bq[6], accC);
    accC = key3_kstep<7>(E1, O1, kt, bq[7], accC);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // coordinates 4c .. 4c+3 of word g4: A = (hi, lo) of pair (4c, 4c+1), then of (4c+2, 4c+3)
      const uint2 x = *reinterpret_cast<const uint2*>(tab + (pair_index<KB>(pw, 2 * c) << 3));
      const uint2 y = *reinterpret_cast<const uint2*>(tab + (pair_index<KB>(pw, 2 * c + 1) << 3));
      accC = __builtin_amdgcn_mfma_f32_16x16x32_f16(u4_to_h8(x.x, x.y, y.x, y.y), bq[c], accC, 0, 0, 0);
    }
  }
  // sign K-step c: coordinates 8c .. 8c+7 of word g4 = byte c of the sign
  // word; its low / high nibble selects the +-1 quad of slots 0..3 / 4..7
  accS = sign_kstep<0>(sw, sw << 4, tab + kSgnOff, bu[0], accS);
  accS = sign_kstep<1>(sw, sw << 4, tab + kSgnOff, bu[1], accS);
  accS = sign_kstep<2>(sw, sw << 4, tab + kSgnOff, bu[2], accS);
  accS = sign_kstep<3>(sw, sw << 4, tab + kSgnOff, bu[3], accS);
}

// the hi column n plus the lo column G + n of the two accumulators
template <int G>
__device__ __forceinline__ void tile_finish(const floatx4& accC, const floatx4& accS, float (&cen)[4],
                                            float (&qj)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cen[i] = accC[i] + row_shl<G>(accC[i]);
    qj[i] = accS[i] + row_shl<G>(accS[i]);
  }
}

template <int G, int KB, bool X2, bool MX = false>
__device__ __forceinline__ void tile_logits(const uint32_t* pw, uint32_t sw, const half8 (&bq)[8],
                                            const half8 (&bu)[4], const char* tab, float (&cen)[4],
                                            float (&qj)[4], const char* ktab = nullptr, uint32_t kbias = 0u) {
  floatx4 accC = {0.f, 0.f, 0.f, 0.f}, accS = {0.f, 0.f, 0.f, 0.f};
  tile_accumulate<G, KB, X2, MX>(pw, sw, bq, bu, tab, accC, accS, ktab, kbias);
  tile_finish<G>(accC, accS, cen, qj);
}

// This lane's query fragments for KV head s, built from the rotated queries
// (q' = Pi q, u = S q', one row of d floats per query head) times the
// factors fq and fu, in the layout described above.
template <int G, bool X2>
__device__ __forceinline__ void query_frags(const float* __restrict__ qr, const float* __restrict__ u,
                                            int64_t s, int lane, float fq, float fu, half8 (&bq)[8],
                                            half8 (&bu)[4]) {
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
  // X2 (exact float16 levels): 4 centroid K-steps, slot i = coordinate 8c + i
  constexpr int kNC = X2 ? 4 : 8;
#pragma unroll
  for (int c = 0; c < kNC; ++c) {
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = part(fq * qg[32 * g4 + (X2 ? 8 * c + i : 4 * c + kSlot[i])]);
    bq[c] = u4_to_h8(h2u(h[0], h[1]), h2u(h[2], h[3]), h2u(h[4], h[5]), h2u(h[6], h[7]));
  }
#pragma unroll
  for (int c = kNC; c < 8; ++c) bq[c] = u4_to_h8(0u, 0u, 0u, 0u);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = part(fu * ug[32 * g4 + 8 * c + i]);
    bu[c] = u4_to_h8(h2u(h[0], h[1]), h2u(h[2], h[3]), h2u(h[4], h[5]), h2u(h[6], h[7]));
  }
}

// ------------------------------------------------------------ exact 2-bit levels
// A 2-bit Lloyd-Max codebook is -a, -b, b, a (a > b > 0; symmetric about 0,
// as the quantizer also assumes).  Under one common factor both magnitudes
// become exact float16 numbers to about 1e-6 relative: a -> la = Q 2^(E-11)
// (Q in [1024, 2047], a in [2^(E-1), 2^E), so la lies in a's binade) and
// b -> lb = P 2^(e-11) la / Q, with P the 11-bit rounding of r Q (r = b/a,
// r Q in [2^(e-1), 2^e)).  Every workgroup tries all 1024 values of Q (4 per
// thread) and keeps the one with the smallest |P 2^(e-11) - r Q| / (r Q),
// the smallest Q on a tie, so every workgroup picks the same levels.  The
// decode logits then need one float16 K-slot per coordinate instead of a
// hi + lo pair: 4 centroid K-steps per tile instead of 8.  The factor
// fc = a / la rides on the query fragments, which keep their hi + lo split,
// so the one inexact step is lb's ~1e-6 relative error (1.3e-6 at d = 128),
// far inside decode's output tolerance.  The raw-logits kernel keeps the
// hi + lo centroid pairs (fp32-grade) for its absolute tolerance.
struct Levels2 {
  float la, lb, fc;
};

__device__ __forceinline__ void levels2_from_q(double r, float a, int Q, Levels2& L) {
  int e = 0, E = 0;
  (void)frexp(r * Q, &e);
  const double P = rint(ldexp(r * Q, 11 - e));
  (void)frexpf(a, &E);
  L.la = ldexpf(static_cast<float>(Q), E - 11);
  L.lb = static_cast<float>(ldexp(P, e + E - 22));
  L.fc = a / L.la;
}

// all threads of the workgroup call this (it holds a barrier); red: 4
// 8-byte LDS slots
__device__ __forceinline__ Levels2 exact_levels2(const float* __restrict__ ck, int tid,
                                                 unsigned long long* red) {
  const float a = ck[3];
  const double r = static_cast<double>(ck[2]) / static_cast<double>(a);
  unsigned long long best = ~0ull;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int Q = 1024 + 4 * (tid & 255) + i;
    const double x = r * Q;
    int e = 0;
    (void)frexp(x, &e);
    const double P = rint(ldexp(x, 11 - e));
    const float err = static_cast<float>(fabs(ldexp(P, e - 11) - x) / x);
    // err >= 0 (a NaN from a degenerate table sorts last): its bits order it
    const unsigned long long key = (static_cast<unsigned long long>(__float_as_uint(err)) << 32) |
                                   static_cast<unsigned int>(Q);
    best = key < best ? key : best;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned int lo = __shfl_xor(static_cast<unsigned int>(best), o, 64);
    const unsigned int hi = __shfl_xor(static_cast<unsigned int>(best >> 32), o, 64);
    const unsigned long long other = (static_cast<unsigned long long>(hi) << 32) | lo;
    best = other < best ? other : best;
  }
  if ((tid & 63) == 0) red[tid >> 6] = best;
  __syncthreads();
  unsigned long long m = red[0];
#pragma unroll
  for (int w = 1; w < kDecThreads / 64; ++w) m = red[w] < m ? red[w] : m;
  Levels2 L;
  levels2_from_q(r, a, static_cast<int>(m & 0xFFFFu), L);
  return L;
}

// The workgroup's code tables in LDS (kTabBytes at the start of its LDS),
// built from the codebooks:
//  * 2-bit keys: entry x of the pair table (uint2 at 16x) holds the
//    centroids of 2 consecutive coordinates whose plane-0 bits are x & 3 and
//    plane-1 bits x >> 2, as {hi(c0,c1), lo(c0,c1)} -- half of a centroid
//    K-step's slots;
//  * other widths: entry x of the pair table (uint2 at 8x) holds
//    {hi(c0,c1), lo(c0,c1)} of the coordinate pair whose 2*KB-bit index is x
//    (bit 2p: plane p of the lower coordinate, bit 2p+1: plane p of the upper);
//  * at kSgnOff, entry x (uint2 at 16x) holds the +-1 values of 4 sign bits
//    x (bit i -> slot i) as fp16;
//  * at kVluOff (VB > 0), vlut[x]: the value centroids of the token pair
//    whose fields are x & (2^VB - 1) and x >> VB.
//  * X2 (2-bit keys on exact float16 levels): entry x (4 bytes at 8x) holds
//    the levels of the coordinate pair whose plane-0 bits are x & 3 and
//    plane-1 bits x >> 2, from {-la, -lb, lb, la} (exact_levels2).
// generic pair table of a kb-bit codebook (entry x: uint2 at 8x, as below)
__device__ __forceinline__ void build_pair_table(const float* __restrict__ ck, int kb, char* tab, int tid,
                                                 int nthreads) {
  uint2* pair = reinterpret_cast<uint2*>(tab);
  for (int x = tid; x < (1 << (2 * kb)); x += nthreads) {
    int ia = 0, ib = 0;
    for (int p = 0; p < kb; ++p) {
      ia |= ((x >> (2 * p)) & 1) << p;
      ib |= ((x >> (2 * p + 1)) & 1) << p;
    }
    const float ca = ck[ia], cb = ck[ib];
    const _Float16 ha = static_cast<_Float16>(ca), hb = static_cast<_Float16>(cb);
    const _Float16 la = static_cast<_Float16>(ca - static_cast<float>(ha));
    const _Float16 lb = static_cast<_Float16>(cb - static_cast<float>(hb));
    pair[x] = make_uint2(h2u(ha, hb), h2u(la, lb));
  }
}

// value pair table of a vb-bit codebook (entry x: the centroids of the token
// pair whose fields are x & (2^vb - 1) and x >> vb)
__device__ __forceinline__ void build_value_table(const float* __restrict__ cv, int vb, char* tab, int tid,
                                                  int nthreads) {
  uint32_t* vlut = reinterpret_cast<uint32_t*>(tab);
  for (int x = tid; x < (1 << (2 * vb)); x += nthreads)
    vlut[x] = h2u(static_cast<_Float16>(cv[x & ((1 << vb) - 1)]), static_cast<_Float16>(cv[x >> vb]));
}

// Tables of split streams: key pair tables (KB + 1 bits at 0, KB bits at
// narrow_key_off<KB + 1>(); the lanes of words 0 and 1 index the first, of words 2 and
// 3 the second, with a zero top plane), the sign table, and value tables
// (VB + 1 bits at kVluOff, VB bits at kNarrowVluOff).
template <int KB, int VB>
__device__ __forceinline__ void build_tables_mix(const float* __restrict__ ck, const float* __restrict__ ck_hi,
                                                 const float* __restrict__ cv, const float* __restrict__ cv_hi,
                                                 char* tab, int tid, int nthreads) {
  build_pair_table(ck_hi, KB + 1, tab, tid, nthreads);
  build_pair_table(ck, KB, tab + narrow_key_off<KB + 1>(), tid, nthreads);
  for (int x = tid; x < 16; x += nthreads) {
    auto pm = [&](int i) { return static_cast<_Float16>(((x >> i) & 1) ? 1.f : -1.f); };
    *reinterpret_cast<uint2*>(tab + kSgnOff + 16 * x) = make_uint2(h2u(pm(0), pm(1)), h2u(pm(2), pm(3)));
  }
  if constexpr (VB > 0) {
    build_value_table(cv_hi, VB + 1, tab + kVluOff, tid, nthreads);
    build_value_table(cv, VB, tab + kNarrowVluOff, tid, nthreads);
  }
}

template <int KB, int VB, bool X2>
__device__ __forceinline__ void build_tables(const float* __restrict__ ck, const float* __restrict__ cv,
                                             char* tab, int tid, int nthreads, float la = 0.f,
                                             float lb = 0.f) {
  auto hilo = [&](float c, _Float16& h, _Float16& l) {
    h = static_cast<_Float16>(c);
    l = static_cast<_Float16>(c - static_cast<float>(h));
  };
  if constexpr (X2) {
    static_assert(KB == 2, "exact float16 levels exist for 2-bit keys only");
    for (int x = tid; x < 16; x += nthreads) {
      auto level = [&](int idx) {   // idx 0..3 = -a, -b, b, a
        const float v = (idx == 0 || idx == 3) ? la : lb;
        return static_cast<_Float16>(idx < 2 ? -v : v);
      };
      const int i0 = (x & 1) | (((x >> 2) & 1) << 1), i1 = ((x >> 1) & 1) | (((x >> 3) & 1) << 1);
      *reinterpret_cast<uint32_t*>(tab + 8 * x) = h2u(level(i0), level(i1));
    }
  } else if constexpr (KB == 2) {
    for (int x = tid; x < 16; x += nthreads) {
      _Float16 h[2], l[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) hilo(ck[((x >> i) & 1) | (((x >> (2 + i)) & 1) << 1)], h[i], l[i]);
      *reinterpret_cast<uint2*>(tab + 16 * x) = make_uint2(h2u(h[0], h[1]), h2u(l[0], l[1]));
    }
  } else {
    uint2* pair = reinterpret_cast<uint2*>(tab);
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
      pair[x] = make_uint2(h2u(ha, hb), h2u(la, lb));
    }
  }
  for (int x = tid; x < 16; x += nthreads) {
    auto pm = [&](int i) { return static_cast<_Float16>(((x >> i) & 1) ? 1.f : -1.f); };
    *reinterpret_cast<uint2*>(tab + kSgnOff + 16 * x) = make_uint2(h2u(pm(0), pm(1)), h2u(pm(2), pm(3)));
  }
  if constexpr (VB > 0) {
    uint32_t* vlut = reinterpret_cast<uint32_t*>(tab + kVluOff);
    for (int x = tid; x < (1 << (2 * VB)); x += nthreads)
      vlut[x] = h2u(static_cast<_Float16>(cv[x & ((1 << VB) - 1)]), static_cast<_Float16>(cv[x >> VB]));
  }
}

// ------------------------------------------------------------ the kernel
// Every 32-token block a wave works on is streamed whole into the wave's
// part of an LDS ring by LDS DMA (global_load_lds_dwordx4: 16 bytes per lane
// straight into LDS, no registers), kRing blocks deep: while the wave
// computes block j, blocks j+1 and j+2 are in flight.  A block's packet is
// the concatenation of its key plane words, sign words, value records and
// the three norm rows -- all contiguous, 16-byte aligned runs in the packed
// streams, since every stream holds whole 32-token blocks.
constexpr int kRing = 3;
static_assert(kRing == 2 || kRing == 3, "the waits below cover rings of 2 or 3 blocks");

// NK / NV: bytes per stored key / value norm (2: float16, 4: float32).  MX:
// split streams, whose key records hold 4 KB + 2 words per token (words 0
// and 1 at KB + 1 planes) and value records 128 VB + 64 words per block.
template <int KB, int VB, int NK, int NV, bool MX = false>
struct Packet {
  static constexpr int kKeyRec = MX ? 4 * KB + 2 : 4 * KB;          // words per token
  static constexpr int kValRec = VB == 0 ? 0 : (MX ? 128 * VB + 64 : 128 * VB);  // words per block
  static constexpr int kKC = 0;                // key plane words [32 tokens][kKeyRec]
  static constexpr int kSG = 128 * kKeyRec;    // sign words [32][4]
  static constexpr int kVC = kSG + 512;        // value records [kValRec]
  static constexpr int kNK = kVC + 4 * kValRec;   // ||k|| [32]
  static constexpr int kNR = kNK + 32 * NK;    // ||k|| ||r|| [32]
  static constexpr int kNV = kNR + 32 * NK;    // ||v|| [32]
  static constexpr int kBytes = kNV + 32 * NV;
  static constexpr int kChunks = kBytes / 16;
  static constexpr int kInstr = (kChunks + 63) / 64;   // DMA instructions per block
  static constexpr int kTail = kChunks - 64 * (kInstr - 1);  // lanes of the last one
};
static_assert(Packet<3, 4, 4, 2>::kBytes == 512 * 3 + 512 + 512 * 4 + 64 * 4 + 32 * 2, "packet layout");

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// 16 bytes from global `src` (this lane's) to LDS at lds + 16 * lane; `lds`
// is wave-uniform.  Issued as inline assembly so that the compiler does not
// treat the ring as written by a load it tracks (it would then wait for every
// DMA in flight before any LDS read); the waits are explicit instead.  M0
// (the LDS base of the DMA) is written here and read by nothing else in these
// kernels: they use no other M0-based instruction (the compiler's note that
// M0 is a reserved register is silenced for this one statement).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
#pragma clang diagnostic pop
#endif
}

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory");
#endif
}

// Token order of the key-plane and sign chunks in the ring.  Tile row n of
// tile `tile` is token t = 8 (n/4) + 4 tile + n%4; its chunks sit at slot
// ring_slot(t) = 16 tile + n, so the 16 tokens one tile reads fill 16
// consecutive 16-byte slots.  In stream order (token t at slot t) the 16
// rows would share 4 slots modulo 16 and every read of key-plane or sign
// words would be a 4-way LDS bank conflict (measured ~3x the conflict-free
// time); in this order 8-byte key-plane reads are conflict-free and 4-byte
// sign-word reads 2-way.  The DMA lanes fetch their chunks in this order.
__device__ __forceinline__ int ring_token(int slot) {   // inverse of ring_slot
  return 8 * ((slot & 15) >> 2) + 4 * (slot >> 4) + (slot & 3);
}

// Key-plane words (KB per coordinate word g4) and the sign word of the token
// at ring slot 16 tile + n of a packet.  A token's 4 KB plane words are its
// KB chunks, chunk h at slot 32 h + slot: the 16 rows of a tile read 16
// consecutive chunks.  With 3 planes a lane's 3 words would straddle two
// such chunks, so there a token's 3 chunks are adjacent (slot 3 slot + h)
// and the 3 words contiguous: two reads, 2-way conflicts.
//
// key_lane_off: byte offset of lane (n, g4)'s words of tile 0 from the
// packet's key segment; tile 1 lies key_tile_bytes further, word q 4q.
// Sign words: P::kSG + 16 n + 4 g4, tile 1 256 bytes further.
template <int KB>
__device__ __forceinline__ uint32_t key_lane_off(int n, int g4) {
  if constexpr (KB == 2) return 512 * (g4 >> 1) + 16 * n + 8 * (g4 & 1);
  else if constexpr (KB == 3) return 48 * n + 12 * g4;
  else if constexpr (KB == 4) return 512 * g4 + 16 * n;
  else return 16 * n + 4 * g4;
}
template <int KB>
constexpr int key_tile_bytes() { return KB == 3 ? 768 : 256; }

// kb, sb: this lane's key words and sign word of tile 0 (lds_at)
template <int KB>
__device__ __forceinline__ void ring_key_words(const char* kb, const char* sb, int tile, uint32_t (&kw)[KB],
                                               uint32_t& sw) {
  const char* k = kb + key_tile_bytes<KB>() * tile;
  if constexpr (KB == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(k);
    kw[0] = v.x;
    kw[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < KB; ++q) kw[q] = reinterpret_cast<const uint32_t*>(k)[q];
  }
  sw = *reinterpret_cast<const uint32_t*>(sb + 256 * tile);
}

// base + off, with off pinned in one VGPR: the compiler would otherwise add
// the per-block ring offset to every read's own lane offset separately; from
// one pinned address per lane pattern the reads at constant distances carry
// those distances as instruction immediates.
__device__ __forceinline__ const char* lds_at(const char* base, uint32_t off) {
  asm("" : "+v"(off));
  return base + off;
}

// The LDS-DMA ring of one wave: the sources of this lane's 16-byte chunks of
// the wave's first block, their advance per block of the wave (4 blocks of
// the split), the ring slot addresses, and the waits.  P is the Packet.
template <typename P>
struct BlockStream {
  const char* src[P::kInstr];
  int64_t step[P::kInstr];
  uint32_t ring0;   // LDS address of this wave's packet in slot 0
  int kslot;        // bytes per ring slot (the 4 waves' packets)

  // tok / tokv: index of the wave's first token in the key / value stream
  // (sequence * its stride + token); value segment and value norms are empty
  // when P has VB = 0 / NV = 0
  template <int KB, int VB, int NK, int NV, bool MX = false>
  __device__ __forceinline__ void init(const uint32_t* kcodes, const uint32_t* ksigns, const void* knorm,
                                       const void* krnorm, const uint32_t* vcodes, const void* vnorm,
                                       int64_t tok, int64_t tokv, int lane, uint32_t ring_wave0,
                                       int slot_bytes) {
    ring0 = ring_wave0;
    kslot = slot_bytes;
    constexpr int kKeyChunks = 8 * P::kKeyRec;         // 32 tokens x kKeyRec words / 16 B
    constexpr int kValChunks = P::kValRec / 4;
#pragma unroll
    for (int i = 0; i < P::kInstr; ++i) {
      const int c = 64 * i + lane;
      const char* p = reinterpret_cast<const char*>(kcodes);
      int64_t st = 0;
      if (MX && c < kKeyChunks) {
        // split keys: the block's records in token order
        p = reinterpret_cast<const char*>(kcodes) + tok * 4 * P::kKeyRec + 16 * c;
        st = 4 * 32 * 4 * P::kKeyRec;
      } else if (MX && c < kKeyChunks + 32) {
        p = reinterpret_cast<const char*>(ksigns) + tok * 16 + 16 * ring_token(c - kKeyChunks);
        st = 4 * 32 * 16;
      } else if (MX && c < kKeyChunks + 32 + kValChunks) {
        p = reinterpret_cast<const char*>(vcodes) + (tokv / 32) * 4 * P::kValRec + 16 * (c - kKeyChunks - 32);
        st = 4 * 4 * P::kValRec;
      } else if (MX && c < kKeyChunks + 32 + kValChunks + 4 * NK) {
        const int e = c - kKeyChunks - 32 - kValChunks;
        const int row = e / (2 * NK);
        p = reinterpret_cast<const char*>(row == 0 ? knorm : krnorm) + tok * NK + 16 * (e - 2 * NK * row);
        st = 4 * 32 * NK;
      } else if (MX && c < P::kChunks) {
        const int e = c - kKeyChunks - 32 - kValChunks - 4 * NK;
        p = reinterpret_cast<const char*>(vnorm) + tokv * NV + 16 * e;
        st = 4 * 32 * NV;
      } else if (MX) {
        // past the packet: nothing is fetched (lanes of the last instruction only)
      } else if (c < 32 * KB) {
        // ring slot c holds chunk h of token t: c = 32 h + ring_slot(t), or
        // c = 3 ring_slot(t) + h for 3-plane keys (ring_key_words)
        const int t = ring_token(KB == 3 ? c / 3 : c & 31);
        const int hh = KB == 3 ? c % 3 : c >> 5;
        p = reinterpret_cast<const char*>(kcodes) + tok * 16 * KB + 16 * (t * KB + hh);
        st = 4 * 32 * 16 * KB;
      } else if (c < 32 * KB + 32) {
        p = reinterpret_cast<const char*>(ksigns) + tok * 16 + 16 * ring_token(c - 32 * KB);
        st = 4 * 32 * 16;
      } else if (c < 32 * (KB + 1 + VB)) {
        p = reinterpret_cast<const char*>(vcodes) + (tokv / 32) * 512 * VB + 16 * (c - 32 * (KB + 1));
        st = 4 * 512 * VB;
      } else if (c < 32 * (KB + 1 + VB) + 4 * NK) {
        const int e = c - 32 * (KB + 1 + VB);        // 2 NK chunks per key norm row
        const int row = e / (2 * NK);
        p = reinterpret_cast<const char*>(row == 0 ? knorm : krnorm) + tok * NK + 16 * (e - 2 * NK * row);
        st = 4 * 32 * NK;
      } else if (c < P::kChunks) {
        const int e = c - 32 * (KB + 1 + VB) - 4 * NK;
        p = reinterpret_cast<const char*>(vnorm) + tokv * NV + 16 * e;
        st = 4 * 32 * NV;
      }
      src[i] = p;
      step[i] = st;
    }
  }

  // DMA of the wave's block j into ring slot `slot`
  __device__ __forceinline__ void issue(int j, int slot, int lane) const {
    const uint32_t l = ring0 + slot * kslot;
#pragma unroll
    for (int i = 0; i < P::kInstr; ++i) {
      const char* a = src[i] + j * step[i];
      if (i + 1 < P::kInstr || lane < P::kTail) dma16(a, l + 1024 * i);
    }
  }

  // before block j of nbw: issue block j + kRing - 1 into the slot block j-1
  // used (read in the previous iteration), then wait until block j has
  // landed -- blocks j+1 .. j+kRing-1 stay in flight
  __device__ __forceinline__ void advance(int j, int nbw, int slot, int lane) const {
    if (j + kRing - 1 < nbw) {
      issue(j + kRing - 1, slot == 0 ? kRing - 1 : slot - 1, lane);
      wait_vm<(kRing - 1) * P::kInstr>();
    } else if (kRing > 2 && j + 2 < nbw) {
      wait_vm<(kRing > 2 ? 2 : 0) * P::kInstr>();
    } else if (j + 1 < nbw) {
      wait_vm<P::kInstr>();
    } else {
      wait_vm<0>();
    }
  }
};

template <int NB>
__device__ __forceinline__ float norm_at(const char* p, int i) {
  if constexpr (NB == 2) return static_cast<float>(reinterpret_cast<const _Float16*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

// workgroups per CU that the LDS of a workgroup (tables + ring of packets of
// `bytes`) allows, at most 3; the host sizes decode splits by it
constexpr int ring_occupancy_bytes(int bytes, bool mx = false) {
  return ((mx ? kTabBytesMix : kTabBytes) + kRing * 4 * bytes) * 3 <= 160 * 1024 ? 3 : 2;
}

// bytes of one block's packet (Packet<KB, VB, NK, NV, MX>::kBytes)
constexpr int packet_bytes(int kb, int vb, int nk, int nv, bool mx = false) {
  return 512 * kb + 512 + 512 * vb + 64 * nk + 32 * nv + (mx ? 256 + (vb > 0 ? 256 : 0) : 0);
}

template <typename P, bool MX = false>
constexpr int ring_occupancy() {
  return ring_occupancy_bytes(P::kBytes, MX);
}
static_assert(packet_bytes(3, 3, 2, 2, true) == Packet<3, 3, 2, 2, true>::kBytes, "split packet size");
static_assert(packet_bytes(2, 3, 2, 2) == Packet<2, 3, 2, 2>::kBytes, "packet size");

// The key-table base and key-word offset of lane (n, g4) in a split stream:
// words 0 and 1 (lane groups 0, 1) use the wide table, 2 and 3 the narrow
// one; the lane's token row t = 8 (n/4) + n%4 of tile 0 (tile 1: 4 tokens
// on), its word's planes after those of the words before it.
template <int KB>
__device__ __forceinline__ uint32_t mix_key_lane_off(int n, int g4) {
  constexpr int rec = 4 * KB + 2;
  const int t = 8 * (n >> 2) + (n & 3);
  return 4 * (t * rec + g4 * KB + (g4 < 2 ? g4 : 2));
}

template <int G, int KB, int VB, int NK, int NV, bool MX = false>
__global__ __launch_bounds__(kDecThreads, (ring_occupancy<Packet<KB, VB, NK, NV, MX>, MX>())) void decode_mfma_kernel(
    const float* __restrict__ qr, const float* __restrict__ u, const float* __restrict__ ck,
    const float* __restrict__ cv, int64_t T, int64_t TpK, int64_t TpV, int split_len,
    const uint32_t* __restrict__ kcodes, const uint32_t* __restrict__ ksigns, const void* knorm,
    const void* krnorm, const uint32_t* __restrict__ vcodes, const void* vnorm, float fq, float fu,
    int nsplit, float* __restrict__ partials, const float* __restrict__ ck_hi = nullptr,
    const float* __restrict__ cv_hi = nullptr) {
  using P = Packet<KB, VB, NK, NV, MX>;
  constexpr int VL = 1 << (2 * VB);
  constexpr int kSlot = 4 * P::kBytes;   // one ring slot: the 4 waves' packets
  // code tables (build_tables); the ring; after the main loop the ring holds
  // the four waves' softmax states for the merge
  __shared__ __align__(16) char lds[tab_bytes<MX>()];
  constexpr int kMerge = (2 * 4 * 16 + 4 * G * kDD) * 4;
  __shared__ __align__(16) char ring[kRing * kSlot > kMerge ? kRing * kSlot : kMerge];
  const uint32_t* vlut = reinterpret_cast<const uint32_t*>(lds + kVluOff);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int64_t h0 = s * G;
  const int t0 = split * split_len;                  // T < 2^28 (checked on the host)
  const int Ti = static_cast<int>(T);
  const int t1 = (t0 + split_len < Ti) ? t0 + split_len : Ti;
  const int nb_split = (t1 - t0 + 31) / 32;
  // this wave takes the split's blocks wave, wave + 4, ...
  const int nbw = (nb_split > wave) ? (nb_split - wave + 3) / 4 : 0;

  BlockStream<P> st;
  st.template init<KB, VB, NK, NV, MX>(kcodes, ksigns, knorm, krnorm, vcodes, vnorm, s * TpK + t0 + 32 * wave,
                                       s * TpV + t0 + 32 * wave, lane, lds_addr(ring) + wave * P::kBytes, kSlot);
#pragma unroll
  for (int jj = 0; jj + 1 < kRing; ++jj)
    if (jj < nbw) st.issue(jj, jj, lane);

  // 2-bit keys: exact float16 levels, one K-slot per coordinate
  constexpr bool X2 = KB == 2 && !MX;
  __shared__ unsigned long long red2[X2 ? kDecThreads / 64 : 1];
  Levels2 lev{0.f, 0.f, 1.f};
  if constexpr (X2) lev = exact_levels2(ck, tid, red2);
  // visible after the barrier below
  if constexpr (MX) build_tables_mix<KB, VB>(ck, ck_hi, cv, cv_hi, lds, tid, kDecThreads);
  else build_tables<KB, VB, X2>(ck, cv, lds, tid, kDecThreads, lev.la, lev.lb);
  half8 bq[8], bu[4];
  query_frags<G, X2>(qr, u, s, lane, fq * lev.fc, fu, bq, bu);
  __syncthreads();

  floatx4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Online softmax in base 2, per head column n (every lane group of a
  // column holds the same state).  Logits arrive as sv = l - r with the
  // reference r = m + log2(sigma): m a lazily raised running max, sigma the
  // running max of ||v||.  Then p'' = 2^sv = p / sigma and the value weight
  // p'' ||v|| = p ||v|| / sigma stays <= 2^kTau, inside float16 range.
  // lsum and O are both kept in units of 2^-r, so out = O / lsum.
  float r_ref = 0.f, m_ref = -INFINITY, lsum = 0.f;
  float sig = 0.f, lthr = 0.f;                         // sigma; kTau - log2(sigma)
  bool first = true;
  const int vbit0 = 8 * VB * g4;                       // this lane group's 8 value fields
  // the fields lie in record words vwlo and vwlo + 1 (the word after a
  // record is the next record's first, or the first norm row: read, unused)
  const int vwlo = vbit0 >> 5, vsh = vbit0 & 31;
  // this lane's byte offsets within a packet: key words, sign word, its 8
  // tokens' norms (key and value), value record words
  const uint32_t koff = P::kKC + (MX ? mix_key_lane_off<KB>(n, g4) : key_lane_off<KB>(n, g4));
  const uint32_t soff = P::kSG + 16 * n + 4 * g4;
  const uint32_t nkoff = 8 * NK * g4, nvoff = 8 * NV * g4;
  const uint32_t voff = P::kVC + 4 * (n * VB + vwlo);
  // split streams: lane's key table, and the value record words / shifts of
  // the wide coordinates (0..63, VB + 1 bits) and the narrow ones (VB bits)
  const char* ktab = lds + ((MX && g4 >= 2) ? narrow_key_off<KB + 1>() : 0);
  const uint32_t kbias = (MX && KB + 1 == 3 && g4 >= 2) ? kNarrowIndexBit : 0u;   // 2.5-bit keys
  constexpr int VW = MX ? VB + 1 : VB;
  const int vbitW = 8 * VW * g4;
  const uint32_t voffW = P::kVC + 4 * (n * VW + (vbitW >> 5));
  const uint32_t voffN = P::kVC + 4 * (64 * VW + n * VB + vwlo);
  const int vshW = vbitW & 31;

  int slot = 0;
  for (int j = 0; j < nbw; ++j) {
    st.advance(j, nbw, slot, lane);
    const uint32_t pko = slot * kSlot + wave * P::kBytes;   // the block's packet in the ring
    slot = (slot == kRing - 1) ? 0 : slot + 1;
    const char* kb = lds_at(ring, pko + koff);
    const char* sb = lds_at(ring, pko + soff);
    const char* nkb = lds_at(ring, pko + nkoff);
    const int tb = t0 + 32 * (wave + 4 * j);           // first token of the block
    const bool full = tb + 32 <= Ti;

    // ---------------- logits of the block's 32 tokens
    float sv[8];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      float cen[4], qj[4];
      if constexpr (MX) {
        // split keys: KB + 1 plane words read for every word, the narrow
        // words' top one cleared; token rows 4 tokens apart between tiles
        uint32_t kw[KB + 1];
        const uint32_t* kp = reinterpret_cast<const uint32_t*>(kb + 16 * (4 * KB + 2) * tile);
#pragma unroll
        for (int q = 0; q <= KB; ++q) kw[q] = kp[q];
        if (g4 >= 2) kw[KB] = 0u;
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(sb + 256 * tile);
        tile_logits<G, KB + 1, false, true>(kw, sw, bq, bu, lds, cen, qj, ktab, kbias);
      } else {
        uint32_t kw[KB], sw;
        ring_key_words<KB>(kb, sb, tile, kw, sw);
        tile_logits<G, KB, X2>(kw, sw, bq, bu, lds, cen, qj);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float nk = norm_at<NK>(nkb + P::kNK, 4 * tile + i), nr = norm_at<NK>(nkb + P::kNR, 4 * tile + i);
        sv[4 * tile + i] = fmaf(nk, cen[i], fmaf(nr, qj[i], -r_ref));
      }
    }
    // ||v|| of this lane group's 8 tokens, and their largest
    float nv[8];
    uint32_t nvh[4];   // float16 norms: the 4 packed pairs as stored
    const char* nvb = NV == NK ? nkb : lds_at(ring, pko + nvoff);
    if constexpr (NV == 2) {
      const uint4 w = *reinterpret_cast<const uint4*>(nvb + P::kNV);
      nvh[0] = w.x; nvh[1] = w.y; nvh[2] = w.z; nvh[3] = w.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) nv[k] = norm_at<NV>(nvb + P::kNV, k);
    }
    if (!full) {
      // the context's last, partial block: tokens past T get no weight, and
      // whatever their storage holds (padding, an append's leftovers) is
      // never read as a number
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (tb + 8 * g4 + k >= Ti) {
          sv[k] = -INFINITY;
          if constexpr (NV == 2) nvh[k / 2] &= (k & 1) ? 0x0000FFFFu : 0u;
          else nv[k] = 0.f;
        }
      }
    }
    float vm;
    if constexpr (NV == 2) {
      const half2_t m = __builtin_elementwise_max(
          __builtin_elementwise_max(__builtin_bit_cast(half2_t, nvh[0]), __builtin_bit_cast(half2_t, nvh[1])),
          __builtin_elementwise_max(__builtin_bit_cast(half2_t, nvh[2]), __builtin_bit_cast(half2_t, nvh[3])));
      vm = static_cast<float>(m.x > m.y ? m.x : m.y);   // norms are finite and >= 0
    } else {
      vm = fmaxf(fmaxf(fmaxf(nv[0], nv[1]), fmaxf(nv[2], nv[3])),
                 fmaxf(fmaxf(nv[4], nv[5]), fmaxf(nv[6], nv[7])));
    }
    // ---------------- raise the reference when a logit passes m + kTau or a
    // value norm passes sigma (rare after the first block)
    float bm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    // (each lane tests its own maxima: a column's threshold is passed by its
    // row maximum exactly when it is passed by one of its lanes)
    if (__builtin_amdgcn_ballot_w64(first || bm > lthr || vm > sig) != 0) {
      bm = max_over_rows(bm);
      sig = fmaxf(sig, max_over_rows(vm));
      const float ls = __builtin_amdgcn_logf(fmaxf(sig, 0x1p-90f));   // log2
      const float m_new = fmaxf(m_ref, bm + r_ref);
      const float r_new = m_new + ls;
      const float delta = r_ref - r_new;
      const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(delta);
      first = false;
      lsum *= alpha;
      m_ref = m_new;
      r_ref = r_new;
      lthr = kTau - ls;
#pragma unroll
      for (int k = 0; k < 8; ++k) sv[k] += delta;
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * g4 + i);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) O[nt][i] *= a4[i];
      }
    }
    // A = p'' ||v|| (float16, <= 2^kTau); B = c_V[idx] for tokens 8*g4 .. 8*g4+7
    half8 pa;
    if constexpr (NV == 2) {
      // p'' ||v|| rounded once to float16 straight from the stored float16
      // norm: one mixed-precision fma per token
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(sv[2 * i]), p1 = __builtin_amdgcn_exp2f(sv[2 * i + 1]);
        lsum += p0 + p1;
        pw[i] = 0;
#if defined(__HIP_DEVICE_COMPILE__)
        asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(pw[i]) : "v"(p0), "v"(nvh[i]));
        asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
            : "+v"(pw[i]) : "v"(p1), "v"(nvh[i]));
#endif
      }
      pa = u4_to_h8(pw[0], pw[1], pw[2], pw[3]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = __builtin_amdgcn_exp2f(sv[k]);
        lsum += p;
        pa[k] = static_cast<_Float16>(p * nv[k]);
      }
    }
    if constexpr (MX) {
      // split values: coordinates 0..63 (nt < 4) at VB + 1 bits, 64..127 at VB
      const uint32_t* vrw = reinterpret_cast<const uint32_t*>(lds_at(ring, pko + voffW));
      const uint32_t* vrn = reinterpret_cast<const uint32_t*>(lds_at(ring, pko + voffN));
      const uint32_t* vlutW = reinterpret_cast<const uint32_t*>(lds + kVluOff);
      const uint32_t* vlutN = reinterpret_cast<const uint32_t*>(lds + kNarrowVluOff);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bool wide_nt = nt < 4;
        const uint32_t* vr = wide_nt ? vrw + 16 * nt * VW : vrn + 16 * (nt - 4) * VB;
        const uint32_t X = __builtin_amdgcn_alignbit(vr[1], vr[0], wide_nt ? vshW : vsh);
        uint32_t bw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          bw[q] = wide_nt ? vlutW[(X >> (2 * VW * q)) & ((1 << (2 * VW)) - 1)] : vlutN[(X >> (2 * VB * q)) & (VL - 1)];
        O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, u4_to_h8(bw[0], bw[1], bw[2], bw[3]), O[nt], 0, 0, 0);
      }
    } else {
    // two base addresses, so that every record word is an immediate offset
    // of a paired 4-byte read (at most 255 words away)
    const uint32_t* vrec0 = reinterpret_cast<const uint32_t*>(lds_at(ring, pko + voff));
    const uint32_t* vrec1 = vrec0 + 64 * VB;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint32_t* vr = (nt < 4 ? vrec0 : vrec1) + 16 * (nt & 3) * VB;
      const uint32_t X = __builtin_amdgcn_alignbit(vr[1], vr[0], vsh);
      uint32_t bw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) bw[q] = vlut[(X >> (2 * VB * q)) & (VL - 1)];
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, u4_to_h8(bw[0], bw[1], bw[2], bw[3]), O[nt], 0, 0, 0);
    }
    }
  }

  // ---------------- merge the 4 waves' states, write this split's partial
  __syncthreads();  // every wave is done with the ring, which holds the merge area
  float (*m_s)[16] = reinterpret_cast<float (*)[16]>(ring);
  float (*l_s)[16] = reinterpret_cast<float (*)[16]>(ring + 4 * 16 * 4);
  float (*o_s)[G][kDD] = reinterpret_cast<float (*)[G][kDD]>(ring + 2 * 4 * 16 * 4);
  float ltot = lsum;
  ltot += __shfl_xor(ltot, 16);
  ltot += __shfl_xor(ltot, 32);
  if (g4 == 0) {
    m_s[wave][n] = (nbw > 0) ? r_ref : -INFINITY;    // a wave without blocks adds nothing
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
    const int g = e / kDD, jj = e % kDD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, m_s[w][g]);
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (m_s[w][g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_s[w][g] - M);
      acc += f * o_s[w][g][jj];
      L += f * l_s[w][g];
    }
    float* out = partials + ((h0 + g) * nsplit + split) * (kDD + 2);
    out[jj] = acc;
    if (jj == 0) {
      out[kDD] = M;
      out[kDD + 1] = L;
    }
  }
}

// ------------------------------------------------------------ logits only
// Raw logits of the G query heads sharing KV head s (same page, Stage 2
// closing paragraph): l_t = ||k_t|| <q', c[idx_t]> + sqrt(pi/2)/m ||r_t|| <u, 2 s_t - 1>
// with ||r_t|| the stored ||k|| ||r^||.  One workgroup per (split, KV head),
// the same tiles and block stream as decode (no value segment);
// out[(s*G + g) * T + t].  fu = sqrt(pi/2)/m rides on the sign fragments.
template <int G, int KB, int NK, bool MX = false>
__global__ __launch_bounds__(kDecThreads, (ring_occupancy<Packet<KB, 0, NK, 0, MX>, MX>())) void logits_mfma_kernel(
    const float* __restrict__ qr, const float* __restrict__ u, const float* __restrict__ ck,
    int64_t T, int64_t TpK, int split_len, const uint32_t* __restrict__ kcodes,
    const uint32_t* __restrict__ ksigns, const void* knorm, const void* krnorm, float fu,
    float* __restrict__ out, const float* __restrict__ ck_hi = nullptr) {
  using P = Packet<KB, 0, NK, 0, MX>;
  constexpr int kSlot = 4 * P::kBytes;
  __shared__ __align__(16) char lds[tab_bytes<MX>()];
  __shared__ __align__(16) char ring[kRing * kSlot];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int t0 = split * split_len;                  // T < 2^28 (checked on the host)
  const int Ti = static_cast<int>(T);
  const int t1 = (t0 + split_len < Ti) ? t0 + split_len : Ti;
  const int nb_split = (t1 - t0 + 31) / 32;
  const int nbw = (nb_split > wave) ? (nb_split - wave + 3) / 4 : 0;

  BlockStream<P> st;
  st.template init<KB, 0, NK, 0, MX>(kcodes, ksigns, knorm, krnorm, nullptr, nullptr, s * TpK + t0 + 32 * wave, 0,
                                     lane, lds_addr(ring) + wave * P::kBytes, kSlot);
#pragma unroll
  for (int jj = 0; jj + 1 < kRing; ++jj)
    if (jj < nbw) st.issue(jj, jj, lane);

  if constexpr (MX) build_tables_mix<KB, 0>(ck, ck_hi, nullptr, nullptr, lds, tid, kDecThreads);
  else build_tables<KB, 0, false>(ck, nullptr, lds, tid, kDecThreads);
  const char* ktab = lds + ((MX && g4 >= 2) ? narrow_key_off<KB + 1>() : 0);
  const uint32_t kbias = (MX && KB + 1 == 3 && g4 >= 2) ? kNarrowIndexBit : 0u;   // 2.5-bit keys
  half8 bq[8], bu[4];
  query_frags<G, false>(qr, u, s, lane, 1.f, fu, bq, bu);
  __syncthreads();

  float* out_h = out + (s * G + (n < G ? n : 0)) * T;
  const bool vec_ok = (Ti & 3) == 0;                  // 16-byte aligned output rows
  // this lane's byte offsets within a packet: key words, sign word, norms
  const uint32_t koff = P::kKC + (MX ? mix_key_lane_off<KB>(n, g4) : key_lane_off<KB>(n, g4));
  const uint32_t soff = P::kSG + 16 * n + 4 * g4;
  const uint32_t nkoff = 8 * NK * g4;
  int slot = 0;
  for (int j = 0; j < nbw; ++j) {
    st.advance(j, nbw, slot, lane);
    const uint32_t pko = slot * kSlot + wave * P::kBytes;   // the block's packet in the ring
    slot = (slot == kRing - 1) ? 0 : slot + 1;
    const char* kb = lds_at(ring, pko + koff);
    const char* sb = lds_at(ring, pko + soff);
    const char* nkb = lds_at(ring, pko + nkoff);
    const int tb = t0 + 32 * (wave + 4 * j);           // first token of the block
    float lv[8];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      float cen[4], qj[4];
      if constexpr (MX) {
        uint32_t kw[KB + 1];
        const uint32_t* kp = reinterpret_cast<const uint32_t*>(kb + 16 * (4 * KB + 2) * tile);
#pragma unroll
        for (int q = 0; q <= KB; ++q) kw[q] = kp[q];
        if (g4 >= 2) kw[KB] = 0u;
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(sb + 256 * tile);
        tile_logits<G, KB + 1, false, true>(kw, sw, bq, bu, lds, cen, qj, ktab, kbias);
      } else {
        uint32_t kw[KB], sw;
        ring_key_words<KB>(kb, sb, tile, kw, sw);
        tile_logits<G, KB, false>(kw, sw, bq, bu, lds, cen, qj);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lv[4 * tile + i] = fmaf(norm_at<NK>(nkb + P::kNK, 4 * tile + i), cen[i],
                                norm_at<NK>(nkb + P::kNR, 4 * tile + i) * qj[i]);
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

// ------------------------------------------------------------ logits, d up to 256
// The same logits at other head dimensions, up to d = 256 and m = 256 sketch
// rows (the pages' search vectors have d = 200: a2a-mcp.org page,
// "Benchmarks"): the records hold D = ceil(d/32) code-plane words and
// Dm = ceil(m/32) sign words per key, whose padding bits are zero.  A tile
// takes NP passes of 4 words (words 4p + g4 in lane group g4), each one
// group of centroid and sign K-steps added into the same accumulators; the
// query fragments are zero at coordinates >= d and sketch rows >= m, so the
// padding and the words past D or Dm contribute nothing.
//
// Blocks stream through an LDS ring by LDS DMA as in decode, in stream
// order (key records, sign words, the two norm rows: 4 D KB, 4 Dm and 2 NK
// bytes per token).  A ring slot is sized for D = Dm = 8, so that every lane
// of a fixed number of DMA loads per block lands inside it (the waits count
// loads): lanes past the block's real bytes re-read its first 16 bytes into
// the slot's unused end.  Per token a lane reads its KB words and sign word
// at a stride of D KB and Dm words, which spreads the 16 rows of a tile over
// the LDS banks (records are not a multiple of 16 bytes, so there is no
// reordering).

template <int KB, int NK>
struct WidePacket {
  static constexpr int kMaxBytes = 128 * 8 * KB + 128 * 8 + 64 * NK;
  static constexpr int kInstr = (kMaxBytes / 16 + 63) / 64;   // DMA loads per block
  static constexpr int kSlot = 1024 * kInstr;                 // bytes per wave and block
  static constexpr int kTail = 64;                            // every lane of every load
};

template <typename P>
struct WideStream {
  const char* src[P::kInstr];
  int step[P::kInstr];
  uint32_t ring0;   // LDS address of this wave's slot 0
  int kslot;        // bytes per ring slot (the 4 waves' packets)

  template <int KB, int NK>
  __device__ __forceinline__ void init(const uint32_t* kcodes, const uint32_t* ksigns, const void* knorm,
                                       const void* krnorm, int D, int Dm, int64_t tok, int lane,
                                       uint32_t ring_wave0, int slot_bytes) {
    ring0 = ring_wave0;
    kslot = slot_bytes;
    const int ck = 8 * D * KB, cs = 8 * Dm;   // 16-byte chunks of keys and signs per block
#pragma unroll
    for (int i = 0; i < P::kInstr; ++i) {
      const int c = 64 * i + lane;
      const char* p = reinterpret_cast<const char*>(kcodes) + tok * 4 * D * KB;   // past the packet
      int st = 0;
      if (c < ck) {
        p += 16 * c;
        st = 4 * 32 * 4 * D * KB;
      } else if (c < ck + cs) {
        p = reinterpret_cast<const char*>(ksigns) + tok * 4 * Dm + 16 * (c - ck);
        st = 4 * 32 * 4 * Dm;
      } else if (c < ck + cs + 4 * NK) {
        const int e = c - ck - cs, row = e / (2 * NK);
        p = reinterpret_cast<const char*>(row == 0 ? knorm : krnorm) + tok * NK + 16 * (e - 2 * NK * row);
        st = 4 * 32 * NK;
      }
      src[i] = p;
      step[i] = st;
    }
  }

  __device__ __forceinline__ void issue(int j, int slot) const {
    const uint32_t l = ring0 + slot * kslot;
#pragma unroll
    for (int i = 0; i < P::kInstr; ++i) dma16(src[i] + static_cast<int64_t>(j) * step[i], l + 1024 * i);
  }

  __device__ __forceinline__ void advance(int j, int nbw, int slot) const {
    if (j + kRing - 1 < nbw) {
      issue(j + kRing - 1, slot == 0 ? kRing - 1 : slot - 1);
      wait_vm<(kRing - 1) * P::kInstr>();
    } else if (kRing > 2 && j + 2 < nbw) {
      wait_vm<(kRing > 2 ? 2 : 0) * P::kInstr>();
    } else if (j + 1 < nbw) {
      wait_vm<P::kInstr>();
    } else {
      wait_vm<0>();
    }
  }
};

// This lane's fragments for pass p (coordinate words 4p .. 4p+3) of KV head
// s, from rotated queries of d floats and sketched ones of m floats per row.
template <int G>
__device__ __forceinline__ void query_frags_wide(const float* __restrict__ qr, const float* __restrict__ u,
                                                 int64_t s, int lane, float fu, int d, int m, int p,
                                                 half8 (&bq)[8], half8 (&bu)[4]) {
  const int n = lane & 15, g4 = lane >> 4;
  const bool hi_col = n < G, lo_col = (n >= G) && (n < 2 * G);
  const int g = hi_col ? n : (lo_col ? n - G : 0);
  const float* qg = qr + (s * G + g) * d;
  const float* ug = u + (s * G + g) * m;
  const int w0 = 32 * (4 * p + g4);
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
    for (int i = 0; i < 8; ++i) {
      const int j = w0 + 4 * c + kSlot[i];
      h[i] = part(j < d ? qg[j] : 0.f);
    }
    bq[c] = u4_to_h8(h2u(h[0], h[1]), h2u(h[2], h[3]), h2u(h[4], h[5]), h2u(h[6], h[7]));
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = w0 + 8 * c + i;
      h[i] = part(j < m ? fu * ug[j] : 0.f);
    }
    bu[c] = u4_to_h8(h2u(h[0], h[1]), h2u(h[2], h[3]), h2u(h[4], h[5]), h2u(h[6], h[7]));
  }
}

template <int G, int KB, int NK, int NP>
__global__ __launch_bounds__(kDecThreads, 2) void logits_wide_kernel(
    const float* __restrict__ qr, const float* __restrict__ u, const float* __restrict__ ck, int d, int m,
    int64_t T, int64_t TpK, int split_len, const uint32_t* __restrict__ kcodes,
    const uint32_t* __restrict__ ksigns, const void* knorm, const void* krnorm, float fu,
    float* __restrict__ out) {
  using P = WidePacket<KB, NK>;
  constexpr int kSlot = 4 * P::kSlot;   // one ring slot: the 4 waves' packets
  __shared__ __align__(16) char lds[kTabBytes];
  __shared__ __align__(16) char ring[kRing * kSlot];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int t0 = split * split_len;                  // T < 2^28 (checked on the host)
  const int Ti = static_cast<int>(T);
  const int t1 = (t0 + split_len < Ti) ? t0 + split_len : Ti;
  const int nb_split = (t1 - t0 + 31) / 32;
  const int nbw = (nb_split > wave) ? (nb_split - wave + 3) / 4 : 0;
  const int D = (d + 31) >> 5, Dm = (m + 31) >> 5;   // <= 4 NP (checked on the host)

  WideStream<P> st;
  st.template init<KB, NK>(kcodes, ksigns, knorm, krnorm, D, Dm, s * TpK + t0 + 32 * wave, lane,
                           lds_addr(ring) + wave * P::kSlot, kSlot);
#pragma unroll
  for (int jj = 0; jj + 1 < kRing; ++jj)
    if (jj < nbw) st.issue(jj, jj);

  build_tables<KB, 0, false>(ck, nullptr, lds, tid, kDecThreads);
  half8 bq[NP][8], bu[NP][4];
#pragma unroll
  for (int p = 0; p < NP; ++p) query_frags_wide<G>(qr, u, s, lane, fu, d, m, p, bq[p], bu[p]);
  __syncthreads();

  float* out_h = out + (s * G + (n < G ? n : 0)) * T;
  const bool vec_ok = (Ti & 3) == 0;                  // 16-byte aligned output rows
  // this lane's offsets within a packet: its tile-0 token's key words and
  // sign word (tile 1: 4 tokens on), and its group's 8 tokens' norms.  Words
  // past D or Dm read word 0 and are cleared.
  const int trow = 8 * (n >> 2) + (n & 3);
  uint32_t koff[NP], soff[NP];
  bool kin[NP], sin[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int w = 4 * p + g4;
    kin[p] = w < D;
    sin[p] = w < Dm;
    koff[p] = 4 * (trow * D * KB + (kin[p] ? w : 0) * KB);
    soff[p] = 128 * D * KB + 4 * (trow * Dm + (sin[p] ? w : 0));
  }
  const uint32_t ktile = 16 * D * KB, stile = 16 * Dm;   // 4 tokens of records
  const uint32_t nkoff = 128 * D * KB + 128 * Dm + 8 * NK * g4;
  int slot = 0;
  for (int j = 0; j < nbw; ++j) {
    st.advance(j, nbw, slot);
    const uint32_t pko = slot * kSlot + wave * P::kSlot;   // the block's packet in the ring
    slot = (slot == kRing - 1) ? 0 : slot + 1;
    const char* nkb = lds_at(ring, pko + nkoff);
    const int tb = t0 + 32 * (wave + 4 * j);           // first token of the block
    float lv[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      floatx4 accC = {0.f, 0.f, 0.f, 0.f}, accS = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t* kp = reinterpret_cast<const uint32_t*>(lds_at(ring, pko + koff[p] + tau * ktile));
        uint32_t kw[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q) kw[q] = kin[p] ? kp[q] : 0u;
        const uint32_t sw0 = *reinterpret_cast<const uint32_t*>(lds_at(ring, pko + soff[p] + tau * stile));
        const uint32_t sw = sin[p] ? sw0 : 0u;
        tile_accumulate<G, KB, false>(kw, sw, bq[p], bu[p], lds, accC, accS);
      }
      float cen[4], qj[4];
      tile_finish<G>(accC, accS, cen, qj);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lv[4 * tau + i] = fmaf(norm_at<NK>(nkb, 4 * tau + i), cen[i], norm_at<NK>(nkb + 32 * NK, 4 * tau + i) * qj[i]);
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

template <int G, int NP>
static void launch_logits_wide_np(dim3 grid, hipStream_t stream, const tq_tables& tk, const float* qr,
                                  const float* u, const tq_packed& k, int len, float fu, float* out) {
#define TQ_LW(KBV, NKV)                                                                                 \
  hipLaunchKernelGGL((logits_wide_kernel<G, KBV, NKV, NP>), grid, dim3(kDecThreads), 0, stream, qr, u,   \
                     tk.centroids, tk.d, tk.m, k.T, stream_stride(k), len, k.codes, k.signs, k.norm,     \
                     k.rnorm, fu, out)
  const bool f16 = k.norm_dtype == TQ_F16;
  switch (tk.bits) {
    case 1: if (f16) TQ_LW(1, 2); else TQ_LW(1, 4); break;
    case 2: if (f16) TQ_LW(2, 2); else TQ_LW(2, 4); break;
    case 3: if (f16) TQ_LW(3, 2); else TQ_LW(3, 4); break;
    default: if (f16) TQ_LW(4, 2); else TQ_LW(4, 4); break;
  }
#undef TQ_LW
}

template <int G>
static hipError_t launch_logits_wide_g(const tq_tables& tk, const float* qr, const float* u, int64_t nseq,
                                       const tq_packed& k, int len, int nsplit, float* out, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(nsplit), static_cast<unsigned>(nseq));
  const float fu = 1.2533141373155003f / static_cast<float>(tk.m);   // sqrt(pi/2) / m
  const int words = ((tk.d > tk.m ? tk.d : tk.m) + 31) / 32;
  if (words <= 4) launch_logits_wide_np<G, 1>(grid, stream, tk, qr, u, k, len, fu, out);
  else launch_logits_wide_np<G, 2>(grid, stream, tk, qr, u, k, len, fu, out);
  return hipGetLastError();
}

template <int G, int KB, int VB>
static void launch_norms(dim3 grid, hipStream_t stream, const tq_tables& tk, const tq_tables& tv,
                         const float* qr, const float* u, const tq_packed& k, const tq_packed& v,
                         int len, float fq, float fu, int nsplit, float* partials) {
#define TQ_DEC(NKB, NVB)                                                                       \
  hipLaunchKernelGGL((decode_mfma_kernel<G, KB, VB, NKB, NVB>), grid, dim3(kDecThreads), 0,    \
                     stream, qr, u, tk.centroids, tv.centroids, k.T, stream_stride(k),         \
                     stream_stride(v), len, k.codes, k.signs,                                  \
                     k.norm, k.rnorm, v.codes, v.norm, fq, fu, nsplit, partials)
  const bool k16 = k.norm_dtype == TQ_F16, v16 = v.norm_dtype == TQ_F16;
  if (k16 && v16) TQ_DEC(2, 2);
  else if (k16) TQ_DEC(2, 4);
  else if (v16) TQ_DEC(4, 2);
  else TQ_DEC(4, 4);
#undef TQ_DEC
}

template <int G, int KB>
static void launch_vb(int vb, dim3 grid, hipStream_t stream, const tq_tables& tk,
                      const tq_tables& tv, const float* qr, const float* u, const tq_packed& k,
                      const tq_packed& v, int len, float fq, float fu, int nsplit, float* partials) {
  switch (vb) {
    case 1: launch_norms<G, KB, 1>(grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials); break;
    case 2: launch_norms<G, KB, 2>(grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials); break;
    case 3: launch_norms<G, KB, 3>(grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials); break;
    default: launch_norms<G, KB, 4>(grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials); break;
  }
}

// split streams (validated: both split, bits 2 or 3 each, float16 norms)
template <int G, int KB, int VB>
static void launch_mix(dim3 grid, hipStream_t stream, const tq_tables& tk, const tq_tables& tv,
                       const float* qr, const float* u, const tq_packed& k, const tq_packed& v, int len,
                       float fq, float fu, int nsplit, float* partials) {
  hipLaunchKernelGGL((decode_mfma_kernel<G, KB, VB, 2, 2, true>), grid, dim3(kDecThreads), 0, stream, qr, u,
                     tk.centroids, tv.centroids, k.T, stream_stride(k), stream_stride(v), len, k.codes,
                     k.signs, k.norm, k.rnorm, v.codes, v.norm, fq, fu, nsplit, partials, tk.centroids_hi,
                     tv.centroids_hi);
}

template <int G>
static hipError_t launch_g(const tq_tables& tk, const tq_tables& tv, const float* qr,
                           const float* u, int64_t nseq, const tq_packed& k, const tq_packed& v,
                           float fq, float fu, float* partials, int len, int nsplit,
                           hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(nsplit), static_cast<unsigned>(nseq));
  if (tk.hi_coords != 0) {
    if (tk.bits == 2 && tv.bits == 2) launch_mix<G, 2, 2>(grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials);
    else if (tk.bits == 2) launch_mix<G, 2, 3>(grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials);
    else if (tv.bits == 2) launch_mix<G, 3, 2>(grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials);
    else launch_mix<G, 3, 3>(grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials);
    return hipGetLastError();
  }
  switch (tk.bits) {
    case 1: launch_vb<G, 1>(tv.bits, grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials); break;
    case 2: launch_vb<G, 2>(tv.bits, grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials); break;
    case 3: launch_vb<G, 3>(tv.bits, grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials); break;
    default: launch_vb<G, 4>(tv.bits, grid, stream, tk, tv, qr, u, k, v, len, fq, fu, nsplit, partials); break;
  }
  return hipGetLastError();
}

template <int G>
static hipError_t launch_logits_g(const tq_tables& tk, const float* qr, const float* u,
                                  int64_t nseq, const tq_packed& k, int len, int nsplit, float* out,
                                  hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(nsplit), static_cast<unsigned>(nseq));
  const float fu = 1.2533141373155003f / static_cast<float>(tk.m);   // sqrt(pi/2) / m
#define TQ_LOG(KBV)                                                                                \
  do {                                                                                             \
    if (k.norm_dtype == TQ_F16)                                                                    \
      hipLaunchKernelGGL((logits_mfma_kernel<G, KBV, 2>), grid, dim3(kDecThreads), 0, stream, qr,  \
                         u, tk.centroids, k.T, stream_stride(k), len, k.codes, k.signs, k.norm,    \
                         k.rnorm, fu, out);                                                        \
    else                                                                                           \
      hipLaunchKernelGGL((logits_mfma_kernel<G, KBV, 4>), grid, dim3(kDecThreads), 0, stream, qr,  \
                         u, tk.centroids, k.T, stream_stride(k), len, k.codes, k.signs, k.norm,    \
                         k.rnorm, fu, out);                                                        \
  } while (0)
  if (tk.hi_coords != 0) {   // split keys (validated: bits 2 or 3)
#define TQ_LOGM(KBV, NKV)                                                                          \
  hipLaunchKernelGGL((logits_mfma_kernel<G, KBV, NKV, true>), grid, dim3(kDecThreads), 0, stream, qr, u, \
                     tk.centroids, k.T, stream_stride(k), len, k.codes, k.signs, k.norm, k.rnorm, fu, out,  \
                     tk.centroids_hi)
    const bool f16 = k.norm_dtype == TQ_F16;
    if (tk.bits == 2) { if (f16) TQ_LOGM(2, 2); else TQ_LOGM(2, 4); }
    else { if (f16) TQ_LOGM(3, 2); else TQ_LOGM(3, 4); }
#undef TQ_LOGM
    return hipGetLastError();
  }
  switch (tk.bits) {
    case 1: TQ_LOG(1); break;
    case 2: TQ_LOG(2); break;
    case 3: TQ_LOG(3); break;
    default: TQ_LOG(4); break;
  }
#undef TQ_LOG
  return hipGetLastError();
}

// The per-G launchers that decode_g<G>.hip instantiate.
#define TQ_DECODE_G_TU(GV)                                                                         \
  hipError_t decode_launch_g##GV(const tq_tables& tk, const tq_tables& tv, const float* qr,        \
                                 const float* u, int64_t nseq, const tq_packed& k,                 \
                                 const tq_packed& v, float fq, float fu, float* partials, int len, \
                                 int nsplit, hipStream_t stream) {                                 \
    return launch_g<GV>(tk, tv, qr, u, nseq, k, v, fq, fu, partials, len, nsplit, stream);         \
  }                                                                                                \
  hipError_t logits_launch_g##GV(const tq_tables& tk, const float* qr, const float* u,             \
                                 int64_t nseq, const tq_packed& k, int len, int nsplit,            \
                                 float* out, hipStream_t stream) {                                 \
    return launch_logits_g<GV>(tk, qr, u, nseq, k, len, nsplit, out, stream);                      \
  }                                                                                                \
  hipError_t logits_wide_launch_g##GV(const tq_tables& tk, const float* qr, const float* u,        \
                                      int64_t nseq, const tq_packed& k, int len, int nsplit,       \
                                      float* out, hipStream_t stream) {                            \
    return launch_logits_wide_g<GV>(tk, qr, u, nseq, k, len, nsplit, out, stream);                 \
  }

}  // namespace tq
