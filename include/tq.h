/*
 * tq.h -- C ABI of libtq.so: TurboQuant KV-cache vector quantization and
 * decode attention from the packed codes, for AMD Instinct MI355X (gfx950).
 *
 * The method (Zandieh et al., "TurboQuant: Online Vector Quantization with
 * Near-optimal Distortion Rate") as the source pages describe it:
 *   - a data-independent random orthogonal rotation, the Q factor of a
 *     Gaussian matrix, drawn once and cached
 *     (a2a-mcp.org/blog/what-is-turboquant-ja, "How it works", Stage 1;
 *      deepsignal-app.com article, QJL section);
 *   - after rotation each coordinate of the normalised vector follows
 *     Beta((d-1)/2,(d-1)/2) on [-1,1], so an MSE-optimal Lloyd-Max scalar
 *     codebook can be precomputed per (head dim, bit width)
 *     (same page, Stage 1; "How to implement", item 1;
 *      qiita.com/okssusucha/items/81738e4261f2841d40f8, "Rotate, then quantize");
 *   - for keys, a 1-bit quantized JL transform (random projection + sign) of
 *     the residual left by the MSE stage makes inner products unbiased
 *     (Stage 2; qiita page, "One more stage so attention doesn't break");
 *   - attention logits are computed straight from the stored indices with a
 *     query rotated once, with no pass that dequantizes the cache
 *     (Stage 2 closing paragraph; "How to implement", item 1).
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers unless stated otherwise.  The
 *     caller allocates and owns every buffer; the library never allocates or
 *     frees device memory and keeps no pointer after the call returns.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); the
 *     call never synchronizes.  Buffers must stay valid until the stream has
 *     executed the work.
 *   - Arguments are validated on the host before anything is launched.  A
 *     bad argument returns TQ_EINVAL (nothing launched); a shape or width the
 *     kernels were not built for returns TQ_EUNSUPPORTED; a workspace smaller
 *     than the matching *_workspace() size returns TQ_EWORKSPACE; a failed
 *     launch returns TQ_EHIP.  Errors raised by earlier, unrelated work on the
 *     stream are not reported here.
 *   - Device pointers must be 16-byte aligned.  Layouts are dense, row-major,
 *     little-endian.  No global mutable state: calls are thread-safe.
 *
 * Packed layout (bit k of a uint32 word is (word >> k) & 1).  Every stream
 * stores Tp tokens per sequence, Tp = the stream's capacity (a multiple of 32,
 * at least T) or, with capacity 0, 32 * ceil(T / 32): the context is cut into
 * 32-token blocks, so every block of every sequence starts 16-byte aligned
 * and can be streamed whole.  tq_quantize writes tokens T .. 32*ceil(T/32)-1
 * as padding (keys: the encoding of a zero vector; values: fields 0; norms
 * 0); tokens at or past T never contribute to a result.
 *   key stream   codes[s][Tp][d/32][bits] bit k of word (w,p) = bit p of idx[s][t][32w+k]
 *                signs[s][Tp][m/32]       bit k of word w     = [z[s][t][32w+k] >= 0]
 *                norm[s][Tp]  = ||k||,  rnorm[s][Tp] = ||k|| * ||r||
 *   value stream codes[s][Tp/32][d][bits]
 *                the `bits` words (B,j,0..bits-1) form one little-endian
 *                record of 32*bits bits: token k of block B holds
 *                idx[s][32B+k][j] in record bits [bits*k, bits*k+bits)
 *                (a field may straddle two words); fields of tokens past
 *                T are 0.                    norm[s][Tp] = ||v||
 *   idx = number of codebook boundaries <= the rotated, normalised coordinate.
 *   z = S r, r = Pi x/||x|| - centroid[idx] (rotated domain, unit scale).
 *   Norms are float32 or float16 (round to nearest even), per tq_packed.
 *   A zero vector stores norms 0, idx 2^(bits-1) everywhere and sign bits 1.
 *
 * Fractional widths (split streams, hi_coords > 0): the first hi_coords
 * rotated coordinates are quantized with the (bits+1)-bit codebook
 * (centroids_hi / bounds_hi), the others with the bits-bit one -- bits + 1/2
 * per coordinate for hi_coords = d/2, e.g. 2.5 and 3.5 (qiita page, "Which
 * bit width is 'lossless'?", first table; the split of the rotated
 * coordinates is this library's reading, the pages give no mechanism).  The
 * layouts keep the rules above, each coordinate word (keys) or coordinate
 * (values) taking its own width, concatenated in coordinate order:
 *   key stream   codes[s][Tp][W], W = (d/32) bits + hi_coords/32: the planes
 *                of word w (bits+1 of them for 32 w < hi_coords, else bits)
 *                at record word sum of the widths of words 0..w-1
 *   value stream codes[s][Tp/32][V], V = d bits + hi_coords: the record of
 *                coordinate j (bits+1 words for j < hi_coords, else bits) at
 *                record word sum of the widths of coordinates 0..j-1
 *   A zero vector stores idx 2^(width-1) at each coordinate.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 6

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,        /* bad argument; nothing launched */
  TQ_EUNSUPPORTED = -2,  /* valid, but not a shape/width the kernels support */
  TQ_EWORKSPACE = -3,    /* workspace smaller than required */
  TQ_EHIP = -4           /* HIP launch / runtime error */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

typedef enum { TQ_KEY = 0, TQ_VALUE = 1 } tq_role;

/* What `rot` of a tq_tables holds. */
typedef enum {
  TQ_ROT_DENSE = 0,     /* any orthogonal Pi (tq_rotation: QR of a Gaussian)       */
  TQ_ROT_HADAMARD = 1   /* H_d diag(s) / sqrt(d) as written by tq_hadamard_rotation */
} tq_rotation_kind;

/* Data-independent tables of one stream (device memory, caller-owned). */
typedef struct {
  int32_t d;               /* head dimension: 128 on every path; 8..256 for      */
                           /* quantize and logits (padded to 32-bit words)        */
  int32_t m;               /* sketch rows of keys (128 at d = 128, <= 256 else);  */
                           /* 0 for values                                         */
  int32_t bits;            /* code width, 1..4                                    */
  int32_t rot_kind;        /* tq_rotation_kind of rot                             */
  const float *rot;        /* Pi, d x d row-major; y = Pi x                       */
  const float *sketch;     /* S, m x d row-major, iid N(0,1); NULL when m == 0    */
  const float *centroids;  /* 2^bits ascending, unit-sphere scale                 */
  const float *bounds;     /* 2^bits - 1 ascending decision boundaries            */
  int32_t hi_coords;       /* leading rotated coordinates at bits + 1: 0 (every  */
                           /* coordinate at bits) or d/2 (bits + 1/2 per coord)   */
  const float *centroids_hi; /* 2^(bits+1) centroids, NULL when hi_coords == 0    */
  const float *bounds_hi;  /* 2^(bits+1) - 1 boundaries, NULL when hi_coords == 0 */
  int32_t sketch_f16;      /* 1: the caller promises that every entry of sketch */
                           /* is exact in float16, and whole key streams then   */
                           /* compute S r as R_hi S + R_lo S (a lo half of S    */
                           /* would be ignored); 0: any float32 S.  0 for values */
} tq_tables;

/* A packed key or value stream of nseq sequences of T tokens (caller-owned). */
typedef struct {
  int32_t role;            /* tq_role                                             */
  int32_t bits;            /* must equal the tables' bits                         */
  int32_t d;               /* must equal the tables' d                            */
  int32_t m;               /* keys: the tables' m (> 0); values: 0                */
  int64_t nseq;            /* sequences (batch x kv heads), >= 0                  */
  int64_t T;               /* tokens per sequence, >= 0                           */
  uint32_t *codes;         /* layout above                                        */
  uint32_t *signs;         /* keys only, else NULL                                */
  void *norm;              /* [nseq][Tp] of norm_dtype                            */
  void *rnorm;             /* keys only, [nseq][Tp] of norm_dtype, else NULL      */
  int32_t norm_dtype;      /* TQ_F32 or TQ_F16                                    */
  int32_t capacity;        /* tokens stored per sequence (Tp): 0, or a multiple   */
                           /* of 32 that is >= T (a cache that grows by append)   */
  int32_t hi_coords;       /* must equal the tables' hi_coords                    */
} tq_packed;

/* Version of this ABI (TQ_ABI_VERSION of the built library). */
int tq_abi_version(void);

/* Static string for a status code; never NULL. */
const char *tq_status_str(int status);

/*
 * tq_codebook -- Lloyd-Max codebook for Beta((d-1)/2,(d-1)/2) on [-1,1].
 * Cites: a2a-mcp.org page, "How it works", Stage 1 (the Beta law, optimal
 * centroids precomputed); "How to implement", item 1 (codebook per head dim
 * and width); qiita page, "Rotate, then quantize" (Lloyd-Max per coordinate).
 * Iterates the two Lloyd conditions (boundary = midpoint of neighbouring
 * centroids, centroid = conditional mean of its cell) in float64 until no
 * centroid moves by 1e-15.  Setup: run once per (d, bits).
 *   d            3..4096
 *   bits         1..4
 *   centroids64  out, 2^bits doubles, or NULL
 *   bounds64     out, 2^bits - 1 doubles, or NULL
 *   centroids32  out, 2^bits floats (round to nearest), required
 *   bounds32     out, 2^bits - 1 floats, required
 */
tq_status tq_codebook(int d, int bits, double *centroids64, double *bounds64,
                      float *centroids32, float *bounds32, hipStream_t stream);

/*
 * tq_rotation -- Pi = Q diag(sign(diag R)) for G = Q R (Householder QR in
 * float64), the unique QR factor with a positive diagonal.
 * Cites: a2a-mcp.org page, "How it works", Stage 1 (QR of a Gaussian matrix);
 * deepsignal-app.com page, QJL section (drawn once before inference, cached).
 * Setup helper; G is an input drawn by the caller (iid N(0,1)).
 *   d      2..1024 (up to 128 in LDS; past 128 in rot64, an L2-resident
 *          working copy)
 *   G      in, d x d row-major doubles
 *   rot64  out, d x d row-major doubles (also used as working storage)
 *   rot32  out, d x d row-major floats (round to nearest), or NULL
 */
tq_status tq_rotation(int d, const double *G, double *rot64, float *rot32, hipStream_t stream);

/*
 * tq_hadamard_rotation -- the randomized Walsh-Hadamard rotation
 * Pi_H = H_d diag(s) / sqrt(d), H_d Sylvester's Hadamard matrix
 * (H_d[j][k] = (-1)^popcount(j & k)), s a vector of d random signs.
 * Cites: qiita page, "What you hit when you try it" (implementations that
 * stand a Walsh-Hadamard transform in for the rotation).  Setup helper;
 * tables with rot_kind TQ_ROT_HADAMARD must hold its output.  Since
 * sqrt(d) Pi_H has entries +-1, exact in float16, quantization rotates with
 * one matrix-core product instead of the hi + lo pair a general Pi needs.
 *   d      power of two, 2..4096
 *   signs  in, d floats; s_k = -1 where the sign bit of signs[k] is set, else +1
 *   rot32  out, d x d row-major floats: +-(1/sqrt(d)) rounded to nearest
 */
tq_status tq_hadamard_rotation(int d, const float *signs, float *rot32, hipStream_t stream);

/*
 * tq_quantize -- online quantization of key or value vectors.
 * Cites: a2a-mcp.org page, "How it works", Stage 1 (normalise, rotate,
 * Lloyd-Max per coordinate) and Stage 2 (1-bit QJL of the residual, keys);
 * "How to implement", item 1 (quantize on every cache update).
 *   t      tables of the stream (t->m > 0 for keys, 0 for values)
 *   x      in, [out->nseq][out->T][d] of x_dtype (TQ_F32 or TQ_BF16)
 *   out    packed stream to write; role, bits, d, m, hi_coords must match t
 * d = 128 with m = 128 (keys) runs on the matrix cores; other d in 8..256 and
 * m <= 256 on the vector ALU.  Split streams (hi_coords = d/2) take d = 128,
 * bits 1..3 and a dense rotation (TQ_EUNSUPPORTED otherwise).
 */
tq_status tq_quantize(const tq_tables *t, const void *x, int x_dtype, const tq_packed *out,
                      hipStream_t stream);

/*
 * tq_append -- quantize n new tokens per sequence onto the end of a stream:
 * the cache update of every decode step, which quantizes each new key and
 * value as it arrives.
 * Cites: a2a-mcp.org page, "How to implement", item 1 (quantize on every
 * cache update); "How it works" (online, data-independent: a token's record
 * depends on that token alone).
 *   t      tables of the stream
 *   x      in, [out->nseq][n][d] of x_dtype (TQ_F32 or TQ_BF16)
 *   n      new tokens per sequence, >= 0
 *   out    a stream holding out->T tokens whose capacity is nonzero and at
 *          least out->T + n (else TQ_EINVAL)
 * Writes tokens T .. T+n-1 with the records tq_quantize gives them, and
 * tokens T+n .. 32*ceil((T+n)/32)-1 as padding; the records of tokens below
 * T are kept (the value record of the block holding token T is merged in
 * place).  After the call the stream equals, bit for bit, tq_quantize of all
 * T+n tokens at the same capacity.  out->T is the caller's to advance: pass
 * T+n to later calls.  Calls that write one stream must not overlap.
 * d = 128 (and m = 128 for keys) only (TQ_EUNSUPPORTED otherwise).
 */
tq_status tq_append(const tq_tables *t, const void *x, int x_dtype, int64_t n, const tq_packed *out,
                    hipStream_t stream);

/* Workspace bytes for tq_attn_logits (the rotated queries). */
size_t tq_logits_workspace(int B, int Hq, int d, int m);

/*
 * tq_attn_logits -- raw <q, k> estimates straight from packed keys:
 *   l = ||k|| <Pi q, c[idx]> + sqrt(pi/2)/m * ||k|| ||r|| <S Pi q, 2s - 1>.
 * Cites: a2a-mcp.org page, Stage 2 closing paragraph and "How to implement",
 * item 1 (query rotated once, dots from indices, no dequantization pass);
 * qiita page, "One more stage..." (unbiased inner product).
 *   tk       key tables
 *   q        in, [B][Hq][d] of q_dtype (TQ_F32 or TQ_BF16)
 *   k        packed keys, nseq = B*Hkv, sequence index b*Hkv + g
 *   logits   out, [B][Hq][T] float32; query head h reads kv head h/(Hq/Hkv)
 *   ws       workspace of at least tq_logits_workspace(B, Hq, d, m) bytes
 * Hq/Hkv must be 1, 2, 4, 8 or 16 (else TQ_EUNSUPPORTED); T < 2^28 and
 * B*Hkv <= 65535 (else TQ_EUNSUPPORTED).  A split key stream (hi_coords =
 * d/2) takes bits 2 or 3 and Hq/Hkv <= 8.  Head dimensions other than 128
 * (d <= 256, m <= 256) run on the same matrix-core tiles in one or two passes of
 * 128 coordinates for Hq/Hkv <= 8, on the vector ALU for 16.
 */
tq_status tq_attn_logits(const tq_tables *tk, const void *q, int q_dtype, int B, int Hq, int Hkv,
                         const tq_packed *k, float *logits, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Workspace bytes for tq_attn_decode (rotated queries + split partials). */
size_t tq_decode_workspace(int B, int Hq, int Hkv, int64_t T, int d, int m);

/*
 * tq_attn_decode -- one query token per (batch, query head) attends to all T
 * cached tokens: softmax(scale * l) over the logits above, then the weighted
 * sum of the values, accumulated in the rotated domain from the value codes
 * and rotated back once (out = Pi^T sum_t a_t ||v_t|| c_V[idx_t]).
 * Cites: a2a-mcp.org page, Stage 2 closing paragraph (no full dequantization
 * during inference); "How to implement", item 1.
 *   tk, tv   key / value tables of the same d; each may have its own rotation
 *            (queries are rotated with tk->rot, the output back with tv->rot)
 *   q        in, [B][Hq][d] of q_dtype
 *   k, v     packed keys and values, nseq = B*Hkv, same T >= 1
 *   scale    softmax scale, > 0 (1/sqrt(d) for standard attention)
 *   out      out, [B][Hq][d] float32
 *   ws       workspace of at least tq_decode_workspace(B, Hq, Hkv, T, d, m) bytes
 * d = 128 with m = 128, Hq/Hkv 1, 2, 4 or 8, T < 2^28 and B*Hkv <= 65535
 * (else TQ_EUNSUPPORTED).  Key and value norms may be stored as float16 or float32
 * independently.  Split streams (hi_coords = d/2: 2.5 / 3.5-bit keys or
 * values) are decoded when both streams are split, with bits 2 or 3 each and
 * float16 norms (else TQ_EUNSUPPORTED).  Logits carry float32-grade accuracy (float16 hi/lo operand
 * pairs, float32 accumulation); the value weights enter the value contraction
 * as float16 (at most 2^8 relative to the running maximum): out matches an
 * exact evaluation to a few 1e-4 of its norm (the tests bound it by 2e-3).
 */
tq_status tq_attn_decode(const tq_tables *tk, const tq_tables *tv, const void *q, int q_dtype,
                         int B, int Hq, int Hkv, const tq_packed *k, const tq_packed *v,
                         float scale, float *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * tq_attn_decode_static -- tq_attn_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same computation, same kernels; the
 * workspace is an array the library keeps in the memory of every GPU it runs
 * on (tq_attn_decode_static_capacity() bytes, 16 MiB, held until the process
 * ends).  The call allocates nothing and calls no allocating routine.
 *   Arguments as tq_attn_decode, without ws / ws_bytes.
 *   TQ_EWORKSPACE when tq_decode_workspace() of the call's shape exceeds the
 *   capacity (about 30,000 query-head x split partials: e.g. 512 query heads
 *   over 131072 tokens need 4.8 MB, 64 heads over 524288 tokens 3.3 MB).
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents (each call writes every byte of it that it reads
 * before reading it).  Calls whose execution overlaps on one GPU -- on
 * different streams, or from threads that do not order their streams --
 * race on the array and must not be issued; calls on one stream are ordered.
 */
size_t tq_attn_decode_static_capacity(void);
tq_status tq_attn_decode_static(const tq_tables *tk, const tq_tables *tv, const void *q, int q_dtype,
                                int B, int Hq, int Hkv, const tq_packed *k, const tq_packed *v,
                                float scale, float *out, hipStream_t stream);

/* Workspace bytes for tq_topk (0 for invalid sizes). */
size_t tq_topk_workspace(int64_t rows, int64_t n, int k);

/*
 * tq_topk -- the k largest entries of every row of a score matrix: the
 * selection step of inner-product search over packed keys, whose scores are
 * the tq_attn_logits estimates.
 * Cites: a2a-mcp.org page, "Benchmarks" (vector search judged by top-k
 * recall); "How it works" (inner products estimated straight from codes).
 * An entry ranks above another if its score is larger, or the scores are
 * equal (-0 equals +0) and its column is smaller; each row's result is in
 * that order.
 *   scores   in, [rows][n] float32, no NaN
 *   rows     0..65535
 *   n        1..2^31-1 columns
 *   k        1..32, k <= n
 *   idx      out, [rows][k] int32 column indices
 *   val      out, [rows][k] float32 scores (as stored, -0 returned as +0)
 *   ws       workspace of at least tq_topk_workspace(rows, n, k) bytes
 */
tq_status tq_topk(const float *scores, int64_t rows, int64_t n, int k, int32_t *idx, float *val,
                  void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
