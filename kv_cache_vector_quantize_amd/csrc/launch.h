// Internal launchers (host side), one per kernel family.  Arguments have
// been validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/tq.h"

namespace tq {

// Tokens stored per sequence in a packed stream (its row stride).
inline int64_t stream_stride(const tq_packed& p) {
  return p.capacity != 0 ? static_cast<int64_t>(p.capacity) : (p.T + 31) / 32 * 32;
}

hipError_t launch_codebook(int d, int bits, double* c64, double* b64, float* c32, float* b32,
                           hipStream_t stream);

hipError_t launch_rotation(int d, const double* G, double* Q, float* Q32, hipStream_t stream);

hipError_t launch_hadamard_rotation(int d, const float* signs, float* rot32, hipStream_t stream);

// Quantizes tokens pos .. pos+n-1 of every sequence (x holds n tokens per
// sequence) into `out`.  append = false: the whole stream (pos = 0, n = T);
// append = true: tokens below pos are kept.
hipError_t launch_quantize(const tq_tables& t, const void* x, int x_dtype, const tq_packed& out,
                           int64_t pos, int64_t n, bool append, hipStream_t stream);

// Pre-rotated queries: qr[h][d] = Pi q, u[h][m] = S qr, for nh = B*Hq heads.
hipError_t launch_qprep(const tq_tables& tk, const void* q, int q_dtype, int nh, float* qr,
                        float* u, hipStream_t stream);

hipError_t launch_logits(const tq_tables& tk, const float* qr, const float* u, int B, int Hq,
                         int Hkv, const tq_packed& k, float* logits, hipStream_t stream);

// Split-K decode.  Workspace: rotated queries (qr, u), then one
// (acc[d], max, sum) partial per query head and split.
struct DecodeWorkspace {
  size_t qr, u, partials, total;
};
DecodeWorkspace decode_workspace_layout(int B, int Hq, int Hkv, int64_t T, int d, int m);
hipError_t launch_decode(const tq_tables& tk, const tq_tables& tv, const float* qr, const float* u,
                         int B, int Hq, int Hkv, const tq_packed& k, const tq_packed& v,
                         float scale, void* ws, const DecodeWorkspace& lay, float* out,
                         hipStream_t stream);

// Logits through the decode tiles (G = Hq/Hkv in {1, 2, 4, 8}) from the
// rotated queries.
hipError_t launch_logits_mfma(const tq_tables& tk, const float* qr, const float* u, int B, int Hq,
                              int Hkv, const tq_packed& k, float* logits, hipStream_t stream);

// Logits on the matrix cores at any d <= 256 and 1 <= m <= 256 from the
// rotated queries of launch_qprep_generic (rows of d and m floats), for
// G = Hq/Hkv in {1, 2, 4, 8} and keys of one width.
hipError_t launch_logits_wide(const tq_tables& tk, const float* qr, const float* u, int B, int Hq,
                              int Hkv, const tq_packed& k, float* logits, hipStream_t stream);

// Head dimensions other than 128 (d <= 256, m <= 256): vector-ALU quantize,
// query preparation and logits (generic.hip).
hipError_t launch_quantize_generic(const tq_tables& t, const void* x, int x_dtype, const tq_packed& out,
                                   hipStream_t stream);
hipError_t launch_qprep_generic(const tq_tables& tk, const void* q, int q_dtype, int nh, float* qr, float* u,
                                hipStream_t stream);
hipError_t launch_logits_generic(const tq_tables& tk, const float* qr, const float* u, int B, int Hq, int Hkv,
                                 const tq_packed& k, float* logits, hipStream_t stream);

// Top-k of each score row (k <= 32): chunk lists in ws, then one merge per row.
int64_t topk_chunks(int64_t n);
size_t topk_workspace(int64_t rows, int64_t n, int k);
hipError_t launch_topk(const float* scores, int64_t rows, int64_t n, int k, int32_t* idx, float* val, void* ws,
                       hipStream_t stream);

}  // namespace tq
