// Split-K decode: the combine kernel, the split length, the workspace layout
// and the entry launchers; the main kernels are in decode_kernels.h.
#include "decode_kernels.h"

namespace tq {

// per-G launchers (decode_g<G>.hip)
#define TQ_DECL_G(GV)                                                                              \
  hipError_t decode_launch_g##GV(const tq_tables& tk, const tq_tables& tv, const float* qr,        \
                                 const float* u, int64_t nseq, const tq_packed& k,                 \
                                 const tq_packed& v, float fq, float fu, float* partials, int len, \
                                 int nsplit, hipStream_t stream);                                  \
  hipError_t logits_launch_g##GV(const tq_tables& tk, const float* qr, const float* u,             \
                                 int64_t nseq, const tq_packed& k, int len, int nsplit,            \
                                 float* out, hipStream_t stream);                                  \
  hipError_t logits_wide_launch_g##GV(const tq_tables& tk, const float* qr, const float* u,        \
                                      int64_t nseq, const tq_packed& k, int len, int nsplit,       \
                                      float* out, hipStream_t stream);
TQ_DECL_G(1)
TQ_DECL_G(2)
TQ_DECL_G(4)
TQ_DECL_G(8)
#undef TQ_DECL_G

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

// Split length: about `target` workgroups in all, in whole 32-token blocks,
// at most `cap` (kLogMaxSplit, kDecMaxSplit).  Decode aims at exactly one
// round of the chip (its resident workgroups per CU x 256 CUs): a second,
// partial round leaves most CUs idle at the tail (1024 workgroups at 3 per
// CU ran 6% slower than 768 for 8 sequences of 524288 tokens).  Logits aim at
// one round of two per CU: for 8 sequences of 32768 tokens, 512 workgroups of
// 512 tokens took 18 us against 19-20 us for 1024 of 256 (more set-up per
// token) and 19 us for 256 of 1024.
constexpr int kCus = 256;
constexpr int kLogTarget = 2 * kCus;

static int split_length(int64_t nseq, int64_t T, int cap, int64_t target) {
  int64_t per_seq = (target + nseq - 1) / nseq;
  if (per_seq < 1) per_seq = 1;
  int64_t len = (T + per_seq - 1) / per_seq;
  len = ((len + 31) / 32) * 32;
  if (len < 128) len = 128;
  if (len > cap) len = cap;
  return static_cast<int>(len);
}

static size_t a256(size_t x) { return (x + 255u) & ~static_cast<size_t>(255u); }

DecodeWorkspace decode_workspace_layout(int B, int Hq, int Hkv, int64_t T, int d, int m) {
  DecodeWorkspace w{};
  const size_t nh = static_cast<size_t>(B) * Hq;
  const int64_t nseq = static_cast<int64_t>(B) * Hkv;
  // the most splits any decode launch of this shape uses (3 resident per CU)
  const int64_t len = split_length(nseq > 0 ? nseq : 1, T, kDecMaxSplit, 3 * kCus);
  const size_t nsplit = static_cast<size_t>((T + len - 1) / len);
  w.qr = 0;
  w.u = a256(nh * d * sizeof(float));
  w.partials = w.u + a256(nh * m * sizeof(float));
  w.total = w.partials + a256(nh * nsplit * (d + 2) * sizeof(float));
  return w;
}

hipError_t launch_decode(const tq_tables& tk, const tq_tables& tv, const float* qr, const float* u,
                         int B, int Hq, int Hkv, const tq_packed& k, const tq_packed& v,
                         float scale, void* ws, const DecodeWorkspace& lay, float* out,
                         hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t nseq = static_cast<int64_t>(B) * Hkv;
  const bool mx = tk.hi_coords != 0;
  const int occ = ring_occupancy_bytes(packet_bytes(k.bits, v.bits, k.norm_dtype == TQ_F16 ? 2 : 4,
                                                    v.norm_dtype == TQ_F16 ? 2 : 4, mx), mx);
  const int len = split_length(nseq, k.T, kDecMaxSplit, static_cast<int64_t>(occ) * kCus);
  const int nsplit = static_cast<int>((k.T + len - 1) / len);
  // the softmax runs in base 2: the query fragments carry scale * log2(e),
  // the sign fragments also the QJL factor sqrt(pi/2) / m
  const float fq = scale * 1.4426950408889634f;
  const float fu = fq * (1.2533141373155003f / static_cast<float>(tk.m));
  float* partials = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.partials);
  hipError_t e;
  switch (G) {
    case 1: e = decode_launch_g1(tk, tv, qr, u, nseq, k, v, fq, fu, partials, len, nsplit, stream); break;
    case 2: e = decode_launch_g2(tk, tv, qr, u, nseq, k, v, fq, fu, partials, len, nsplit, stream); break;
    case 4: e = decode_launch_g4(tk, tv, qr, u, nseq, k, v, fq, fu, partials, len, nsplit, stream); break;
    case 8: e = decode_launch_g8(tk, tv, qr, u, nseq, k, v, fq, fu, partials, len, nsplit, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // the value accumulator is in the value stream's rotated domain: rotate
  // back with the value table's Pi (the query was rotated with the key's)
  hipLaunchKernelGGL(decode_combine_kernel, dim3(B * Hq), dim3(kCombThreads), 0, stream, tv.rot,
                     partials, nsplit, out);
  return hipGetLastError();
}

hipError_t launch_logits_mfma(const tq_tables& tk, const float* qr, const float* u, int B, int Hq,
                              int Hkv, const tq_packed& k, float* logits, hipStream_t stream) {
  if (B == 0 || k.T == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t nseq = static_cast<int64_t>(B) * Hkv;
  const int len = split_length(nseq, k.T, kLogMaxSplit, kLogTarget);
  const int nsplit = static_cast<int>((k.T + len - 1) / len);
  switch (G) {
    case 1: return logits_launch_g1(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 2: return logits_launch_g2(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 4: return logits_launch_g4(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 8: return logits_launch_g8(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    default: return hipErrorInvalidValue;
  }
}

// The wide logits kernel holds its query fragments for two passes in
// registers (about 250 VGPRs: 2 workgroups per CU) and sets up for longer
// than the d = 128 one: one round of the chip, up to 8192 tokens a split.
constexpr int kWideTarget = 2 * kCus;
constexpr int kWideMaxSplit = 8192;

hipError_t launch_logits_wide(const tq_tables& tk, const float* qr, const float* u, int B, int Hq,
                              int Hkv, const tq_packed& k, float* logits, hipStream_t stream) {
  if (B == 0 || k.T == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t nseq = static_cast<int64_t>(B) * Hkv;
  const int len = split_length(nseq, k.T, kWideMaxSplit, kWideTarget);
  const int nsplit = static_cast<int>((k.T + len - 1) / len);
  switch (G) {
    case 1: return logits_wide_launch_g1(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 2: return logits_wide_launch_g2(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 4: return logits_wide_launch_g4(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    case 8: return logits_wide_launch_g8(tk, qr, u, nseq, k, len, nsplit, logits, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
