// extern "C" entry points of libtq.so: validate on the host, size the
// workspaces, then hand over to the launchers.  See include/tq.h for the
// contract of every call.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/tq.h"
#include "launch.h"

namespace {

constexpr int kSupportedD = 128;   // the matrix-core kernels
constexpr int kSupportedM = 128;
constexpr int kGenericMinD = 8, kGenericMax = 256;   // the vector-ALU kernels (generic.hip)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }


tq_status from_hip(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_EHIP; }

size_t align256(size_t x) { return (x + 255u) & ~static_cast<size_t>(255u); }

// Tables of a stream as the hot-path kernels need them.
tq_status check_tables(const tq_tables* t, bool key) {
  if (t == nullptr) return TQ_EINVAL;
  if (t->rot_kind != TQ_ROT_DENSE && t->rot_kind != TQ_ROT_HADAMARD) return TQ_EINVAL;
  if (t->bits < 1 || t->bits > 4 || t->d < 2) return TQ_EINVAL;
  if (t->m < 0) return TQ_EINVAL;
  if (key ? t->m == 0 : t->m != 0) return TQ_EINVAL;
  if (!ok_ptr(t->rot) || !ok_ptr(t->centroids) || !ok_ptr(t->bounds)) return TQ_EINVAL;
  if (key ? !ok_ptr(t->sketch) : t->sketch != nullptr) return TQ_EINVAL;
  if (t->sketch_f16 != 0 && (t->sketch_f16 != 1 || !key)) return TQ_EINVAL;
  // split (fractional) widths: the leading hi_coords coordinates at bits + 1
  if (t->hi_coords < 0 || t->hi_coords > t->d || t->hi_coords % 32 != 0) return TQ_EINVAL;
  if (t->hi_coords > 0) {
    if (t->bits > 3 || !ok_ptr(t->centroids_hi) || !ok_ptr(t->bounds_hi)) return TQ_EINVAL;
  } else if (t->centroids_hi != nullptr || t->bounds_hi != nullptr) {
    return TQ_EINVAL;
  }
  const bool mfma = t->d == kSupportedD && (key ? t->m == kSupportedM : true);
  if (!mfma) {   // the generic kernels: any d and m up to 256, no split widths
    if (t->d < kGenericMinD || t->d > kGenericMax || t->m > kGenericMax || t->hi_coords != 0)
      return TQ_EUNSUPPORTED;
  }
  if (t->hi_coords != 0 && t->hi_coords != t->d / 2) return TQ_EUNSUPPORTED;
  return TQ_OK;
}

bool split(const tq_tables* t) { return t->hi_coords != 0; }

// head dimension / sketch size of the vector-ALU kernels (not the 128 of the
// matrix-core ones)
bool generic(const tq_tables* t) { return !(t->d == kSupportedD && (t->m == kSupportedM || t->m == 0)); }

tq_status check_packed(const tq_packed* p, const tq_tables* t, int role) {
  if (p == nullptr) return TQ_EINVAL;
  if (p->role != role) return TQ_EINVAL;
  if (p->capacity < 0 || p->capacity % 32 != 0 || (p->capacity != 0 && p->capacity < p->T)) return TQ_EINVAL;
  if (p->bits != t->bits || p->d != t->d || p->m != t->m || p->hi_coords != t->hi_coords)
    return TQ_EINVAL;
  if (p->nseq < 0 || p->T < 0) return TQ_EINVAL;
  if (p->norm_dtype != TQ_F32 && p->norm_dtype != TQ_F16) return TQ_EINVAL;
  const bool empty = p->nseq == 0 || p->T == 0;
  if (!empty && (!ok_ptr(p->codes) || !ok_ptr(p->norm))) return TQ_EINVAL;
  if (empty && (!ok_opt(p->codes) || !ok_opt(p->norm))) return TQ_EINVAL;
  if (role == TQ_KEY) {
    if (!empty && (!ok_ptr(p->signs) || !ok_ptr(p->rnorm))) return TQ_EINVAL;
    if (empty && (!ok_opt(p->signs) || !ok_opt(p->rnorm))) return TQ_EINVAL;
  } else if (p->signs != nullptr || p->rnorm != nullptr) {
    return TQ_EINVAL;
  }
  return TQ_OK;
}

// The array behind tq_attn_decode_static: decode's workspace for callers
// that cannot allocate.  Every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as a
// device address: device_scratch() takes the address of the current
// device's copy from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = static_cast<size_t>(16) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

tq_status device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TQ_EHIP;
  if (dev >= kMaxDevices) return TQ_EUNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return TQ_EHIP;
  *ptr = g_scratch_ptr[dev];
  return TQ_OK;
}

tq_status decode_args(const tq_tables* tk, const tq_tables* tv, const void* q, int q_dtype, int B,
                      int Hq, int Hkv, const tq_packed* k, const tq_packed* v, float scale,
                      const float* out);
tq_status decode_checked(const tq_tables* tk, const tq_tables* tv, const void* q, int q_dtype,
                         int B, int Hq, int Hkv, const tq_packed* k, const tq_packed* v,
                         float scale, float* out, void* ws, size_t ws_bytes, hipStream_t stream);

tq_status check_heads(int B, int Hq, int Hkv, int max_group) {
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return TQ_EINVAL;
  const int G = Hq / Hkv;
  if (G > max_group || (G & (G - 1)) != 0) return TQ_EUNSUPPORTED;
  return TQ_OK;
}

}  // namespace

extern "C" {

int tq_abi_version(void) { return TQ_ABI_VERSION; }

const char* tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "TQ_OK";
    case TQ_EINVAL: return "TQ_EINVAL: invalid argument";
    case TQ_EUNSUPPORTED: return "TQ_EUNSUPPORTED: shape or width not supported by the kernels";
    case TQ_EWORKSPACE: return "TQ_EWORKSPACE: workspace too small";
    case TQ_EHIP: return "TQ_EHIP: HIP launch or runtime error";
    default: return "unknown tq_status";
  }
}

tq_status tq_codebook(int d, int bits, double* centroids64, double* bounds64, float* centroids32,
                      float* bounds32, hipStream_t stream) {
  if (d < 3 || d > 4096 || bits < 1 || bits > 4) return TQ_EINVAL;
  if (!ok_ptr(centroids32) || !ok_ptr(bounds32) || !ok_opt(centroids64) || !ok_opt(bounds64))
    return TQ_EINVAL;
  return from_hip(tq::launch_codebook(d, bits, centroids64, bounds64, centroids32, bounds32, stream));
}

tq_status tq_rotation(int d, const double* G, double* rot64, float* rot32, hipStream_t stream) {
  if (d < 2 || d > 1024 || !ok_ptr(G) || !ok_ptr(rot64) || !ok_opt(rot32)) return TQ_EINVAL;
  return from_hip(tq::launch_rotation(d, G, rot64, rot32, stream));
}

tq_status tq_hadamard_rotation(int d, const float* signs, float* rot32, hipStream_t stream) {
  if (d < 2 || d > 4096 || (d & (d - 1)) != 0 || !ok_ptr(signs) || !ok_ptr(rot32)) return TQ_EINVAL;
  return from_hip(tq::launch_hadamard_rotation(d, signs, rot32, stream));
}

tq_status tq_quantize(const tq_tables* t, const void* x, int x_dtype, const tq_packed* out,
                      hipStream_t stream) {
  if (t == nullptr || out == nullptr) return TQ_EINVAL;
  const bool key = out->role == TQ_KEY;
  if (out->role != TQ_KEY && out->role != TQ_VALUE) return TQ_EINVAL;
  tq_status st = check_tables(t, key);
  if (st != TQ_OK) return st;
  st = check_packed(out, t, out->role);
  if (st != TQ_OK) return st;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_EINVAL;
  if (split(t) && t->rot_kind != TQ_ROT_DENSE) return TQ_EUNSUPPORTED;
  if (out->nseq == 0 || out->T == 0) return TQ_OK;
  if (!ok_ptr(x)) return TQ_EINVAL;
  if (generic(t)) return from_hip(tq::launch_quantize_generic(*t, x, x_dtype, *out, stream));
  return from_hip(tq::launch_quantize(*t, x, x_dtype, *out, 0, out->T, false, stream));
}

tq_status tq_append(const tq_tables* t, const void* x, int x_dtype, int64_t n, const tq_packed* out,
                    hipStream_t stream) {
  if (t == nullptr || out == nullptr) return TQ_EINVAL;
  const bool key = out->role == TQ_KEY;
  if (out->role != TQ_KEY && out->role != TQ_VALUE) return TQ_EINVAL;
  tq_status st = check_tables(t, key);
  if (st != TQ_OK) return st;
  st = check_packed(out, t, out->role);
  if (st != TQ_OK) return st;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_EINVAL;
  if (split(t) && t->rot_kind != TQ_ROT_DENSE) return TQ_EUNSUPPORTED;
  if (generic(t)) return TQ_EUNSUPPORTED;   // appends run on the d = 128 kernels
  // the new tokens must fit the stream's storage
  if (n < 0 || out->capacity == 0 || n > out->capacity - out->T) return TQ_EINVAL;
  if (out->nseq == 0 || n == 0) return TQ_OK;
  if (!ok_ptr(x)) return TQ_EINVAL;
  return from_hip(tq::launch_quantize(*t, x, x_dtype, *out, out->T, n, true, stream));
}

size_t tq_logits_workspace(int B, int Hq, int d, int m) {
  if (B < 0 || Hq < 0 || d < 0 || m < 0) return 0;
  const size_t nh = static_cast<size_t>(B) * Hq;
  return align256(nh * d * sizeof(float)) + align256(nh * m * sizeof(float));
}

tq_status tq_attn_logits(const tq_tables* tk, const void* q, int q_dtype, int B, int Hq, int Hkv,
                         const tq_packed* k, float* logits, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  tq_status st = check_tables(tk, true);
  if (st != TQ_OK) return st;
  st = check_packed(k, tk, TQ_KEY);
  if (st != TQ_OK) return st;
  st = check_heads(B, Hq, Hkv, 16);
  if (st != TQ_OK) return st;
  if (k->nseq != static_cast<int64_t>(B) * Hkv) return TQ_EINVAL;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_EINVAL;
  if (k->nseq > 65535) return TQ_EUNSUPPORTED;  // one grid row per sequence
  // split keys: 2.5 / 3.5 bits on the matrix-core tiles
  if (split(tk) && (tk->bits < 2 || Hq / Hkv > 8)) return TQ_EUNSUPPORTED;
  if (B == 0 || k->T == 0) return TQ_OK;
  if (!ok_ptr(q) || !ok_ptr(logits) || !ok_ptr(ws)) return TQ_EINVAL;
  if (ws_bytes < tq_logits_workspace(B, Hq, tk->d, tk->m)) return TQ_EWORKSPACE;
  if (k->T >= (static_cast<int64_t>(1) << 28)) return TQ_EUNSUPPORTED;  // 32-bit record offsets
  float* qr = static_cast<float*>(ws);
  float* u = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                      align256(static_cast<size_t>(B) * Hq * tk->d * sizeof(float)));
  if (generic(tk)) {
    if (tq::launch_qprep_generic(*tk, q, q_dtype, B * Hq, qr, u, stream) != hipSuccess) return TQ_EHIP;
    // matrix-core tiles up to 8 heads per KV head; 16 take the vector-ALU kernel
    if (Hq / Hkv <= 8 && tk->m > 0 && !split(tk))
      return from_hip(tq::launch_logits_wide(*tk, qr, u, B, Hq, Hkv, *k, logits, stream));
    return from_hip(tq::launch_logits_generic(*tk, qr, u, B, Hq, Hkv, *k, logits, stream));
  }
  hipError_t e = tq::launch_qprep(*tk, q, q_dtype, B * Hq, qr, u, stream);
  if (e != hipSuccess) return TQ_EHIP;
  if (Hq / Hkv <= 8)  // matrix-core tiles; 16 heads per KV head take the vector-ALU kernel
    return from_hip(tq::launch_logits_mfma(*tk, qr, u, B, Hq, Hkv, *k, logits, stream));
  return from_hip(tq::launch_logits(*tk, qr, u, B, Hq, Hkv, *k, logits, stream));
}

size_t tq_decode_workspace(int B, int Hq, int Hkv, int64_t T, int d, int m) {
  if (B < 0 || Hq < 0 || Hkv < 1 || T < 0 || d < 0 || m < 0) return 0;
  return tq::decode_workspace_layout(B, Hq, Hkv, T, d, m).total;
}

tq_status tq_attn_decode(const tq_tables* tk, const tq_tables* tv, const void* q, int q_dtype,
                         int B, int Hq, int Hkv, const tq_packed* k, const tq_packed* v,
                         float scale, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_checked(tk, tv, q, q_dtype, B, Hq, Hkv, k, v, scale, out, ws, ws_bytes, stream);
}

size_t tq_attn_decode_static_capacity(void) { return kScratchBytes; }

tq_status tq_attn_decode_static(const tq_tables* tk, const tq_tables* tv, const void* q, int q_dtype,
                                int B, int Hq, int Hkv, const tq_packed* k, const tq_packed* v,
                                float scale, float* out, hipStream_t stream) {
  // arguments first, then the workspace the shape needs against the array,
  // then the current device's copy of the array
  tq_status st = decode_args(tk, tv, q, q_dtype, B, Hq, Hkv, k, v, scale, out);
  if (st != TQ_OK || B == 0) return st;
  if (tq_decode_workspace(B, Hq, Hkv, k->T, tk->d, tk->m) > kScratchBytes) return TQ_EWORKSPACE;
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st != TQ_OK) return st;
  return decode_checked(tk, tv, q, q_dtype, B, Hq, Hkv, k, v, scale, out, ws, kScratchBytes, stream);
}

}  // extern "C"

namespace {

// Every argument of a decode call but the workspace.
tq_status decode_args(const tq_tables* tk, const tq_tables* tv, const void* q, int q_dtype, int B,
                      int Hq, int Hkv, const tq_packed* k, const tq_packed* v, float scale,
                      const float* out) {
  // keys and values may use different rotations (of either kind): queries are
  // rotated with the key table's Pi, the output rotated back with the value
  // table's; both tables hold Pi densely.  The head dimensions must agree.
  if (tk == nullptr || tv == nullptr || tv->d != tk->d) return TQ_EINVAL;
  tq_status st = check_tables(tk, true);
  if (st != TQ_OK) return st;
  st = check_tables(tv, false);
  if (st != TQ_OK) return st;
  st = check_packed(k, tk, TQ_KEY);
  if (st != TQ_OK) return st;
  st = check_packed(v, tv, TQ_VALUE);
  if (st != TQ_OK) return st;
  st = check_heads(B, Hq, Hkv, 8);
  if (st != TQ_OK) return st;
  if (k->nseq != static_cast<int64_t>(B) * Hkv || v->nseq != k->nseq || v->T != k->T)
    return TQ_EINVAL;
  if (k->T < 1 && B > 0) return TQ_EINVAL;
  if (k->nseq > 65535) return TQ_EUNSUPPORTED;  // one grid row per sequence
  if (k->T >= (static_cast<int64_t>(1) << 28)) return TQ_EUNSUPPORTED;  // 32-bit record offsets
  if (generic(tk) || generic(tv)) return TQ_EUNSUPPORTED;   // decode runs at d = 128
  // split streams: both split, bits 2 or 3 each, float16 norms
  if (split(tk) || split(tv)) {
    if (!split(tk) || !split(tv) || tk->bits < 2 || tv->bits < 2 || k->norm_dtype != TQ_F16 ||
        v->norm_dtype != TQ_F16)
      return TQ_EUNSUPPORTED;
  }
  if (!(scale > 0.0f) || !isfinite(scale)) return TQ_EINVAL;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_EINVAL;
  if (B == 0) return TQ_OK;
  if (!ok_ptr(q) || !ok_ptr(out)) return TQ_EINVAL;
  return TQ_OK;
}

tq_status decode_checked(const tq_tables* tk, const tq_tables* tv, const void* q, int q_dtype,
                         int B, int Hq, int Hkv, const tq_packed* k, const tq_packed* v,
                         float scale, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const tq_status st = decode_args(tk, tv, q, q_dtype, B, Hq, Hkv, k, v, scale, out);
  if (st != TQ_OK || B == 0) return st;
  if (!ok_ptr(ws)) return TQ_EINVAL;
  const tq::DecodeWorkspace lay = tq::decode_workspace_layout(B, Hq, Hkv, k->T, tk->d, tk->m);
  if (ws_bytes < lay.total) return TQ_EWORKSPACE;
  char* base = static_cast<char*>(ws);
  float* qr = reinterpret_cast<float*>(base + lay.qr);
  float* u = reinterpret_cast<float*>(base + lay.u);
  hipError_t e = tq::launch_qprep(*tk, q, q_dtype, B * Hq, qr, u, stream);
  if (e != hipSuccess) return TQ_EHIP;
  return from_hip(tq::launch_decode(*tk, *tv, qr, u, B, Hq, Hkv, *k, *v, scale, ws, lay, out, stream));
}

}  // namespace

extern "C" {

size_t tq_topk_workspace(int64_t rows, int64_t n, int k) {
  if (rows < 0 || rows > 65535 || n < 1 || n > INT32_MAX || k < 1 || k > 32 || k > n) return 0;
  return tq::topk_workspace(rows, n, k);
}

tq_status tq_topk(const float* scores, int64_t rows, int64_t n, int k, int32_t* idx, float* val, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  if (rows < 0 || n < 1 || n > INT32_MAX || k < 1 || k > 32 || k > n) return TQ_EINVAL;
  if (rows > 65535) return TQ_EUNSUPPORTED;  // one grid row per score row
  if (rows == 0) return TQ_OK;
  if (!ok_ptr(scores) || !ok_ptr(idx) || !ok_ptr(val) || !ok_ptr(ws)) return TQ_EINVAL;
  if (ws_bytes < tq::topk_workspace(rows, n, k)) return TQ_EWORKSPACE;
  return from_hip(tq::launch_topk(scores, rows, n, k, idx, val, ws, stream));
}

}  // extern "C"
