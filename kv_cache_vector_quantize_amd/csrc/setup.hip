// Setup kernels: the Lloyd-Max codebook and the QR rotation (run once per
// (d, bits) and once per model respectively; float64 throughout).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace tq {

// ---------------------------------------------------------------- codebook
//
// Law of one rotated, normalised coordinate (a2a-mcp.org page, "How it
// works", Stage 1): t = 2u - 1, u ~ Beta((d-1)/2, (d-1)/2), density
// proportional to (1 - t^2)^((d-3)/2) on [-1, 1].
//
// Cell mass: with t = sin(th), dt = cos(th) dth, so the mass of [t0, t1] is
// the integral of cos(th)^(d-2) over [asin t0, asin t1]; that integrand is
// smooth and periodic, so composite Gauss-Legendre converges fast.
// Cell first moment, closed form: the integral of t (1-t^2)^a is
// -(1-t^2)^(a+1) / (2(a+1)), a = (d-3)/2, i.e. g(t) = (1-t^2)^((d-1)/2)
// divided by (d-1).  The normalising constant cancels in the centroid.
//
// One workgroup of 256 threads: thread = (cell, panel).  Lloyd iteration:
// boundaries = midpoints, centroids = mass-weighted cell means, until no
// centroid moves by 1e-15.

constexpr int kGL = 32;          // Gauss-Legendre nodes per panel
constexpr int kCbThreads = 256;

__device__ void gauss_legendre_nodes(double* x, double* w) {
  // Newton iteration on the Legendre polynomial P_n (n = kGL) for the
  // positive roots; nodes and weights on [-1, 1].
  const int i = threadIdx.x;
  if (i < kGL / 2) {
    double z = cos(M_PI * (i + 0.75) / (kGL + 0.5));
    double pp = 1.0;
    for (int it = 0; it < 64; ++it) {
      double p1 = 1.0, p2 = 0.0;
      for (int j = 1; j <= kGL; ++j) {
        double p3 = p2;
        p2 = p1;
        p1 = ((2.0 * j - 1.0) * z * p2 - (j - 1.0) * p3) / j;
      }
      pp = kGL * (z * p1 - p2) / (z * z - 1.0);
      double z1 = z;
      z = z1 - p1 / pp;
      if (fabs(z - z1) <= 1e-16) break;
    }
    // derivative at the converged root for the weight
    double p1 = 1.0, p2 = 0.0;
    for (int j = 1; j <= kGL; ++j) {
      double p3 = p2;
      p2 = p1;
      p1 = ((2.0 * j - 1.0) * z * p2 - (j - 1.0) * p3) / j;
    }
    pp = kGL * (z * p1 - p2) / (z * z - 1.0);
    double wt = 2.0 / ((1.0 - z * z) * pp * pp);
    x[i] = -z;
    x[kGL - 1 - i] = z;
    w[i] = wt;
    w[kGL - 1 - i] = wt;
  }
}

__global__ __launch_bounds__(kCbThreads) void lloyd_max_kernel(int d, int bits, double* c64,
                                                               double* b64, float* c32,
                                                               float* b32) {
  const int L = 1 << bits;
  const int P = kCbThreads / L;  // panels per cell
  const int tid = threadIdx.x;
  __shared__ double gx[kGL], gw[kGL];
  __shared__ double c[16], e[17], part[kCbThreads], moved[16];
  __shared__ int done;

  gauss_legendre_nodes(gx, gw);
  if (tid < L) {
    // any ascending start inside (-1, 1) reaches the unique fixed point
    double span = fmin(0.9, 3.0 / sqrt(static_cast<double>(d)));
    c[tid] = span * (2.0 * (tid + 0.5) / L - 1.0);
  }
  if (tid == 0) done = 0;
  __syncthreads();

  const double pw = static_cast<double>(d - 2);    // exponent in theta
  const double gpw = 0.5 * static_cast<double>(d - 1);
  const int cell = tid / P, panel = tid % P;
  for (int it = 0; it < 200000; ++it) {
    if (tid <= L) {
      e[tid] = (tid == 0) ? -1.0 : (tid == L) ? 1.0 : 0.5 * (c[tid - 1] + c[tid]);
    }
    __syncthreads();
    const double th0 = asin(e[cell]), th1 = asin(e[cell + 1]);
    const double h = (th1 - th0) / P;
    const double a = th0 + panel * h;
    double s = 0.0;
    for (int n = 0; n < kGL; ++n) {
      double th = a + 0.5 * h * (1.0 + gx[n]);
      s += gw[n] * pow(cos(th), pw);
    }
    part[tid] = 0.5 * h * s;
    __syncthreads();
    if (tid < L) {
      double mass = 0.0;
      for (int p = 0; p < P; ++p) mass += part[tid * P + p];
      double t0 = e[tid], t1 = e[tid + 1];
      double g0 = pow(fmax(1.0 - t0 * t0, 0.0), gpw), g1 = pow(fmax(1.0 - t1 * t1, 0.0), gpw);
      double m1 = (g0 - g1) / static_cast<double>(d - 1);
      double cn = m1 / mass;
      moved[tid] = fabs(cn - c[tid]);
      c[tid] = cn;
    }
    __syncthreads();
    if (tid == 0) {
      double mv = 0.0;
      for (int i = 0; i < L; ++i) mv = fmax(mv, moved[i]);
      done = (mv < 1e-15);
    }
    __syncthreads();
    if (done) break;
  }
  if (tid < L) {
    if (c64) c64[tid] = c[tid];
    c32[tid] = static_cast<float>(c[tid]);
    if (tid < L - 1) {
      double b = 0.5 * (c[tid] + c[tid + 1]);
      if (b64) b64[tid] = b;
      b32[tid] = static_cast<float>(b);
    }
  }
}

hipError_t launch_codebook(int d, int bits, double* c64, double* b64, float* c32, float* b32,
                           hipStream_t stream) {
  hipLaunchKernelGGL(lloyd_max_kernel, dim3(1), dim3(kCbThreads), 0, stream, d, bits, c64, b64,
                     c32, b32);
  return hipGetLastError();
}

// ---------------------------------------------------------------- rotation
//
// Householder QR of G (a2a-mcp.org page, Stage 1: the rotation is the Q of
// a Gaussian matrix's QR), then Pi = Q diag(sign(diag R)) so that the factor
// is unique.  One workgroup; the matrix being reduced lives in LDS,
// column-major; thread j owns column j when a reflector is applied.  Q is
// accumulated in the output buffer by applying the reflectors to I in
// reverse order.

constexpr int kRotMax = 128;
constexpr int kRotThreads = 256;
constexpr int kRotGMax = 1024;   // the global-memory factorization (d > kRotMax)

__global__ __launch_bounds__(kRotThreads) void rotation_kernel(int d, const double* __restrict__ G,
                                                               double* __restrict__ Q,
                                                               float* __restrict__ Q32) {
  __shared__ double A[kRotMax][kRotMax + 1];  // A[col][row]
  __shared__ double rdiag[kRotMax];
  __shared__ double red[kRotThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < d * d; i += kRotThreads) A[i % d][i / d] = G[i];
  __syncthreads();

  for (int k = 0; k < d; ++k) {
    double s = 0.0;
    for (int i = k + tid; i < d; i += kRotThreads) s += A[k][i] * A[k][i];
    red[tid] = s;
    __syncthreads();
    for (int o = kRotThreads / 2; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    const double nrm = sqrt(red[0]);
    const double x0 = A[k][k];
    const double alpha = (x0 >= 0.0) ? -nrm : nrm;  // reflect x onto alpha e_1
    const double vn2 = 2.0 * nrm * (nrm + fabs(x0));  // ||x - alpha e_1||^2
    __syncthreads();
    for (int i = k + tid; i < d; i += kRotThreads) {
      double v = (i == k) ? (x0 - alpha) : A[k][i];
      A[k][i] = (vn2 > 0.0) ? v / sqrt(vn2) : 0.0;  // zero column: H = I
    }
    if (tid == 0) rdiag[k] = (vn2 > 0.0) ? alpha : 0.0;
    __syncthreads();
    for (int j = k + 1 + tid; j < d; j += kRotThreads) {
      double w = 0.0;
      for (int i = k; i < d; ++i) w += A[k][i] * A[j][i];
      w *= 2.0;
      for (int i = k; i < d; ++i) A[j][i] -= w * A[k][i];
    }
    __syncthreads();
  }

  for (int c = tid; c < d; c += kRotThreads) {
    for (int r = 0; r < d; ++r) Q[r * d + c] = (r == c) ? 1.0 : 0.0;
    for (int k = d - 1; k >= 0; --k) {
      double w = 0.0;
      for (int i = k; i < d; ++i) w += A[k][i] * Q[i * d + c];
      w *= 2.0;
      for (int i = k; i < d; ++i) Q[i * d + c] -= w * A[k][i];
    }
    const double sg = (rdiag[c] < 0.0) ? -1.0 : 1.0;
    for (int r = 0; r < d; ++r) {
      double v = Q[r * d + c] * sg;
      Q[r * d + c] = v;
      if (Q32) Q32[r * d + c] = static_cast<float>(v);
    }
  }
}

// The same factorization for head dimensions past what LDS holds: one
// workgroup works in global memory (the output buffer, L2-resident), with the
// matrix column-major, A[c * d + r].  The reflectors are reduced in place;
// then Q is formed in place over them, last reflector first: when reflector
// i is applied to columns i+1.. (rows i..), those columns already hold Q's
// trailing block and the reflectors stored there are spent, and column i is
// then replaced by H_i e_i (zeros above row i).  Finally the sign fix, the
// transpose to row-major and the float32 copy.
constexpr int kRotGThreads = 1024;

__global__ __launch_bounds__(kRotGThreads) void rotation_global_kernel(int d, const double* __restrict__ G,
                                                                       double* __restrict__ A,
                                                                       float* __restrict__ Q32) {
  __shared__ double rdiag[kRotGMax];
  __shared__ double red[kRotGThreads];
  const int tid = threadIdx.x;
  for (int e = tid; e < d * d; e += kRotGThreads) A[(e % d) * d + e / d] = G[e];   // column-major copy
  __syncthreads();
  for (int k = 0; k < d; ++k) {
    double* ak = A + static_cast<int64_t>(k) * d;
    double s = 0.0;
    for (int i = k + tid; i < d; i += kRotGThreads) s += ak[i] * ak[i];
    red[tid] = s;
    __syncthreads();
    for (int o = kRotGThreads / 2; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    const double nrm = sqrt(red[0]);
    const double x0 = ak[k];
    const double alpha = (x0 >= 0.0) ? -nrm : nrm;
    const double vn2 = 2.0 * nrm * (nrm + fabs(x0));
    __syncthreads();
    for (int i = k + tid; i < d; i += kRotGThreads) {
      const double v = (i == k) ? (x0 - alpha) : ak[i];
      ak[i] = (vn2 > 0.0) ? v / sqrt(vn2) : 0.0;
    }
    if (tid == 0) rdiag[k] = (vn2 > 0.0) ? alpha : 0.0;
    __syncthreads();
    for (int j = k + 1 + tid; j < d; j += kRotGThreads) {
      double* aj = A + static_cast<int64_t>(j) * d;
      double w = 0.0;
      for (int i = k; i < d; ++i) w += ak[i] * aj[i];
      w *= 2.0;
      for (int i = k; i < d; ++i) aj[i] -= w * ak[i];
    }
    __syncthreads();
  }
  // Q = H_0 H_1 ... H_{d-1} I, formed in place
  for (int i = d - 1; i >= 0; --i) {
    const double* vi = A + static_cast<int64_t>(i) * d;   // reflector i, rows i..d-1
    for (int c = i + 1 + tid; c < d; c += kRotGThreads) {
      double* qc = A + static_cast<int64_t>(c) * d;
      double w = 0.0;
      for (int r = i; r < d; ++r) w += vi[r] * qc[r];
      w *= 2.0;
      for (int r = i; r < d; ++r) qc[r] -= w * vi[r];
    }
    __syncthreads();
    const double a = vi[i];
    __syncthreads();
    double* qi = A + static_cast<int64_t>(i) * d;
    for (int r = tid; r < d; r += kRotGThreads)
      qi[r] = (r < i) ? 0.0 : (r == i ? 1.0 - 2.0 * a * a : -2.0 * a * qi[r]);
    __syncthreads();
  }
  // Pi = Q diag(sign(diag R)), transposed in place to row-major
  for (int e = tid; e < d * d; e += kRotGThreads) {
    if (rdiag[e / d] < 0.0) A[e] = -A[e];
  }
  __syncthreads();
  for (int e = tid; e < d * d; e += kRotGThreads) {
    const int c = e / d, r = e % d;
    if (r < c) {
      const double t = A[e];
      A[e] = A[r * d + c];
      A[r * d + c] = t;
    }
  }
  __syncthreads();
  if (Q32)
    for (int e = tid; e < d * d; e += kRotGThreads) Q32[e] = static_cast<float>(A[e]);
}

hipError_t launch_rotation(int d, const double* G, double* Q, float* Q32, hipStream_t stream) {
  if (d <= kRotMax) hipLaunchKernelGGL(rotation_kernel, dim3(1), dim3(kRotThreads), 0, stream, d, G, Q, Q32);
  else hipLaunchKernelGGL(rotation_global_kernel, dim3(1), dim3(kRotGThreads), 0, stream, d, G, Q, Q32);
  return hipGetLastError();
}

// Randomized Walsh-Hadamard rotation (qiita page, "What you hit when you try
// it"): entry (j, k) = (-1)^popcount(j & k) * s_k / sqrt(d), one thread per
// entry; 1/sqrt(d) in float64, then rounded once to float32.
__global__ void hadamard_rotation_kernel(int d, const float* __restrict__ signs, float* __restrict__ rot) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= static_cast<int64_t>(d) * d) return;
  const int j = static_cast<int>(e / d), k = static_cast<int>(e % d);
  const bool neg = (__popc(static_cast<unsigned>(j & k)) & 1) != (signbit(signs[k]) != 0);
  const double v = 1.0 / sqrt(static_cast<double>(d));
  rot[e] = static_cast<float>(neg ? -v : v);
}

hipError_t launch_hadamard_rotation(int d, const float* signs, float* rot32, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(d) * d;
  hipLaunchKernelGGL(hadamard_rotation_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     stream, d, signs, rot32);
  return hipGetLastError();
}

}  // namespace tq
