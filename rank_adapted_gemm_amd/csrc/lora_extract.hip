// Adapter extraction: rank-r factors (B, A) of the change W_adapted - W_base.
//
// "two 27B models on a single RTX 5090", TL;DR: the adapted model's weights
// differ from the base model's by a merged rank-256 change, which factors back
// out into an adapter.  The pages do not give the method; this computes the
// truncated singular value decomposition of the change D = U S V^T, with
// B = U_r S_r^(1/2) and A = S_r^(1/2) V_r^T, by the randomized range finder
// with power iterations and a direct SVD of the small projected matrix (Halko,
// Martinsson and Tropp, "Finding structure with randomness", 2011, sections
// 4.3-4.5 and 5.1):
//
//   1. D = W_adapted - W_base                                (fp32, N x K)
//   2. Y = D Omega, Q = orth(Y)                              (Omega: the caller's K x l Gaussian draws)
//   3. q times: Q' = orth(D^T Q), Q = orth(D Q')             (power iterations)
//   4. Bm = Q^T D                                            (l x K)
//   5. C = Bm Bm^T = W L W^T                                 (fp64 symmetric eigenproblem, l x l)
//   6. s_i = sqrt(L_i) for the r largest L_i; B = Q W_r S_r^(1/2), A = S_r^(-1/2) W_r^T Bm
//
// B A = Q W_r W_r^T Q^T D, the projection of D onto its top-r left singular
// subspace as seen through Q: the truncated SVD of D whenever Q captures D's
// top-r range, which the power iterations make exact to rounding for a change
// with a gap after its r-th singular value.
//
// The products run on a tiled GEMM of arbitrary strides (LDS staging, 4 x 4
// outputs per thread).  orth() is a Householder QR with the thin Q formed
// explicitly, and step 5 a cyclic Jacobi eigensolver with the round-robin
// pairing, both in fp64 and each in one workgroup: they work on l-wide
// matrices (l = r + oversampling, a few hundred) and take milliseconds.
// Extraction runs once per weight matrix, outside the serving path.
#include <algorithm>
#include <cmath>

#include "lora_internal.h"

namespace lora {
namespace {

constexpr int GT = 64;     // GEMM tile edge
constexpr int GK = 16;     // GEMM K slab

__global__ __launch_bounds__(256) void diff_kernel(const __bf16* __restrict__ a, const __bf16* __restrict__ b,
                                                   float* __restrict__ d, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    d[i] = float(a[i]) - float(b[i]);
}

// C[m][n] = sum_k A(m, k) B(k, n), A(m, k) = a[m sam + k sak], B(k, n) = b[k sbk + n sbn],
// C row-major (ldc), accumulated in TACC.
template <typename TA, typename TB, typename TACC, typename TC>
__global__ __launch_bounds__(256) void gemm_kernel(const TA* __restrict__ a, int64_t sam, int64_t sak,
                                                   const TB* __restrict__ b, int64_t sbk, int64_t sbn,
                                                   TC* __restrict__ c, int64_t ldc, int M, int N, int K) {
  __shared__ TACC as[GK][GT + 1], bs[GK][GT + 1];
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  TACC acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += GK) {
    for (int e = tid; e < GK * GT; e += 256) {
      const int kk = e / GT, mm = e % GT;
      const int m = m0 + mm, k = k0 + kk;
      as[kk][mm] = (m < M && k < K) ? TACC(a[int64_t(m) * sam + int64_t(k) * sak]) : TACC(0);
      const int n = n0 + mm;
      bs[kk][mm] = (n < N && k < K) ? TACC(b[int64_t(k) * sbk + int64_t(n) * sbn]) : TACC(0);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; ++kk) {
      TACC x[4], y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += x[i] * y[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) c[int64_t(m) * ldc + n] = TC(acc[i][j]);
    }
}

__device__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// Thin Q of the Householder QR of Y (m x l, row-major fp32), written over Y.
// V: m x l fp64 work (the reflectors), Qw: m x l fp64 work.  One workgroup.
__global__ __launch_bounds__(256) void householder_q_kernel(float* __restrict__ y, double* __restrict__ v,
                                                            double* __restrict__ qw, double* __restrict__ beta,
                                                            int m, int l) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  for (int64_t e = tid; e < int64_t(m) * l; e += 256) v[e] = double(y[e]);
  __syncthreads();
  for (int j = 0; j < l; ++j) {
    double part = 0;
    for (int i = j + tid; i < m; i += 256) part += v[int64_t(i) * l + j] * v[int64_t(i) * l + j];
    const double nrm2 = block_sum(part, red);
    const double alpha = v[int64_t(j) * l + j];
    const double nrm = sqrt(nrm2);
    // reflector v = x - s e_1 with s = -sign(alpha) |x|, beta = 2 / |v|^2
    const double sgn = alpha >= 0 ? -nrm : nrm;
    const double vn2 = nrm2 - alpha * alpha + (alpha - sgn) * (alpha - sgn);
    const double bj = (nrm2 > 0 && vn2 > 0) ? 2.0 / vn2 : 0.0;
    __syncthreads();
    if (tid == 0) {
      v[int64_t(j) * l + j] = alpha - sgn;
      beta[j] = bj;
    }
    __syncthreads();
    // columns c > j: x_c -= beta (v . x_c) v
    for (int c = j + 1 + tid; c < l; c += 256) {
      double w = 0;
      for (int i = j; i < m; ++i) w += v[int64_t(i) * l + j] * v[int64_t(i) * l + c];
      w *= bj;
      for (int i = j; i < m; ++i) v[int64_t(i) * l + c] -= w * v[int64_t(i) * l + j];
    }
    __syncthreads();
  }
  // Q = H_0 H_1 ... H_{l-1} [I; 0]: apply the reflectors in reverse; H_j leaves
  // columns c < j alone (they are zero in rows >= j)
  for (int64_t e = tid; e < int64_t(m) * l; e += 256) {
    const int64_t i = e / l, c = e % l;
    qw[e] = i == c ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int j = l - 1; j >= 0; --j) {
    const double bj = beta[j];
    for (int c = j + tid; c < l; c += 256) {
      double w = 0;
      for (int i = j; i < m; ++i) w += v[int64_t(i) * l + j] * qw[int64_t(i) * l + c];
      w *= bj;
      for (int i = j; i < m; ++i) qw[int64_t(i) * l + c] -= w * v[int64_t(i) * l + j];
    }
    __syncthreads();
  }
  for (int64_t e = tid; e < int64_t(m) * l; e += 256) y[e] = float(qw[e]);
}

// Eigenpairs of the symmetric l x l matrix C (fp64, overwritten): cyclic Jacobi
// with the round-robin pairing, so each round rotates l/2 disjoint (p, q)
// pairs at once (Golub and Van Loan, "Matrix Computations", 8.5).  Leaves the
// eigenvalues on C's diagonal and the eigenvectors in the columns of U.  l is
// even.  Stops when the off-diagonal mass is below tol^2 of the total.
__global__ __launch_bounds__(256) void jacobi_kernel(double* __restrict__ cm, double* __restrict__ u, int l,
                                                     int max_sweeps, double tol) {
  __shared__ double red[256];
  __shared__ double cs[256], sn[256];
  __shared__ int pp[256], qq[256];
  const int tid = threadIdx.x;
  for (int64_t e = tid; e < int64_t(l) * l; e += 256) u[e] = (e / l == e % l) ? 1.0 : 0.0;
  __syncthreads();
  const int half = l / 2;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    double off = 0, tot = 0;
    for (int64_t e = tid; e < int64_t(l) * l; e += 256) {
      const double x = cm[e] * cm[e];
      tot += x;
      if (e / l != e % l) off += x;
    }
    off = block_sum(off, red);
    tot = block_sum(tot, red);
    if (off <= tol * tol * tot) break;
    for (int round = 0; round < l - 1; ++round) {
      // pairing of round `round`: (round, l-1) and ((round + k) mod (l-1), (round - k) mod (l-1))
      for (int k = tid; k < half; k += 256) {
        int p, q;
        if (k == 0) {
          p = round;
          q = l - 1;
        } else {
          p = (round + k) % (l - 1);
          q = (round - k + (l - 1)) % (l - 1);
        }
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        const double apq = cm[int64_t(p) * l + q];
        double c = 1, s = 0;
        if (apq != 0) {
          const double tau = (cm[int64_t(q) * l + q] - cm[int64_t(p) * l + p]) / (2 * apq);
          const double t = tau >= 0 ? 1.0 / (tau + sqrt(1 + tau * tau)) : -1.0 / (-tau + sqrt(1 + tau * tau));
          c = 1.0 / sqrt(1 + t * t);
          s = t * c;
        }
        pp[k] = p;
        qq[k] = q;
        cs[k] = c;
        sn[k] = s;
      }
      __syncthreads();
      // rows: C <- J^T C
      for (int64_t e = tid; e < int64_t(half) * l; e += 256) {
        const int k = int(e / l), j = int(e % l);
        const int p = pp[k], q = qq[k];
        const double c = cs[k], s = sn[k];
        const double xp = cm[int64_t(p) * l + j], xq = cm[int64_t(q) * l + j];
        cm[int64_t(p) * l + j] = c * xp - s * xq;
        cm[int64_t(q) * l + j] = s * xp + c * xq;
      }
      __syncthreads();
      // columns: C <- C J, U <- U J
      for (int64_t e = tid; e < int64_t(half) * l; e += 256) {
        const int k = int(e / l), i = int(e % l);
        const int p = pp[k], q = qq[k];
        const double c = cs[k], s = sn[k];
        const double xp = cm[int64_t(i) * l + p], xq = cm[int64_t(i) * l + q];
        cm[int64_t(i) * l + p] = c * xp - s * xq;
        cm[int64_t(i) * l + q] = s * xp + c * xq;
        const double up = u[int64_t(i) * l + p], uq = u[int64_t(i) * l + q];
        u[int64_t(i) * l + p] = c * up - s * uq;
        u[int64_t(i) * l + q] = s * up + c * uq;
      }
      __syncthreads();
    }
  }
}

// From the eigenpairs: order by eigenvalue (largest first), s_i = sqrt(L_i);
// G1 = W_r S^(1/2) (l x r), G2 = S^(-1/2) W_r^T (r x l), sigma = s_r.  One workgroup.
__global__ __launch_bounds__(256) void assemble_kernel(const double* __restrict__ cm, const double* __restrict__ u,
                                                       int l, int r, float* __restrict__ g1, float* __restrict__ g2,
                                                       float* __restrict__ sigma) {
  __shared__ int order[1024];
  __shared__ double sv[1024];
  const int tid = threadIdx.x;
  if (tid == 0) {
    for (int i = 0; i < l; ++i) order[i] = i;
    for (int i = 0; i < r; ++i) {            // selection of the r largest, in order
      int best = i;
      for (int j = i + 1; j < l; ++j)
        if (cm[int64_t(order[j]) * l + order[j]] > cm[int64_t(order[best]) * l + order[best]]) best = j;
      const int t = order[i];
      order[i] = order[best];
      order[best] = t;
      const double lam = cm[int64_t(order[i]) * l + order[i]];
      sv[i] = lam > 0 ? sqrt(lam) : 0.0;
    }
  }
  __syncthreads();
  for (int e = tid; e < l * r; e += 256) {
    const int i = e / r, j = e % r;
    const double w = u[int64_t(i) * l + order[j]];
    const double root = sqrt(sv[j]);
    g1[int64_t(i) * r + j] = float(w * root);
    g2[int64_t(j) * l + i] = root > 0 ? float(w / root) : 0.0f;
  }
  for (int j = tid; j < r; j += 256) sigma[j] = float(sv[j]);
}

template <typename TA, typename TB, typename TACC, typename TC>
hipError_t gemm(const TA* a, int64_t sam, int64_t sak, const TB* b, int64_t sbk, int64_t sbn, TC* c, int64_t ldc,
                int M, int N, int K, hipStream_t s) {
  const dim3 grid(unsigned((N + GT - 1) / GT), unsigned((M + GT - 1) / GT));
  hipLaunchKernelGGL((gemm_kernel<TA, TB, TACC, TC>), grid, dim3(256), 0, s, a, sam, sak, b, sbk, sbn, c, ldc, M, N,
                     K);
  return hipGetLastError();
}

size_t r256(size_t x) { return (x + 255) & ~size_t(255); }

struct ExtractLayout {
  size_t d, y, z, v, qw, beta, bm, cm, u, g1, g2, total;
};

ExtractLayout extract_layout(int64_t N, int64_t K, int64_t l, int64_t r) {
  ExtractLayout o;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += r256(bytes); return at; };
  const int64_t mx = std::max(N, K);
  o.d = take(size_t(N) * K * 4);
  o.y = take(size_t(N) * l * 4);
  o.z = take(size_t(K) * l * 4);
  o.v = take(size_t(mx) * l * 8);
  o.qw = take(size_t(mx) * l * 8);
  o.beta = take(size_t(l) * 8);
  o.bm = take(size_t(l) * K * 4);
  o.cm = take(size_t(l) * l * 8);
  o.u = take(size_t(l) * l * 8);
  o.g1 = take(size_t(l) * r * 4);
  o.g2 = take(size_t(r) * l * 4);
  o.total = off;
  return o;
}

}  // namespace

size_t extract_workspace_bytes(int64_t N, int64_t K, int64_t l, int64_t r) { return extract_layout(N, K, l, r).total; }

hipError_t launch_extract(const void* w_adapted, const void* w_base, int64_t N, int64_t K, const float* omega,
                          int l, int r, int power_iters, float* b_out, float* a_out, float* sigma_out,
                          void* workspace, hipStream_t s) {
  const ExtractLayout o = extract_layout(N, K, l, r);
  char* ws = static_cast<char*>(workspace);
  float* d = reinterpret_cast<float*>(ws + o.d);
  float* y = reinterpret_cast<float*>(ws + o.y);
  float* z = reinterpret_cast<float*>(ws + o.z);
  double* v = reinterpret_cast<double*>(ws + o.v);
  double* qw = reinterpret_cast<double*>(ws + o.qw);
  double* beta = reinterpret_cast<double*>(ws + o.beta);
  float* bm = reinterpret_cast<float*>(ws + o.bm);
  double* cm = reinterpret_cast<double*>(ws + o.cm);
  double* u = reinterpret_cast<double*>(ws + o.u);
  float* g1 = reinterpret_cast<float*>(ws + o.g1);
  float* g2 = reinterpret_cast<float*>(ws + o.g2);
  const int n = int(N), k = int(K);
  hipLaunchKernelGGL(diff_kernel, dim3(4096), dim3(256), 0, s, static_cast<const __bf16*>(w_adapted),
                     static_cast<const __bf16*>(w_base), d, N * K);
  hipError_t e = hipGetLastError();
  auto orth = [&](float* m_, int rows) {
    hipLaunchKernelGGL(householder_q_kernel, dim3(1), dim3(256), 0, s, m_, v, qw, beta, rows, l);
    return hipGetLastError();
  };
  // Y = D Omega (N x l), Q = orth(Y)
  if (e == hipSuccess) e = gemm<float, float, float, float>(d, K, 1, omega, l, 1, y, l, n, l, k, s);
  if (e == hipSuccess) e = orth(y, n);
  for (int it = 0; it < power_iters && e == hipSuccess; ++it) {
    e = gemm<float, float, float, float>(d, 1, K, y, l, 1, z, l, k, l, n, s);   // Z = D^T Q (K x l)
    if (e == hipSuccess) e = orth(z, k);
    if (e == hipSuccess) e = gemm<float, float, float, float>(d, K, 1, z, l, 1, y, l, n, l, k, s);   // Y = D Z
    if (e == hipSuccess) e = orth(y, n);
  }
  // Bm = Q^T D (l x K); C = Bm Bm^T (fp64)
  if (e == hipSuccess) e = gemm<float, float, float, float>(y, 1, l, d, K, 1, bm, K, l, k, n, s);
  if (e == hipSuccess) e = gemm<float, float, double, double>(bm, K, 1, bm, 1, K, cm, l, l, l, k, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(256), 0, s, cm, u, l, 30, 1e-12);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(assemble_kernel, dim3(1), dim3(256), 0, s, cm, u, l, r, g1, g2, sigma_out);
    e = hipGetLastError();
  }
  // B = Q G1 (N x r), A = G2 Bm (r x K)
  if (e == hipSuccess) e = gemm<float, float, float, float>(y, l, 1, g1, r, 1, b_out, r, n, r, l, s);
  if (e == hipSuccess) e = gemm<float, float, float, float>(g2, l, 1, bm, K, 1, a_out, K, r, k, l, s);
  return e;
}

}  // namespace lora
