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
// outputs per thread); the l x l ones split their long sums over many
// workgroups and add the partial products in fp64.  orth() is CholeskyQR2
// (Fukaya, Nakatsukasa, Yanagisawa and Yamamoto, 2014; Yamamoto et al.,
// "Roundoff error analysis of the CholeskyQR2 algorithm", 2015): the fp64 Gram
// matrix G = Y^T Y, its Cholesky factor R (one workgroup), Q = Y R^-1 (row
// tiles in LDS), done twice.  A column of Y whose Cholesky pivot falls below
// 1e-5 of its own length (relative, so 1e-10 on the squares) lies, to the
// rounding of Y, in the span of the earlier ones; it becomes a zero column of Q
// rather than an amplified rounding error, so a change of rank below l yields a
// Q with zero columns, whose eigenvalues in step 5 are zero.  Step 5 is a cyclic
// Jacobi eigensolver with the round-robin pairing in one workgroup, fp64.
// Extraction runs once per weight matrix, outside the serving path.
#include <algorithm>
#include <cmath>

#include "lora_internal.h"

namespace lora {
namespace {

constexpr int GT = 64;            // GEMM tile edge
constexpr int GK = 16;            // GEMM K slab
constexpr int kMaxL = 512;        // largest l (range width) the one-workgroup kernels hold
constexpr int kTrsmRows = 8;      // rows of Y per triangular-solve workgroup
constexpr int kTrsmStage = 8;     // rows of R staged in LDS at a time
constexpr double kDropTol = 1e-10;   // Cholesky pivot^2 / diagonal below which a column is dependent

__global__ __launch_bounds__(256) void diff_kernel(const __bf16* __restrict__ a, const __bf16* __restrict__ b,
                                                   float* __restrict__ d, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    d[i] = float(a[i]) - float(b[i]);
}

// C[m][n] = sum_k A(m, k) B(k, n), A(m, k) = a[m sam + k sak], B(k, n) = b[k sbk + n sbn],
// C row-major (ldc), accumulated in TACC.  Split K: workgroup z sums k in
// [z kchunk, (z + 1) kchunk) and writes its partial product at c + z cz.
template <typename TA, typename TB, typename TACC, typename TC>
__global__ __launch_bounds__(256) void gemm_kernel(const TA* __restrict__ a, int64_t sam, int64_t sak,
                                                   const TB* __restrict__ b, int64_t sbk, int64_t sbn,
                                                   TC* __restrict__ c, int64_t ldc, int M, int N, int K, int kchunk,
                                                   int64_t cz) {
  __shared__ TACC as[GK][GT + 1], bs[GK][GT + 1];
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
  c += int64_t(blockIdx.z) * cz;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  TACC acc[4][4] = {};
  for (int k0 = kb; k0 < ke; k0 += GK) {
    for (int e = tid; e < GK * GT; e += 256) {
      const int kk = e / GT, mm = e % GT;
      const int m = m0 + mm, k = k0 + kk;
      as[kk][mm] = (m < M && k < ke) ? TACC(a[int64_t(m) * sam + int64_t(k) * sak]) : TACC(0);
      const int n = n0 + mm;
      bs[kk][mm] = (n < N && k < ke) ? TACC(b[int64_t(k) * sbk + int64_t(n) * sbn]) : TACC(0);
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

// out[e] = sum over the `parts` partial products part[z * n + e], in z order.
__global__ __launch_bounds__(256) void sum_parts_kernel(const double* __restrict__ part, double* __restrict__ out,
                                                        int64_t n, int parts) {
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += int64_t(gridDim.x) * 256) {
    double s = 0;
    for (int z = 0; z < parts; ++z) s += part[int64_t(z) * n + e];
    out[e] = s;
  }
}

template <int NT>
__device__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// Upper-triangular R with G = R^T R for the Gram matrix G = Y^T Y (l x l fp64;
// its upper triangle is overwritten by the Schur complements), right-looking,
// one workgroup.  A column whose pivot has fallen to tau times its diagonal in
// G lies, to rounding, in the span of the earlier columns: its row of R is zero
// and it takes no part in later updates, so the orthonormal factor gets a zero
// column there.
__global__ __launch_bounds__(1024) void cholesky_kernel(double* __restrict__ g, double* __restrict__ rm, int l,
                                                        double tau) {
  __shared__ double d0[kMaxL];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < l; i += 1024) d0[i] = g[int64_t(i) * l + i];
  __syncthreads();
  for (int j = 0; j < l; ++j) {
    const double* gj = g + int64_t(j) * l;
    const double gjj = gj[j];
    const bool keep = d0[j] > 0 && gjj > tau * d0[j];   // the same for every thread
    const double piv = keep ? sqrt(gjj) : 0.0;
    for (int c = tid; c < l; c += 1024)
      rm[int64_t(j) * l + c] = (!keep || c < j) ? 0.0 : (c == j ? piv : gj[c] / piv);
    if (keep) {
      const double inv = 1.0 / gjj;
      for (int i = j + 1 + wave; i < l; i += 16) {       // rows of the trailing upper triangle
        const double f = gj[i] * inv;
        double* gi = g + int64_t(i) * l;
        for (int c = i + lane; c < l; c += 64) gi[c] -= f * gj[c];
      }
    }
    __syncthreads();
  }
}

// Q = Y R^-1 in place (Y: m x l row-major fp32; R from cholesky_kernel, a zero
// pivot giving a zero column).  Each workgroup solves kTrsmRows rows of Y in
// LDS in fp64, column by column: the columns stay unscaled until the end, so
// step j subtracts y_j (R_jc / R_jj) from every later column c, with the rows
// of R / diag(R) staged through LDS kTrsmStage at a time.
__global__ __launch_bounds__(256) void trsm_kernel(float* __restrict__ y, const double* __restrict__ rm, int m,
                                                   int l) {
  extern __shared__ double lds[];
  double* qs = lds;                           // kTrsmRows x l
  double* rs = lds + kTrsmRows * l;           // kTrsmStage x l
  const int tid = threadIdx.x, tx = tid & 63, ty = tid >> 6;
  const int r0 = blockIdx.x * kTrsmRows, rows = min(kTrsmRows, m - r0);
  float* yt = y + int64_t(r0) * l;
  for (int e = tid; e < kTrsmRows * l; e += 256) qs[e] = e < rows * l ? double(yt[e]) : 0.0;
  for (int j0 = 0; j0 < l - 1; j0 += kTrsmStage) {
    __syncthreads();
    for (int e = tid; e < kTrsmStage * l; e += 256) {
      const int j = j0 + e / l, c = e % l;
      double f = 0;
      if (j < l && c > j) {
        const double rjj = rm[int64_t(j) * l + j];
        if (rjj != 0) f = rm[int64_t(j) * l + c] / rjj;
      }
      rs[e] = f;
    }
    __syncthreads();
    const int jn = min(kTrsmStage, l - 1 - j0);
    for (int jj = 0; jj < jn; ++jj) {
      const int j = j0 + jj;
      for (int c = j + 1 + tx; c < l; c += 64) {
        const double f = rs[jj * l + c];
#pragma unroll
        for (int r = ty; r < kTrsmRows; r += 4) qs[r * l + c] -= qs[r * l + j] * f;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  for (int e = tid; e < rows * l; e += 256) {
    const int c = e % l;
    const double rcc = rm[int64_t(c) * l + c];
    yt[e] = rcc != 0 ? float(qs[e] / rcc) : 0.0f;
  }
}

// Eigenpairs of the symmetric l x l matrix C (fp64, overwritten): cyclic Jacobi
// with the round-robin pairing (Golub and Van Loan, "Matrix Computations",
// 8.5), one workgroup.  A round rotates l/2 disjoint (p, q) pairs at once, so
// C <- J^T C J splits into independent 2 x 2 blocks (rows of one pair, columns
// of another), each updated in one step; the eigenvector matrix is kept
// transposed (ut: row i = eigenvector i) so its update reads whole rows.
// Leaves the eigenvalues on C's diagonal and eigenvector i in row i of ut.  l
// is even.  Stops when the off-diagonal mass is below tol^2 of the total.
__global__ __launch_bounds__(1024) void jacobi_kernel(double* __restrict__ cm, double* __restrict__ ut, int l,
                                                      int max_sweeps, double tol) {
  constexpr int NT = 1024, NB = 4;
  __shared__ double red[NT];
  __shared__ double cs[kMaxL / 2], sn[kMaxL / 2], tn[kMaxL / 2];
  __shared__ int pp[kMaxL / 2], qq[kMaxL / 2];
  const int tid = threadIdx.x;
  for (int64_t e = tid; e < int64_t(l) * l; e += NT) ut[e] = (e / l == e % l) ? 1.0 : 0.0;
  const int half = l / 2, nblk = half * half;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    __syncthreads();
    double off = 0, tot = 0;
    for (int64_t e = tid; e < int64_t(l) * l; e += NT) {
      const double x = cm[e] * cm[e];
      tot += x;
      if (e / l != e % l) off += x;
    }
    off = block_sum<NT>(off, red);
    tot = block_sum<NT>(tot, red);
    if (off <= tol * tol * tot) break;
    for (int round = 0; round < l - 1; ++round) {
      // pairing of round `round`: (round, l-1) and ((round + k) mod (l-1), (round - k) mod (l-1))
      for (int k = tid; k < half; k += NT) {
        int p = k == 0 ? round : (round + k) % (l - 1);
        int q = k == 0 ? l - 1 : (round - k + (l - 1)) % (l - 1);
        if (p > q) {
          const int t = p;
          p = q;
          q = t;
        }
        const double apq = cm[int64_t(p) * l + q];
        double c = 1, s = 0, t = 0;
        if (apq != 0) {
          const double tau = (cm[int64_t(q) * l + q] - cm[int64_t(p) * l + p]) / (2 * apq);
          t = tau >= 0 ? 1.0 / (tau + sqrt(1 + tau * tau)) : -1.0 / (-tau + sqrt(1 + tau * tau));
          c = 1.0 / sqrt(1 + t * t);
          s = t * c;
        }
        pp[k] = p;
        qq[k] = q;
        cs[k] = c;
        sn[k] = s;
        tn[k] = t;
      }
      __syncthreads();
      // C blocks: rows (p, q) of pair k, columns (p', q') of pair k'; the rows
      // take (c, -s; s, c), the columns its transpose from the right.  NB blocks
      // are loaded before any is stored (they are disjoint).
      for (int e0 = tid; e0 < nblk; e0 += NT * NB) {
        double x[NB][4];
        int64_t at[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int e = min(e0 + b * NT, nblk - 1);
          const int k = e / half, k2 = e % half;
          const int64_t p = pp[k], q = qq[k], p2 = pp[k2], q2 = qq[k2];
          at[b][0] = p * l + p2;
          at[b][1] = p * l + q2;
          at[b][2] = q * l + p2;
          at[b][3] = q * l + q2;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[b][i] = cm[at[b][i]];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int e = e0 + b * NT;
          if (e >= nblk) break;
          const int k = e / half, k2 = e % half;
          double o0, o1, o2, o3;
          if (k == k2) {       // the pair's own block: diagonalised
            const double t = tn[k], apq = x[b][1];
            o0 = x[b][0] - t * apq;
            o3 = x[b][3] + t * apq;
            o1 = o2 = 0;
          } else {
            const double c = cs[k], s = sn[k], c2 = cs[k2], s2 = sn[k2];
            const double r0 = c * x[b][0] - s * x[b][2], r1 = c * x[b][1] - s * x[b][3];
            const double r2 = s * x[b][0] + c * x[b][2], r3 = s * x[b][1] + c * x[b][3];
            o0 = c2 * r0 - s2 * r1;
            o1 = s2 * r0 + c2 * r1;
            o2 = c2 * r2 - s2 * r3;
            o3 = s2 * r2 + c2 * r3;
          }
          cm[at[b][0]] = o0;
          cm[at[b][1]] = o1;
          cm[at[b][2]] = o2;
          cm[at[b][3]] = o3;
        }
      }
      // eigenvectors: rows p, q of ut, two columns per item
      const int hl = l / 2, nu = half * hl;
      for (int e0 = tid; e0 < nu; e0 += NT * NB) {
        double2 xp[NB], xq[NB];
        int64_t ap[NB], aq[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int e = min(e0 + b * NT, nu - 1);
          const int k = e / hl, j = 2 * (e % hl);
          ap[b] = int64_t(pp[k]) * l + j;
          aq[b] = int64_t(qq[k]) * l + j;
          xp[b] = *reinterpret_cast<const double2*>(ut + ap[b]);
          xq[b] = *reinterpret_cast<const double2*>(ut + aq[b]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int e = e0 + b * NT;
          if (e >= nu) break;
          const int k = e / hl;
          const double c = cs[k], s = sn[k];
          *reinterpret_cast<double2*>(ut + ap[b]) = double2{c * xp[b].x - s * xq[b].x, c * xp[b].y - s * xq[b].y};
          *reinterpret_cast<double2*>(ut + aq[b]) = double2{s * xp[b].x + c * xq[b].x, s * xp[b].y + c * xq[b].y};
        }
      }
      __syncthreads();
    }
  }
}

// From the eigenpairs: order by eigenvalue (largest first), s_i = sqrt(L_i);
// G1 = W_r S^(1/2) (l x r), G2 = S^(-1/2) W_r^T (r x l), sigma = s_r.  One
// workgroup; each eigenvalue's place is the count of those ahead of it (larger,
// or equal with a smaller index; a NaN counts as the smallest), a permutation.
__global__ __launch_bounds__(256) void assemble_kernel(const double* __restrict__ cm, const double* __restrict__ ut,
                                                       int l, int r, float* __restrict__ g1, float* __restrict__ g2,
                                                       float* __restrict__ sigma) {
  __shared__ int order[kMaxL];
  __shared__ double lam[kMaxL], sv[kMaxL];
  const int tid = threadIdx.x;
  for (int i = tid; i < l; i += 256) {
    const double x = cm[int64_t(i) * l + i];
    lam[i] = x == x ? x : -INFINITY;
  }
  __syncthreads();
  for (int i = tid; i < l; i += 256) {
    const double li = lam[i];
    int place = 0;
    for (int j = 0; j < l; ++j) place += (lam[j] > li || (lam[j] == li && j < i)) ? 1 : 0;
    if (place < r) {
      order[place] = i;
      sv[place] = li > 0 ? sqrt(li) : 0.0;
    }
  }
  __syncthreads();
  for (int e = tid; e < l * r; e += 256) {
    const int i = e / r, j = e % r;
    const double w = ut[int64_t(order[j]) * l + i];
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
                     K, K, int64_t(0));
  return hipGetLastError();
}

// Slabs of the split-K products (a few hundred terms each, at most 32).
int split_count(int64_t k) { return int(std::min<int64_t>(std::max<int64_t>((k + 511) / 512, 1), 32)); }

// C (M x N fp64, row-major) = A B over a long K, in fp64: the K range splits
// into slabs whose partial products (in `part`) are then summed in slab order.
template <typename TA, typename TB>
hipError_t gemm_splitk(const TA* a, int64_t sam, int64_t sak, const TB* b, int64_t sbk, int64_t sbn, double* c,
                       double* part, int M, int N, int K, hipStream_t s) {
  const int want = split_count(K);
  const int chunk = ((K + want - 1) / want + GK - 1) / GK * GK;
  const int parts = (K + chunk - 1) / chunk;
  const int64_t mn = int64_t(M) * N;
  const dim3 grid(unsigned((N + GT - 1) / GT), unsigned((M + GT - 1) / GT), unsigned(parts));
  hipLaunchKernelGGL((gemm_kernel<TA, TB, double, double>), grid, dim3(256), 0, s, a, sam, sak, b, sbk, sbn, part,
                     int64_t(N), M, N, K, chunk, mn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned blocks = unsigned(std::min<int64_t>((mn + 255) / 256, 1024));
  hipLaunchKernelGGL(sum_parts_kernel, dim3(blocks), dim3(256), 0, s, part, c, mn, parts);
  return hipGetLastError();
}

size_t r256(size_t x) { return (x + 255) & ~size_t(255); }

struct ExtractLayout {
  size_t d, y, z, part, g, rm, bm, cm, ut, g1, g2, total;
};

ExtractLayout extract_layout(int64_t N, int64_t K, int64_t l, int64_t r) {
  ExtractLayout o;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += r256(bytes); return at; };
  o.d = take(size_t(N) * K * 4);
  o.y = take(size_t(N) * l * 4);
  o.z = take(size_t(K) * l * 4);
  o.part = take(size_t(split_count(std::max(N, K))) * l * l * 8);
  o.g = take(size_t(l) * l * 8);
  o.rm = take(size_t(l) * l * 8);
  o.bm = take(size_t(l) * K * 4);
  o.cm = take(size_t(l) * l * 8);
  o.ut = take(size_t(l) * l * 8);
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
  double* part = reinterpret_cast<double*>(ws + o.part);
  double* g = reinterpret_cast<double*>(ws + o.g);
  double* rm = reinterpret_cast<double*>(ws + o.rm);
  float* bm = reinterpret_cast<float*>(ws + o.bm);
  double* cm = reinterpret_cast<double*>(ws + o.cm);
  double* ut = reinterpret_cast<double*>(ws + o.ut);
  float* g1 = reinterpret_cast<float*>(ws + o.g1);
  float* g2 = reinterpret_cast<float*>(ws + o.g2);
  const int n = int(N), k = int(K);
  hipLaunchKernelGGL(diff_kernel, dim3(4096), dim3(256), 0, s, static_cast<const __bf16*>(w_adapted),
                     static_cast<const __bf16*>(w_base), d, N * K);
  hipError_t e = hipGetLastError();
  // orth(): CholeskyQR twice (the second pass restores orthogonality to
  // rounding), Y (rows x l) overwritten by Q
  auto orth = [&](float* m_, int rows) {
    hipError_t err = hipSuccess;
    for (int pass = 0; pass < 2 && err == hipSuccess; ++pass) {
      err = gemm_splitk<float, float>(m_, 1, l, m_, l, 1, g, part, l, l, rows, s);   // G = Y^T Y
      if (err != hipSuccess) break;
      hipLaunchKernelGGL(cholesky_kernel, dim3(1), dim3(1024), 0, s, g, rm, l, kDropTol);
      err = hipGetLastError();
      if (err != hipSuccess) break;
      const unsigned tiles = unsigned((rows + kTrsmRows - 1) / kTrsmRows);
      const size_t lds = size_t(kTrsmRows + kTrsmStage) * l * sizeof(double);
      hipLaunchKernelGGL(trsm_kernel, dim3(tiles), dim3(256), lds, s, m_, rm, rows, l);
      err = hipGetLastError();
    }
    return err;
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
  if (e == hipSuccess) e = gemm_splitk<float, float>(bm, K, 1, bm, 1, K, cm, part, l, l, k, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(1024), 0, s, cm, ut, l, 30, 1e-12);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(assemble_kernel, dim3(1), dim3(256), 0, s, cm, ut, l, r, g1, g2, sigma_out);
    e = hipGetLastError();
  }
  // B = Q G1 (N x r), A = G2 Bm (r x K)
  if (e == hipSuccess) e = gemm<float, float, float, float>(y, l, 1, g1, r, 1, b_out, r, n, r, l, s);
  if (e == hipSuccess) e = gemm<float, float, float, float>(g2, l, 1, bm, K, 1, a_out, K, r, k, l, s);
  return e;
}

}  // namespace lora
