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
// outputs per thread); products with few output tiles split their long sums
// over slabs of workgroups and add the partial products in slab order (fp64
// for the l x l ones).  orth() is CholeskyQR (Fukaya, Nakatsukasa, Yanagisawa
// and Yamamoto, 2014; Yamamoto et al., "Roundoff error analysis of the
// CholeskyQR2 algorithm", 2015): the fp64 Gram matrix G = Y^T Y, its Cholesky
// factor R (blocked, one workgroup), Q = Y R^-1 (row tiles in LDS); the range
// that steps 4-6 use takes two passes (CholeskyQR2), the power-iteration steps
// one.  A column of Y whose Cholesky pivot falls below 1e-5 of its own length
// (relative, so 1e-10 on the squares) lies, to the rounding of Y, in the span
// of the earlier ones; it becomes a zero column of Q rather than an amplified
// rounding error, so a change of rank below l yields a Q with zero columns,
// whose eigenvalues in step 5 are zero.  Step 5 is a cyclic Jacobi eigensolver
// with the round-robin pairing, fp64, its rounds spread over a cooperative
// grid.
// Extraction runs once per weight matrix, outside the serving path.
#include <algorithm>
#include <cmath>

#include "lora_device.h"

namespace lora {
namespace {

constexpr int GT = 64;            // GEMM tile edge
constexpr int GK = 16;            // GEMM K slab
constexpr int kMaxL = 512;        // largest l (range width) the one-workgroup kernels hold
constexpr int kTrsmRows = 8;      // rows of Y per triangular-solve workgroup
constexpr int kTrsmStage = 8;     // rows of R staged in LDS at a time
constexpr double kDropTol = 1e-10;   // Cholesky pivot^2 / diagonal below which a column is dependent
constexpr int kMaxF32Splits = 4;     // K slabs of a split fp32 product

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
template <typename T>
__global__ __launch_bounds__(256) void sum_parts_kernel(const T* __restrict__ part, T* __restrict__ out, int64_t n,
                                                        int parts) {
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < n; e += int64_t(gridDim.x) * 256) {
    T s = 0;
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
// its upper triangle is overwritten by the Schur complements), one workgroup,
// blocked right-looking: each panel of kCholPanel rows of G's upper triangle is
// factored in LDS (one barrier per column), stored as rows of R, and then
// subtracted from the trailing upper triangle as one rank-kCholPanel update.
// A column whose pivot has fallen to tau times its diagonal in G lies, to
// rounding, in the span of the earlier columns: its row of R is zero and it
// takes no part in later updates, so the orthonormal factor gets a zero column
// there.
constexpr int kCholPanel = 32;

__global__ __launch_bounds__(1024) void cholesky_kernel(double* __restrict__ g, double* __restrict__ rm, int l,
                                                        double tau) {
  __shared__ double pnl[kCholPanel * kMaxL];   // panel row j, column c at pnl[j * kMaxL + c - jb]
  __shared__ double d0[kMaxL], pv[kCholPanel];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < l; i += 1024) d0[i] = g[int64_t(i) * l + i];
  for (int jb = 0; jb < l; jb += kCholPanel) {
    const int w = min(kCholPanel, l - jb), wl = l - jb;
    __syncthreads();
    for (int e = tid; e < w * wl; e += 1024) {
      const int j = e / wl, cc = e % wl;
      pnl[j * kMaxL + cc] = cc >= j ? g[int64_t(jb + j) * l + jb + cc] : 0.0;
    }
    __syncthreads();
    // factor the panel: eliminate column jb + j from the panel's later rows
    for (int j = 0; j < w; ++j) {
      const double gjj = pnl[j * kMaxL + j];
      const bool keep = d0[jb + j] > 0 && gjj > tau * d0[jb + j];   // the same for every thread
      if (tid == 0) pv[j] = keep ? sqrt(gjj) : 0.0;
      if (keep) {
        const double inv = 1.0 / gjj;
        for (int i = j + 1 + wave; i < w; i += 16) {
          const double f = pnl[j * kMaxL + i] * inv;
          for (int cc = i + lane; cc < wl; cc += 64) pnl[i * kMaxL + cc] -= f * pnl[j * kMaxL + cc];
        }
      }
      __syncthreads();
    }
    // rows jb .. jb + w - 1 of R, kept in LDS for the trailing update
    for (int e = tid; e < w * l; e += 1024) {
      const int j = e / l, c = e % l, cc = c - jb;
      double v = 0;
      if (cc >= j && pv[j] > 0) {
        v = pnl[j * kMaxL + cc] / pv[j];
        pnl[j * kMaxL + cc] = v;
      } else if (cc >= 0) {
        pnl[j * kMaxL + cc] = 0.0;
      }
      rm[int64_t(jb + j) * l + c] = v;
    }
    __syncthreads();
    // trailing upper triangle: G_ic -= sum_j R_ji R_jc
    for (int i = jb + w + wave; i < l; i += 16) {
      const int ci = i - jb;
      for (int c = i + lane; c < l; c += 64) {
        const int cc = c - jb;
        double acc = g[int64_t(i) * l + c];
#pragma unroll 8
        for (int j = 0; j < w; ++j) acc -= pnl[j * kMaxL + ci] * pnl[j * kMaxL + cc];
        g[int64_t(i) * l + c] = acc;
      }
    }
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
// 8.5).  A round rotates l/2 disjoint (p, q) pairs at once, so C <- J^T C J
// splits into independent 2 x 2 blocks (rows of one pair, columns of another),
// each updated in one step.  The eigenvector matrix is kept transposed (ut: row
// i = eigenvector i) so its update reads whole rows.  Leaves the eigenvalues on
// C's diagonal and eigenvector i in row i of ut.  l is even.  Stops when the
// off-diagonal mass is below tol^2 of the total.
//
// The work of a round is spread over the grid's kJacobiBlocks workgroups
// (cooperative launch, so all are resident), with a counter barrier between
// rounds.  C, ut and the convergence partials are written and read with
// device-scope (sc1) accesses, so the barrier is a vmcnt wait and one atomic
// add; the spin on the counter is bounded.  Every workgroup computes every
// pair's rotation from the same values, and sums the convergence partials in
// workgroup order, so all take the same decisions.  C alternates between two
// buffers from round to round (each round reads one and writes every element
// of the other), so a workgroup that runs ahead never overwrites an element
// that another still has to read in the same round; the result ends in cm.
constexpr int kJacobiBlocks = 64;

__device__ inline double ld64(__amdgpu_buffer_rsrc_t r, int64_t e) {
  return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, uint32_t(e * 8), 0, kDeviceScope));
}
__device__ inline void st64(__amdgpu_buffer_rsrc_t r, int64_t e, double v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, uint32_t(e * 8), 0, kDeviceScope);
}

// Every workgroup's stores are out, then each counts itself in and waits for
// `target` arrivals in all.
__device__ inline void grid_barrier(unsigned long long* ctr, unsigned long long target) {
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0; it < (1 << 24); ++it) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Pair k of round `round`: (round, l-1) and ((round + k) mod (l-1), (round - k)
// mod (l-1)), smaller index first.
__device__ inline void pair_of(int round, int k, int l, int& p, int& q) {
  p = k == 0 ? round : (round + k) % (l - 1);
  q = k == 0 ? l - 1 : (round - k + (l - 1)) % (l - 1);
  if (p > q) {
    const int t = p;
    p = q;
    q = t;
  }
}

__global__ __launch_bounds__(256) void jacobi_kernel(double* __restrict__ cm, double* __restrict__ cm2,
                                                     double* __restrict__ ut, double* __restrict__ part,
                                                     unsigned long long* ctr, int l, int max_sweeps, double tol) {
  constexpr int NB = 2, NU = 3;
  __shared__ double red[256];
  __shared__ double cs[kMaxL / 2], sn[kMaxL / 2], tn[kMaxL / 2];
  const int tid = threadIdx.x, nwg = gridDim.x;
  const int64_t stride = int64_t(nwg) * 256, first = int64_t(blockIdx.x) * 256 + tid;
  const uint32_t lb = uint32_t(l) * uint32_t(l) * 8u;
  const auto c0 = make_rsrc(cm, lb), c1 = make_rsrc(cm2, lb), ur = make_rsrc(ut, lb);
  const auto pr = make_rsrc(part, uint32_t(nwg) * 16u);
  int parity = 0;                          // C is in cm (0) or cm2 (1)
  unsigned long long target = 0;
  for (int64_t e = first; e < int64_t(l) * l; e += stride) st64(ur, e, (e / l == e % l) ? 1.0 : 0.0);
  target += nwg;
  grid_barrier(ctr, target);
  const int half = l / 2, nblk = half * half;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    const auto cr = parity ? c1 : c0;
    double off = 0, tot = 0;
    for (int64_t e = first; e < int64_t(l) * l; e += stride) {
      const double x = ld64(cr, e);
      tot += x * x;
      if (e / l != e % l) off += x * x;
    }
    off = block_sum<256>(off, red);
    tot = block_sum<256>(tot, red);
    if (tid == 0) {
      st64(pr, 2 * blockIdx.x, off);
      st64(pr, 2 * blockIdx.x + 1, tot);
    }
    target += nwg;
    grid_barrier(ctr, target);
    off = block_sum<256>(tid < nwg ? ld64(pr, 2 * tid) : 0.0, red);
    tot = block_sum<256>(tid < nwg ? ld64(pr, 2 * tid + 1) : 0.0, red);
    if (off <= tol * tol * tot) break;     // the same in every workgroup
    for (int round = 0; round < l - 1; ++round, parity ^= 1) {
      const auto cr = parity ? c1 : c0, cw = parity ? c0 : c1;
      // Batches of NB C blocks and NU eigenvector elements (rows p, q of ut at
      // one column); an index past the end loads a valid address and stores
      // nothing.  Every address depends on the round alone.
      double x[NB][4], xp[NU], xq[NU];
      int64_t at[NB][4], ap[NU], aq[NU];
      const int64_t nitem = int64_t(half) * l;
      auto load_blocks = [&](int64_t e0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          int64_t e = e0 + b * stride;
          if (e >= nblk) e = nblk - 1;
          int p, q, p2, q2;
          pair_of(round, int(e / half), l, p, q);
          pair_of(round, int(e % half), l, p2, q2);
          at[b][0] = int64_t(p) * l + p2;
          at[b][1] = int64_t(p) * l + q2;
          at[b][2] = int64_t(q) * l + p2;
          at[b][3] = int64_t(q) * l + q2;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[b][i] = ld64(cr, at[b][i]);
        }
      };
      auto load_vectors = [&](int64_t e0) {
#pragma unroll
        for (int b = 0; b < NU; ++b) {
          int64_t e = e0 + b * stride;
          if (e >= nitem) e = nitem - 1;
          int p, q;
          pair_of(round, int(e / l), l, p, q);
          const int j = int(e % l);
          ap[b] = int64_t(p) * l + j;
          aq[b] = int64_t(q) * l + j;
          xp[b] = ld64(ur, ap[b]);
          xq[b] = ld64(ur, aq[b]);
        }
      };
      // rows of pair k take (c, -s; s, c), the columns of pair k' its transpose
      // from the right; the pair's own block is diagonalised
      auto update_blocks = [&](int64_t e0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int64_t e = e0 + b * stride;
          if (e >= nblk) break;
          const int k = int(e / half), k2 = int(e % half);
          double o0, o1, o2, o3;
          if (k == k2) {
            const double t = tn[k], a = x[b][1];
            o0 = x[b][0] - t * a;
            o3 = x[b][3] + t * a;
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
          st64(cw, at[b][0], o0);
          st64(cw, at[b][1], o1);
          st64(cw, at[b][2], o2);
          st64(cw, at[b][3], o3);
        }
      };
      auto update_vectors = [&](int64_t e0) {
#pragma unroll
        for (int b = 0; b < NU; ++b) {
          const int64_t e = e0 + b * stride;
          if (e >= nitem) break;
          const int k = int(e / l);
          const double c = cs[k], s = sn[k];
          st64(ur, ap[b], c * xp[b] - s * xq[b]);
          st64(ur, aq[b], s * xp[b] + c * xq[b]);
        }
      };
      // the rotation inputs (one pair per thread) and the first batches go out
      // together
      int pk = 0, qk = 0;
      double app = 0, aqq = 0, apq = 0;
      if (tid < half) {
        pair_of(round, tid, l, pk, qk);
        app = ld64(cr, int64_t(pk) * l + pk);
        aqq = ld64(cr, int64_t(qk) * l + qk);
        apq = ld64(cr, int64_t(pk) * l + qk);
      }
      load_blocks(first);
      load_vectors(first);
      if (tid < half) {
        double c = 1, s = 0, t = 0;
        if (apq != 0) {
          const double tau = (aqq - app) / (2 * apq);
          t = tau >= 0 ? 1.0 / (tau + sqrt(1 + tau * tau)) : -1.0 / (-tau + sqrt(1 + tau * tau));
          c = 1.0 / sqrt(1 + t * t);
          s = t * c;
        }
        cs[tid] = c;
        sn[tid] = s;
        tn[tid] = t;
      }
      __syncthreads();
      update_blocks(first);
      update_vectors(first);
      for (int64_t e0 = first + NB * stride; e0 < nblk; e0 += NB * stride) {
        load_blocks(e0);
        update_blocks(e0);
      }
      for (int64_t e0 = first + NU * stride; e0 < nitem; e0 += NU * stride) {
        load_vectors(e0);
        update_vectors(e0);
      }
      target += nwg;
      grid_barrier(ctr, target);
    }
  }
  if (parity)
    for (int64_t e = first; e < int64_t(l) * l; e += stride) st64(c0, e, ld64(c1, e));
}

__global__ void zero_counter_kernel(unsigned long long* ctr) { *ctr = 0; }

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

// Slabs of an fp32 product whose output has too few tiles to fill the GPU
// (at least 1024 workgroups wanted), each slab at least 1024 terms long.
int fp32_splits(int64_t tiles, int64_t k) {
  if (tiles >= 1024) return 1;
  return int(std::max<int64_t>(1, std::min<int64_t>({(1024 + tiles - 1) / tiles, k / 1024, kMaxF32Splits})));
}

// C = A B in fp32 (C row-major, ldc = N).  With few output tiles the K range
// splits into slabs; their partial products (in `part`) are then summed in
// slab order.
hipError_t gemm(const float* a, int64_t sam, int64_t sak, const float* b, int64_t sbk, int64_t sbn, float* c,
                float* part, int M, int N, int K, hipStream_t s) {
  const int64_t tiles = int64_t((N + GT - 1) / GT) * ((M + GT - 1) / GT);
  const int want = fp32_splits(tiles, K);
  const int chunk = ((K + want - 1) / want + GK - 1) / GK * GK;
  const int parts = (K + chunk - 1) / chunk;
  const int64_t mn = int64_t(M) * N;
  const dim3 grid(unsigned((N + GT - 1) / GT), unsigned((M + GT - 1) / GT), unsigned(parts));
  hipLaunchKernelGGL((gemm_kernel<float, float, float, float>), grid, dim3(256), 0, s, a, sam, sak, b, sbk, sbn,
                     parts > 1 ? part : c, int64_t(N), M, N, K, chunk, parts > 1 ? mn : int64_t(0));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || parts == 1) return e;
  const unsigned blocks = unsigned(std::min<int64_t>((mn + 255) / 256, 2048));
  hipLaunchKernelGGL(sum_parts_kernel<float>, dim3(blocks), dim3(256), 0, s, part, c, mn, parts);
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
  hipLaunchKernelGGL(sum_parts_kernel<double>, dim3(blocks), dim3(256), 0, s, part, c, mn, parts);
  return hipGetLastError();
}

size_t r256(size_t x) { return (x + 255) & ~size_t(255); }

struct ExtractLayout {
  size_t d, y, z, part, fpart, g, rm, bm, cm, cm2, ut, g1, g2, jpart, ctr, total;
};

ExtractLayout extract_layout(int64_t N, int64_t K, int64_t l, int64_t r) {
  ExtractLayout o;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += r256(bytes); return at; };
  o.d = take(size_t(N) * K * 4);
  o.y = take(size_t(N) * l * 4);
  o.z = take(size_t(K) * l * 4);
  o.part = take(size_t(split_count(std::max(N, K))) * l * l * 8);
  o.fpart = take(size_t(kMaxF32Splits) * std::max(std::max(N, K) * l, r * K) * 4);
  o.g = take(size_t(l) * l * 8);
  o.rm = take(size_t(l) * l * 8);
  o.bm = take(size_t(l) * K * 4);
  o.cm = take(size_t(l) * l * 8);
  o.cm2 = take(size_t(l) * l * 8);
  o.ut = take(size_t(l) * l * 8);
  o.g1 = take(size_t(l) * r * 4);
  o.g2 = take(size_t(r) * l * 4);
  o.jpart = take(size_t(kJacobiBlocks) * 16);
  o.ctr = take(8);
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
  float* fpart = reinterpret_cast<float*>(ws + o.fpart);
  double* g = reinterpret_cast<double*>(ws + o.g);
  double* rm = reinterpret_cast<double*>(ws + o.rm);
  float* bm = reinterpret_cast<float*>(ws + o.bm);
  double* cm = reinterpret_cast<double*>(ws + o.cm);
  double* cm2 = reinterpret_cast<double*>(ws + o.cm2);
  double* ut = reinterpret_cast<double*>(ws + o.ut);
  float* g1 = reinterpret_cast<float*>(ws + o.g1);
  float* g2 = reinterpret_cast<float*>(ws + o.g2);
  double* jpart = reinterpret_cast<double*>(ws + o.jpart);
  unsigned long long* ctr = reinterpret_cast<unsigned long long*>(ws + o.ctr);
  const int n = int(N), k = int(K);
  hipLaunchKernelGGL(diff_kernel, dim3(4096), dim3(256), 0, s, static_cast<const __bf16*>(w_adapted),
                     static_cast<const __bf16*>(w_base), d, N * K);
  hipError_t e = hipGetLastError();
  // orth(): CholeskyQR, Y (rows x l) overwritten by Q.  Inside the power
  // iterations only the span of Q matters, and one pass keeps it (its Q is
  // orthogonal to about u cond(Y)^2, cond(Y) at most 1e5 after the drop
  // test); the range that Bm and B are formed from takes a second pass, which
  // restores orthogonality to rounding.
  auto orth = [&](float* m_, int rows, int passes) {
    hipError_t err = hipSuccess;
    for (int pass = 0; pass < passes && err == hipSuccess; ++pass) {
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
  if (e == hipSuccess) e = gemm(d, K, 1, omega, l, 1, y, fpart, n, l, k, s);
  if (e == hipSuccess) e = orth(y, n, power_iters > 0 ? 1 : 2);
  for (int it = 0; it < power_iters && e == hipSuccess; ++it) {
    e = gemm(d, 1, K, y, l, 1, z, fpart, k, l, n, s);   // Z = D^T Q (K x l)
    if (e == hipSuccess) e = orth(z, k, 1);
    if (e == hipSuccess) e = gemm(d, K, 1, z, l, 1, y, fpart, n, l, k, s);   // Y = D Z
    if (e == hipSuccess) e = orth(y, n, it + 1 == power_iters ? 2 : 1);
  }
  // Bm = Q^T D (l x K); C = Bm Bm^T (fp64)
  if (e == hipSuccess) e = gemm(y, 1, l, d, K, 1, bm, fpart, l, k, n, s);
  if (e == hipSuccess) e = gemm_splitk<float, float>(bm, K, 1, bm, 1, K, cm, part, l, l, k, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(1), 0, s, ctr);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    int ll = l, sweeps = 30;
    double tol = 1e-10;
    void* args[] = {&cm, &cm2, &ut, &jpart, &ctr, &ll, &sweeps, &tol};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&jacobi_kernel), dim3(kJacobiBlocks), dim3(256),
                                   args, 0, s);
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(assemble_kernel, dim3(1), dim3(256), 0, s, cm, ut, l, r, g1, g2, sigma_out);
    e = hipGetLastError();
  }
  // B = Q G1 (N x r), A = G2 Bm (r x K)
  if (e == hipSuccess) e = gemm(y, l, 1, g1, r, 1, b_out, fpart, n, r, l, s);
  if (e == hipSuccess) e = gemm(g2, l, 1, bm, K, 1, a_out, fpart, r, k, l, s);
  return e;
}

}  // namespace lora
