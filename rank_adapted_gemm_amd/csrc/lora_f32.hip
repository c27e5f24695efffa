// fp32 test-mode kernels of the mixed-adapter LoRA projection.
//
// Same two launches and the same segment scheduling as the bf16 path, in fp32
// throughout: shrink T = s_a X_a A_a^T (fp32 workspace), then
// Y = X W^T (+ T B_a^T on adapter rows).  64x64 output tiles, 256 threads with
// a 4x4 register block each, 16-wide K slabs staged transposed in LDS, fused
// multiply-adds in ascending k order.  Meant for tight parity checks of the
// scheduling and indexing, not for speed.
#include "lora_device.h"

namespace lora {
namespace {

constexpr int T64 = 64;     // tile edge
constexpr int FK = 16;      // K slab
constexpr int PAD = 4;

struct FSide {            // rows of a row-major fp32 matrix; rows outside [lo, hi) read as zero
  __amdgpu_buffer_rsrc_t res;
  uint32_t ld_bytes;
  int32_t row0, lo, hi;
};

// Load a 64 x 16 slab (rows of the side, k0..k0+15) and store it k-major in LDS.
__device__ __forceinline__ void stage(float (*dst)[T64 + PAD], const FSide& s, int k0, int kdim, int tid) {
  const int r = tid >> 2, c = (tid & 3) * 4;
  const int grow = s.row0 + r, kk = k0 + c;
  const bool ok = grow >= s.lo && grow < s.hi && kk < kdim;
  const uint32_t off = ok ? uint32_t(grow) * s.ld_bytes + uint32_t(kk) * 4u : kMaskedOffset;
  const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(s.res, off, 0, 0));
  dst[c + 0][r] = v[0];
  dst[c + 1][r] = v[1];
  dst[c + 2][r] = v[2];
  dst[c + 3][r] = v[3];
}

// acc[i][j] += sum_k x[m_i, k] w[n_j, k]
__device__ __forceinline__ void accumulate(float (&acc)[4][4], const FSide& ws, const FSide& xs, int kdim,
                                           float (*xl)[T64 + PAD], float (*wl)[T64 + PAD], int tid) {
  const int tx = tid & 15, ty = tid >> 4;
  for (int k0 = 0; k0 < kdim; k0 += FK) {
    stage(xl, xs, k0, kdim, tid);
    stage(wl, ws, k0, kdim, tid);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xl[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = wl[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
}

// Grid: (rank tiles) x (row tiles).  T[m, j] = s sum_k X[m, k] A_a[j, k] on adapter rows.
__global__ __launch_bounds__(256) void f32_shrink_kernel(ProjArgs p, SegTable st, AdapterTable at) {
  __shared__ float xl[FK][T64 + PAD], wl[FK][T64 + PAD];
  const int j0 = blockIdx.x * T64, m0 = blockIdx.y * T64;
  const int m1 = min(m0 + T64, p.M);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const auto xres = make_rsrc(p.X, p.x_bytes);
  const auto tres = make_rsrc(p.T, p.t_bytes);
  for (int g = first_segment(st, m0); g < st.n && st.start[g] < m1; ++g) {
    const int a = st.adapter[g];
    if (a < 0) continue;
    const int lo = max(st.start[g], m0), hi = min(st.start[g + 1], m1);
    float acc[4][4] = {};
    const FSide as{make_rsrc(at.A[a], at.a_bytes[a]), uint32_t(p.K) * 4u, j0, 0, p.sl.n * at.rank[a]};
    const FSide xs{xres, uint32_t(p.K) * 4u, m0, lo, hi};
    accumulate(acc, as, xs, p.K, xl, wl, tid);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + ty * 4 + i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int jr = j0 + tx * 4 + j;
        const bool ok = m >= lo && m < hi && jr < p.trank;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, at.scale[a] * acc[i][j]), tres,
                                              ok ? (uint32_t(m) * uint32_t(p.trank) + uint32_t(jr)) * 4u
                                                 : kMaskedOffset, 0, 0);
      }
    }
  }
}

// Grid: (column tiles) x (row tiles).
__global__ __launch_bounds__(256) void f32_main_kernel(ProjArgs p, SegTable st, AdapterTable at, int has_adapter) {
  __shared__ float xl[FK][T64 + PAD], wl[FK][T64 + PAD];
  const int n0 = blockIdx.x * T64, m0 = blockIdx.y * T64;
  const int m1 = min(m0 + T64, p.M);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  {
    const FSide ws{make_rsrc(p.W, p.w_bytes), uint32_t(p.K) * 4u, n0, 0, p.N};
    const FSide xs{make_rsrc(p.X, p.x_bytes), uint32_t(p.K) * 4u, m0, 0, p.M};
    accumulate(acc, ws, xs, p.K, xl, wl, tid);
  }
  if (has_adapter) {   // the tile's slice reads its own r_a columns of T
    const int slice = slice_of(p.sl, n0);
    for (int g = first_segment(st, m0); g < st.n && st.start[g] < m1; ++g) {
      const int a = st.adapter[g];
      if (a < 0) continue;
      const int lo = max(st.start[g], m0), hi = min(st.start[g + 1], m1), ra = at.rank[a];
      const uint32_t tcol = uint32_t(slice * ra) * 4u;
      const auto tres = make_rsrc(static_cast<const char*>(p.T) + tcol, p.t_bytes - tcol);
      const FSide bs{make_rsrc(at.B[a], at.b_bytes[a]), uint32_t(ra) * 4u, n0, 0, p.N};
      const FSide ts{tres, uint32_t(p.trank) * 4u, m0, lo, hi};
      accumulate(acc, bs, ts, ra, xl, wl, tid);
    }
  }
  const auto yres = make_rsrc(p.Y, p.y_bytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      const bool ok = m < p.M && n < p.N;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[i][j]), yres,
                                            ok ? (uint32_t(m) * uint32_t(p.N) + uint32_t(n)) * 4u : kMaskedOffset,
                                            0, 0);
    }
  }
}

}  // namespace

hipError_t launch_f32_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at, hipStream_t stream) {
  ProjArgs pa = p;
  SegTable sa = st;
  AdapterTable aa = at;
  void* args[] = {&pa, &sa, &aa};
  const dim3 grid((p.trank + T64 - 1) / T64, (p.M + T64 - 1) / T64);
  return hipLaunchKernel(reinterpret_cast<const void*>(&f32_shrink_kernel), grid, dim3(256), args, 0, stream);
}

hipError_t launch_f32_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at, bool has_adapter,
                           hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  ProjArgs pa = p;
  SegTable sa = st;
  AdapterTable aa = at;
  int ha = has_adapter ? 1 : 0;
  void* args[] = {&pa, &sa, &aa, &ha};
  const dim3 grid((p.N + T64 - 1) / T64, (p.M + T64 - 1) / T64);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(&f32_main_kernel), grid, dim3(256), args, 0, stream, e0, e1,
                            0);
}

}  // namespace lora
