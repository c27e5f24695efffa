// bf16 kernels of the mixed-adapter LoRA projection for gfx950 (CDNA4).
//
// Two launches per call ("two 27B models on a single RTX 5090", section 4
// request-path figure: each changed matrix runs the base product plus the
// adapter's two thin matrices, for adapter requests only):
//
//   shrink  T = s X_a A_a^T on the rows of adapter segments.  T is stored as
//           two bf16 halves, hi = bf16(T) and lo = bf16(T - hi), so the expand
//           can run on bf16 MFMA while keeping T to about 2^-17 relative.
//   main    per output tile: acc = X W^T over K, then, if the tile holds adapter
//           rows, acc += T_hi B_a^T + T_lo B_a^T over the rank (rows of other
//           segments read as zero), then one round-to-nearest-even store.
//
// Both run the same LDS-staged MFMA K-loop: 16-byte buffer loads of 64-element
// K slabs into registers, a double-buffered LDS stage with an XOR swizzle on
// 16-byte chunks (conflict-free ds_read_b128), and v_mfma_f32_32x32x16_bf16
// with fp32 accumulators.  The MFMA "A" operand is the weight side (rows n) and
// "B" is the activation side (rows m), so each lane ends with four consecutive
// output columns of one row and stores them as one 8-byte write.
//
// Every global access goes through a buffer descriptor sized to its operand:
// masked or out-of-range loads return zero and out-of-range stores are
// dropped by the hardware.
#include "lora_internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;          // K elements per LDS stage (128 bytes per tile row)
constexpr int ROW_BYTES = BK * 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // word3 0x00020000: raw 32-bit data, no swizzle (gfx9 family)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// One operand of a K-loop: rows of a row-major bf16 matrix whose reduction
// index is contiguous.  Tile row i is global row row0 + i; rows outside
// [lo, hi) read as zero.
struct Side {
  __amdgpu_buffer_rsrc_t res;
  uint32_t ld_bytes;
  int32_t row0, lo, hi;
};

// Tile shapes.  TN x TM output tile (TN weight rows, TM activation rows),
// WN x WM waves, each owning a (TN/WN) x (TM/WM) block of 32x32 MFMA tiles.
template <int TN_, int TM_, int WN_, int WM_>
struct Tile {
  static constexpr int TN = TN_, TM = TM_, WN = WN_, WM = WM_;
  static constexpr int NT = 64 * WN * WM;
  static constexpr int FN = TN / WN / 32;        // MFMA tiles per wave along n
  static constexpr int FM = TM / WM / 32;        // ... along m
  static constexpr int CN = TN * 8 / NT;         // 16-byte chunks per thread per stage, weight side
  static constexpr int CM = TM * 8 / NT;         // ... activation side
  static constexpr int STAGE = (TN + TM) * ROW_BYTES;
  static_assert(FN >= 1 && FM >= 1, "wave tile smaller than one MFMA tile");
  static_assert(TN * 8 % NT == 0 && TM * 8 % NT == 0, "tile rows must split evenly over threads");
};

// ------------------------------------------------------------------ staging
template <int ROWS, int NT>
__device__ __forceinline__ void load_rows(u32x4 (&v)[ROWS * 8 / NT], const Side& s, int k0, int kdim, int tid) {
#pragma unroll
  for (int i = 0; i < ROWS * 8 / NT; ++i) {
    const int q = tid + i * NT;
    const int r = q >> 3, c = q & 7;
    const int grow = s.row0 + r;
    const int kk = k0 + c * 8;
    const bool ok = grow >= s.lo && grow < s.hi && kk < kdim;
    const uint32_t off = ok ? uint32_t(grow) * s.ld_bytes + uint32_t(kk) * 2u : kMaskedOffset;
    v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(s.res, off, 0, 0));
  }
}

// Chunk c of tile row r lives at slot c ^ (r & 7): eight consecutive rows read
// at one chunk index land on eight distinct 16-byte slots.
__device__ __forceinline__ int lds_off(int r, int c) { return r * ROW_BYTES + ((c ^ (r & 7)) << 4); }

template <int ROWS, int NT>
__device__ __forceinline__ void store_rows(char* base, const u32x4 (&v)[ROWS * 8 / NT], int tid) {
#pragma unroll
  for (int i = 0; i < ROWS * 8 / NT; ++i) {
    const int q = tid + i * NT;
    *reinterpret_cast<u32x4*>(base + lds_off(q >> 3, q & 7)) = v[i];
  }
}

__device__ __forceinline__ bf16x8 read_frag(const char* base, int r, int c) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + lds_off(r, c)));
}

// acc += (weight tile) x (activation tile)^T over one 64-wide stage.
template <class C>
__device__ __forceinline__ void mma_stage(f32x16 (&acc)[C::FN][C::FM], const char* wt, const char* xt,
                                          int wrow, int xrow, int lane) {
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    const int c = 2 * s + (lane >> 5);
    bf16x8 a[C::FN], b[C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i) a[i] = read_frag(wt, wrow + i * 32 + (lane & 31), c);
#pragma unroll
    for (int j = 0; j < C::FM; ++j) b[j] = read_frag(xt, xrow + j * 32 + (lane & 31), c);
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Double-buffered K-loop over `ntiles` stages.  src(t, ws, xs, k0) names the
// weight-side and activation-side operands and the K offset of stage t.
template <class C, class Src>
__device__ __forceinline__ void k_loop(f32x16 (&acc)[C::FN][C::FM], int ntiles, int kdim, Src src,
                                       char* smem, int tid, int wn, int wm) {
  if (ntiles <= 0) return;
  const int lane = tid & 63;
  const int wrow = wn * (C::TN / C::WN), xrow = wm * (C::TM / C::WM);
  u32x4 wv[C::CN], xv[C::CM];
  {
    Side ws, xs;
    int k0;
    src(0, ws, xs, k0);
    load_rows<C::TN, C::NT>(wv, ws, k0, kdim, tid);
    load_rows<C::TM, C::NT>(xv, xs, k0, kdim, tid);
    store_rows<C::TN, C::NT>(smem, wv, tid);
    store_rows<C::TM, C::NT>(smem + C::TN * ROW_BYTES, xv, tid);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    char* cur = smem + (t & 1) * C::STAGE;
    const bool more = t + 1 < ntiles;
    if (more) {
      Side ws, xs;
      int k0;
      src(t + 1, ws, xs, k0);
      load_rows<C::TN, C::NT>(wv, ws, k0, kdim, tid);
      load_rows<C::TM, C::NT>(xv, xs, k0, kdim, tid);
    }
    mma_stage<C>(acc, cur, cur + C::TN * ROW_BYTES, wrow, xrow, lane);
    if (more) {
      char* nxt = smem + ((t + 1) & 1) * C::STAGE;
      store_rows<C::TN, C::NT>(nxt, wv, tid);
      store_rows<C::TM, C::NT>(nxt + C::TN * ROW_BYTES, xv, tid);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ scheduling
// Blocks are dispatched round-robin over the 8 XCDs, each with its own L2.
// Give each XCD a contiguous run of tiles, then walk those in groups of GM row
// tiles so that blocks running together share activation and weight slabs.
__device__ __forceinline__ void tile_of_block(int b, int ntn, int ntm, int& tn, int& tm) {
  constexpr int GM = 8;
  const int G = ntn * ntm;
  const int per = G / 8, rem = G % 8, x = b % 8, i = b / 8;
  const int L = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
  const int group = L / (GM * ntn);
  const int first = group * GM;
  const int gsz = min(ntm - first, GM);
  const int in = L - group * GM * ntn;
  tm = first + in % gsz;
  tn = in / gsz;
}

// First segment whose rows reach past row m (segments are non-empty and sorted).
__device__ __forceinline__ int first_segment(const SegTable& st, int m) {
  int lo = 0, hi = st.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (st.start[mid] <= m) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

__device__ __forceinline__ uint32_t pack2(float a, float b) { return bf16_bits(a) | (bf16_bits(b) << 16); }

// ------------------------------------------------------------------ shrink
// Grid: one block per (rank tile, row tile).  For every adapter segment that
// overlaps the block's rows: acc = A_a[rank tile] X[rows]^T, then
// T = s acc stored as bf16 hi and lo parts on the segment's rows only.
template <class C>
__global__ __launch_bounds__(C::NT) void shrink_kernel(ProjArgs p, SegTable st, AdapterTable at, int ntn, int ntm) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  int tn, tm;
  tile_of_block(blockIdx.x, ntn, ntm, tn, tm);
  const int j0 = tn * C::TN, m0 = tm * C::TM;
  const int m1 = min(m0 + C::TM, p.M);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;
  const auto xres = make_rsrc(p.X, p.x_bytes);
  const auto tres = make_rsrc(p.T, p.t_bytes);
  const uint32_t lo_base = uint32_t(p.M) * uint32_t(p.rank) * 2u;   // T_lo follows T_hi

  for (int g = first_segment(st, m0); g < st.n && st.start[g] < m1; ++g) {
    const int a = st.adapter[g];
    if (a < 0) continue;
    const int lo = max(st.start[g], m0), hi = min(st.start[g + 1], m1);
    const Side as{make_rsrc(at.A[a], p.a_bytes), uint32_t(p.K) * 2u, j0, 0, p.rank};
    const Side xs{xres, uint32_t(p.K) * 2u, m0, lo, hi};
    f32x16 acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};
    const int nk = (p.K + BK - 1) / BK;
    k_loop<C>(acc, nk, p.K,
              [&](int t, Side& ws, Side& xsd, int& k0) { ws = as; xsd = xs; k0 = t * BK; },
              smem, tid, wn, wm);
    // acc[i][j][r]: rank index j0 + wn*(TN/WN) + i*32 + (r/4)*8 + (lane/32)*4 + r%4,
    //               row m0 + wm*(TM/WM) + j*32 + lane%32
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int m = m0 + wm * (C::TM / C::WM) + j * 32 + (lane & 31);
      const bool row_ok = m >= lo && m < hi;
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jr = j0 + wn * (C::TN / C::WN) + i * 32 + q * 8 + (lane >> 5) * 4;
          float h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = p.scale * acc[i][j][q * 4 + e];
            const __bf16 hb = static_cast<__bf16>(t);
            h[e] = static_cast<float>(hb);
            l[e] = t - h[e];            // exact: t and bf16(t) share their leading bits
          }
          const uint32_t off = (row_ok && jr < p.rank) ? (uint32_t(m) * uint32_t(p.rank) + uint32_t(jr)) * 2u
                                                       : kMaskedOffset;
          const u32x2 hv{pack2(h[0], h[1]), pack2(h[2], h[3])};
          const u32x2 lv{pack2(l[0], l[1]), pack2(l[2], l[3])};
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, hv), tres, off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, lv), tres,
                                                off == kMaskedOffset ? kMaskedOffset : off + lo_base, 0, 0);
        }
    }
    __syncthreads();   // the next segment's K-loop reuses the LDS stages
  }
}

// ------------------------------------------------------------------ main
template <class C, bool F32_OUT>
__global__ __launch_bounds__(C::NT) void main_kernel(ProjArgs p, SegTable st, AdapterTable at, int has_adapter,
                                                     int ntn, int ntm) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  int tn, tm;
  tile_of_block(blockIdx.x, ntn, ntm, tn, tm);
  const int n0 = tn * C::TN, m0 = tm * C::TM;
  const int m1 = min(m0 + C::TM, p.M);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;

  f32x16 acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};

  // base product over K
  {
    const Side ws{make_rsrc(p.W, p.w_bytes), uint32_t(p.K) * 2u, n0, 0, p.N};
    const Side xs{make_rsrc(p.X, p.x_bytes), uint32_t(p.K) * 2u, m0, 0, p.M};
    const int nk = (p.K + BK - 1) / BK;
    k_loop<C>(acc, nk, p.K, [&](int t, Side& w, Side& x, int& k0) { w = ws; x = xs; k0 = t * BK; },
              smem, tid, wn, wm);
  }

  // expand: for each adapter segment overlapping the tile, stages alternate
  // T_hi and T_lo against the same 64-wide slab of B_a
  if (has_adapter) {
    const auto tres = make_rsrc(p.T, p.t_bytes);
    const uint32_t ld = uint32_t(p.rank) * 2u;
    const int lo_row0 = m0 + p.M;          // T_lo rows sit M rows after T_hi rows
    for (int g = first_segment(st, m0); g < st.n && st.start[g] < m1; ++g) {
      const int a = st.adapter[g];
      if (a < 0) continue;
      const int lo = max(st.start[g], m0), hi = min(st.start[g + 1], m1);
      const Side bs{make_rsrc(at.B[a], p.b_bytes), ld, n0, 0, p.N};
      const Side th{tres, ld, m0, lo, hi};
      const Side tl{tres, ld, lo_row0, lo + p.M, hi + p.M};
      const int nr = 2 * ((p.rank + BK - 1) / BK);
      k_loop<C>(acc, nr, p.rank,
                [&](int t, Side& w, Side& x, int& k0) { w = bs; x = (t & 1) ? tl : th; k0 = (t >> 1) * BK; },
                smem, tid, wn, wm);
    }
  }

  // epilogue: acc[i][j][r] is column n0 + wn*(TN/WN) + i*32 + (r/4)*8 + (lane/32)*4 + r%4
  // of row m0 + wm*(TM/WM) + j*32 + lane%32
  const auto yres = make_rsrc(p.Y, p.y_bytes);
  const bool vec = (p.N & 3) == 0;
#pragma unroll
  for (int j = 0; j < C::FM; ++j) {
    const int m = m0 + wm * (C::TM / C::WM) + j * 32 + (lane & 31);
    const bool row_ok = m < p.M;
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * (C::TN / C::WN) + i * 32 + q * 8 + (lane >> 5) * 4;
        const float v[4] = {acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]};
        const uint32_t e0 = uint32_t(m) * uint32_t(p.N) + uint32_t(n);
        if (vec) {
          const bool ok = row_ok && n < p.N;
          if constexpr (F32_OUT) {
            const u32x4 w{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                          __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
            __builtin_amdgcn_raw_buffer_store_b128(w, yres, ok ? e0 * 4u : kMaskedOffset, 0, 0);
          } else {
            const u32x2 w{pack2(v[0], v[1]), pack2(v[2], v[3])};
            __builtin_amdgcn_raw_buffer_store_b64(w, yres, ok ? e0 * 2u : kMaskedOffset, 0, 0);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = row_ok && n + e < p.N;
            if constexpr (F32_OUT) {
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[e]), yres,
                                                    ok ? (e0 + e) * 4u : kMaskedOffset, 0, 0);
            } else {
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(bf16_bits(v[e])), yres,
                                                    ok ? (e0 + e) * 2u : kMaskedOffset, 0, 0);
            }
          }
        }
      }
  }
}

// Tile choices.  Large M: 256x256 tiles, four waves of 128x128 (one wave per
// SIMD, 256 fp32 accumulators per lane, 128 KiB of LDS).  Small M (decode
// batches) and the shrink: smaller tiles so enough blocks exist to fill the CUs.
using MainBig = Tile<256, 256, 2, 2>;
using MainSmall = Tile<64, 64, 2, 2>;
using ShrinkBig = Tile<128, 128, 2, 2>;
using ShrinkSmall = Tile<64, 64, 2, 2>;

template <class C>
hipError_t launch_shrink_t(const ProjArgs& p, const SegTable& st, const AdapterTable& at, hipStream_t s) {
  const int ntn = (p.rank + C::TN - 1) / C::TN, ntm = (p.M + C::TM - 1) / C::TM;
  ProjArgs pa = p;
  SegTable sa = st;
  AdapterTable aa = at;
  int a0 = ntn, a1 = ntm;
  void* args[] = {&pa, &sa, &aa, &a0, &a1};
  return hipLaunchKernel(reinterpret_cast<const void*>(&shrink_kernel<C>), dim3(ntn * ntm), dim3(C::NT), args, 0, s);
}

template <class C, bool F32_OUT>
hipError_t launch_main_t(const ProjArgs& p, const SegTable& st, const AdapterTable& at, bool has_adapter,
                         hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int ntn = (p.N + C::TN - 1) / C::TN, ntm = (p.M + C::TM - 1) / C::TM;
  ProjArgs pa = p;
  SegTable sa = st;
  AdapterTable aa = at;
  int ha = has_adapter ? 1 : 0, a0 = ntn, a1 = ntm;
  void* args[] = {&pa, &sa, &aa, &ha, &a0, &a1};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(&main_kernel<C, F32_OUT>), dim3(ntn * ntm), dim3(C::NT),
                            args, 0, s, e0, e1, 0);
}

}  // namespace

hipError_t launch_bf16_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at, bool small_m,
                              hipStream_t stream) {
  return small_m ? launch_shrink_t<ShrinkSmall>(p, st, at, stream) : launch_shrink_t<ShrinkBig>(p, st, at, stream);
}

hipError_t launch_bf16_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at, bool has_adapter,
                            bool f32_out, bool small_m, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  if (small_m)
    return f32_out ? launch_main_t<MainSmall, true>(p, st, at, has_adapter, stream, e0, e1)
                   : launch_main_t<MainSmall, false>(p, st, at, has_adapter, stream, e0, e1);
  return f32_out ? launch_main_t<MainBig, true>(p, st, at, has_adapter, stream, e0, e1)
                 : launch_main_t<MainBig, false>(p, st, at, has_adapter, stream, e0, e1);
}

}  // namespace lora
