// Decode-path kernels of the mixed-adapter LoRA projection (M <= 128 rows).
//
// At decode sizes the call is bound by HBM: every byte of W, A_a and B_a is
// read once and reused only M times.  Three launches:
//
//   partial  One block per (64-row tile, K split) of W and of each used
//            adapter's A; every tile uses the same K split, so all blocks do
//            the same work.  A block streams its slab of W (or A) and the
//            matching K-range of X through an LDS ring in full 128-byte rows
//            (buffer_load ... lds) and multiplies on MFMA; fp32 partial sums go
//            to the workspace.
//   reduce   T = s * (sum of the A partials) on the rows of each adapter, zero
//            on other rows, stored as bf16 hi = bf16(T) and lo = bf16(T - hi).
//   finish   One block per 64 output columns: acc = sum of the W partials in
//            split order, acc += T_hi B_a^T + T_lo B_a^T on MFMA, one store.
//
// "Two 27B models on a single RTX 5090", section 4 request-path figure: the
// adapter's two thin matrices run only for requests that name it; base-only
// rows get T = 0 and therefore exactly their base sum.
#include <algorithm>

#include "lora_device.h"

namespace lora {

DecodeSplit decode_split(int64_t N, int64_t K) {
  DecodeSplit d;
  d.nstages = int((K + kDecodeStageK - 1) / kDecodeStageK);
  const int64_t ntiles = (N + kDecodeTile - 1) / kDecodeTile;
  int S = int((kDecodeTargetBlocks + ntiles / 2) / ntiles);
  S = std::max(1, std::min(S, d.nstages));
  d.sc = (d.nstages + S - 1) / S;
  d.S = (d.nstages + d.sc - 1) / d.sc;
  return d;
}

static size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t rank, int64_t n_used) {
  const DecodeSplit sp = decode_split(N, K);
  const size_t p = round256(size_t(sp.S) * size_t(M) * size_t(N) * 4);
  const size_t pt = round256(size_t(sp.S) * size_t(M) * size_t(n_used) * size_t(rank) * 4);
  const size_t t = round256(size_t(n_used) * size_t(M) * size_t(rank) * 2);
  return p + pt + 2 * t;
}

namespace {

constexpr int DTN = kDecodeTile;                 // W / A rows per partial tile; columns per finish tile
constexpr int DROW = kDecodeStageK * 2;          // bytes per tile row per stage: one full 128-byte line

// 16-byte chunk c of a 128-byte row r sits at slot c ^ ((r >> 1) & 7): the 16
// lanes a ds_read_b128 serves per cycle read one chunk of 16 consecutive rows,
// and the XOR spreads each parity's eight rows over eight slots, so the 64
// banks see no conflict.
__device__ __forceinline__ int doff(int r, int c) { return r * DROW + ((c ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ bf16x8 dfrag(const char* base, int r, int c) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + doff(r, c)));
}

// Partial-kernel geometry for TM activation rows (M <= TM).  The ring gets as
// many slots as fit in 80 KiB, so two blocks share a CU.
template <int TM_>
struct DGeo {
  static constexpr int TM = TM_;
  static constexpr int FM = TM / 32;
  static constexpr int STAGE = (DTN + TM) * DROW;
  static constexpr int NS = (80 * 1024) / STAGE;
  static constexpr int GROUPS = STAGE / 1024;    // 8-row groups, one wave-wide load each
  static constexpr int PW = GROUPS / 4;          // loads per wave per stage
  static_assert(GROUPS % 4 == 0 && NS >= 3, "stage must split over four waves and leave a 3-slot ring");
};

// Stage: DTN rows of the weight side (W or A) from wrow0, then TM rows of X
// from row 0, K elements [k0, k0 + 64).  Lane l of a group fills row l/8, slot
// l%8.  Rows past an operand's extent are not fetched.
template <class G>
__device__ __forceinline__ void d_issue(char* stage, const i32x4& wres, int wrow0, const i32x4& xres, uint32_t ld,
                                        int k0, int wave, int lane) {
  const uint32_t base = lds_addr(stage);
#pragma unroll
  for (int i = 0; i < G::PW; ++i) {
    const int g = wave * G::PW + i;
    const bool wside = g * 8 < DTN;
    const int r = g * 8 + (lane >> 3) - (wside ? 0 : DTN);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const uint32_t off = uint32_t((wside ? wrow0 : 0) + r) * ld + uint32_t(k0 + c * 8) * 2u;
    dma16(wside ? wres : xres, off, base + uint32_t(g) * 1024u);
  }
}

template <int PW, int NS>
__device__ __forceinline__ void d_wait(int after) {
  if (NS > 4 && after >= 3) wait_vm<PW * (NS > 4 ? 3 : 0)>();
  else if (NS > 3 && after >= 2) wait_vm<PW * (NS > 3 ? 2 : 0)>();
  else if (after >= 1) wait_vm<PW>();
  else wait_vm<0>();
}

// Blocks [0, n_used * n_atiles * S) are A tiles, the rest W tiles; block b of
// a kind takes split b % S of tile b / S.  All four waves load; waves 0 and 1
// multiply (32 weight rows each, all TM activation rows).
template <class G>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs d, AdapterTable at) {
  __shared__ __attribute__((aligned(1024))) char smem[G::NS * G::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int na = d.n_used * d.n_atiles * d.S;
  int b = blockIdx.x;
  const bool aside = b < na;
  if (!aside) b -= na;
  const int s = b % d.S;
  const int tile = b / d.S;
  int slot = 0, row0;
  i32x4 wres;
  if (aside) {
    row0 = (tile % d.n_atiles) * DTN;
    slot = tile / d.n_atiles;
    wres = make_rsrc_words(at.A[d.slot_adapter[slot]], d.a_bytes);
  } else {
    row0 = tile * DTN;
    wres = make_rsrc_words(d.W, d.w_bytes);
  }
  const int st0 = s * d.sc, st1 = min(st0 + d.sc, d.nstages);
  const i32x4 xres = make_rsrc_words(d.X, d.x_bytes);
  const uint32_t ld = uint32_t(d.K) * 2u;
  const int nt = st1 - st0;

  // Every tile of a split reads the same K-range of X; starting each tile at a
  // different stage of its range spreads those reads over many lines at once.
  const int rot = tile % nt;
  auto kof = [&](int t) { return (st0 + (t + rot) % nt) * kDecodeStageK; };

  f32x16 acc[G::FM];
#pragma unroll
  for (int j = 0; j < G::FM; ++j) acc[j] = f32x16{};
#pragma unroll
  for (int p = 0; p < G::NS - 1; ++p)
    if (p < nt) d_issue<G>(smem + p * G::STAGE, wres, row0, xres, ld, kof(p), wave, lane);
  for (int t = 0; t < nt; ++t) {
    d_wait<G::PW, G::NS>(min(G::NS - 2, nt - 1 - t));   // stage t has landed
    __syncthreads();
    if (t + G::NS - 1 < nt)             // refill the slot every wave finished reading in stage t-1
      d_issue<G>(smem + ((t + G::NS - 1) % G::NS) * G::STAGE, wres, row0, xres, ld, kof(t + G::NS - 1), wave,
                 lane);
    if (wave < 2) {
      const char* wt = smem + (t % G::NS) * G::STAGE;
      const char* xt = wt + DTN * DROW;
      const int k0 = kof(t);
#pragma unroll
      for (int sub = 0; sub < kDecodeStageK / 16; ++sub) {
        const int c = 2 * sub + (lane >> 5);
        bf16x8 a = dfrag(wt, wave * 32 + (lane & 31), c);
        bf16x8 bx[G::FM];
#pragma unroll
        for (int j = 0; j < G::FM; ++j) bx[j] = dfrag(xt, j * 32 + (lane & 31), c);
        if (k0 + kDecodeStageK > d.K && k0 + c * 8 >= d.K) {   // K tail: the first test is uniform
          a = bf16x8{};
#pragma unroll
          for (int j = 0; j < G::FM; ++j) bx[j] = bf16x8{};
        }
#pragma unroll
        for (int j = 0; j < G::FM; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bx[j], acc[j], 0, 0, 0);
      }
    }
  }
  if (wave >= 2) return;

  // acc[j][q*4+e]: weight row row0 + wave*32 + q*8 + (lane/32)*4 + e, activation row j*32 + lane%32
  const auto pres = make_rsrc(aside ? static_cast<void*>(d.PT) : static_cast<void*>(d.P),
                              aside ? d.pt_bytes : d.p_bytes);
  const int ncols = aside ? d.rank : d.N;
#pragma unroll
  for (int j = 0; j < G::FM; ++j) {
    const int m = j * 32 + (lane & 31);
    if (m >= d.M) continue;
    const uint32_t rowbase = aside ? uint32_t((s * d.M + m) * d.n_used + slot) * uint32_t(d.rank)
                                   : uint32_t(s * d.M + m) * uint32_t(d.N);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = row0 + wave * 32 + q * 8 + (lane >> 5) * 4;
      if (col + 3 < ncols) {
        const u32x4 v{__float_as_uint(acc[j][q * 4 + 0]), __float_as_uint(acc[j][q * 4 + 1]),
                      __float_as_uint(acc[j][q * 4 + 2]), __float_as_uint(acc[j][q * 4 + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, pres, (rowbase + uint32_t(col)) * 4u, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < ncols)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j][q * 4 + e]), pres,
                                                  (rowbase + uint32_t(col + e)) * 4u, 0, 0);
      }
    }
  }
}

// One thread per four consecutive rank entries of one (adapter slot, row).
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs d) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  const int per_row = d.rank / 4;
  const int total = d.n_used * d.M * per_row;
  if (q >= total) return;
  const int jr = (q % per_row) * 4;
  const int m = (q / per_row) % d.M;
  const int slot = q / (per_row * d.M);
  const auto ptres = make_rsrc(d.PT, d.pt_bytes);
  f32x4 t{0.f, 0.f, 0.f, 0.f};
  if (d.row_slot[m] == slot) {
    for (int s0 = 0; s0 < d.S; s0 += 4) {   // four splits in flight, summed in split order
      f32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = s0 + i;
        const uint32_t off = s < d.S ? ((uint32_t((s * d.M + m) * d.n_used + slot)) * uint32_t(d.rank) +
                                        uint32_t(jr)) * 4u
                                     : kMaskedOffset;
        v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ptres, off, 0, 0));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (s0 + i < d.S) t += v[i];
    }
  }
  float h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_hi_lo(d.scale * t[e], h[e], l[e]);
  const uint32_t o = (uint32_t(slot * d.M + m) * uint32_t(d.rank) + uint32_t(jr)) * 2u;
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(h[0], h[1]), pack2(h[2], h[3])}, make_rsrc(d.TH, d.t_bytes), o, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(l[0], l[1]), pack2(l[2], l[3])}, make_rsrc(d.TL, d.t_bytes), o, 0, 0);
}

// One wave-wide load of 8 rows x 128 bytes (elements [k0, k0 + 64) of rows
// row0 .. row0+7 of a matrix with row stride ld bytes) into rows lr0 .. lr0+7
// of a 128-byte-row LDS region, in the swizzled layout.
__device__ __forceinline__ void dma_rows8(const i32x4& res, int row0, uint32_t ld, int k0, char* region, int lr0,
                                          int lane) {
  const int r = lr0 + (lane >> 3);
  const int c = (lane & 7) ^ ((r >> 1) & 7);
  const uint32_t off = uint32_t(row0 + (lane >> 3)) * ld + uint32_t(k0 + c * 8) * 2u;
  dma16(res, off, lds_addr(region + lr0 * DROW));
}

// Waves: wn picks 32 of the 64 output columns, wm 64 of the TM rows (FM tiles).
// All pieces of T and B for up to 256 rank entries arrive by DMA while the W
// partials are summed, so the block waits on memory about twice in all.
template <int TM, bool F32_OUT>
__global__ __launch_bounds__(256) void decode_finish_kernel(DecodeArgs d, AdapterTable at) {
  constexpr int FMW = TM / 64 > 0 ? (TM / 2) / 32 : 1;    // tiles of 32 rows per wave along m
  constexpr int PIECE_T = TM * DROW, PIECE_B = DTN * DROW;
  __shared__ __attribute__((aligned(1024))) char smem[4 * (2 * PIECE_T + PIECE_B)];
  char* thi = smem;                     // [piece][TM rows][128 B]
  char* tlo = smem + 4 * PIECE_T;
  char* bp = smem + 8 * PIECE_T;        // [piece][64 rows][128 B]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int n0 = blockIdx.x * DTN;
  const uint32_t tld = uint32_t(d.rank) * 2u;

  // DMA of the T rows of one adapter slot and of B_a, rank entries [r0, r0 + 64*np)
  auto fetch = [&](int slot, int r0, int np) {
    const i32x4 thr = make_rsrc_words(d.TH, d.t_bytes), tlr = make_rsrc_words(d.TL, d.t_bytes);
    const i32x4 br = make_rsrc_words(at.B[d.slot_adapter[slot]], d.b_bytes);
    const int tg = TM / 8, groups = np * (2 * tg + DTN / 8);
    for (int g = wave; g < groups; g += 4) {    // 8-row groups, round-robin over the waves
      const int piece = g / (2 * tg + DTN / 8), w = g % (2 * tg + DTN / 8);
      const int k0 = r0 + piece * 64;
      if (w < tg) dma_rows8(thr, slot * d.M + w * 8, tld, k0, thi + piece * PIECE_T, w * 8, lane);
      else if (w < 2 * tg) dma_rows8(tlr, slot * d.M + (w - tg) * 8, tld, k0, tlo + piece * PIECE_T, (w - tg) * 8, lane);
      else dma_rows8(br, n0 + (w - 2 * tg) * 8, tld, k0, bp + piece * PIECE_B, (w - 2 * tg) * 8, lane);
    }
  };
  const bool expand = d.n_used > 0;
  if (expand) fetch(0, 0, min(4, (d.rank + 63) / 64));

  // acc = sum of the W partials, in split order, four splits in flight
  f32x16 acc[FMW];
#pragma unroll
  for (int j = 0; j < FMW; ++j) acc[j] = f32x16{};
  const auto pres = make_rsrc(d.P, d.p_bytes);
  for (int s0 = 0; s0 < d.S; s0 += 4) {
    f32x4 v[4][FMW][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FMW; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int s = s0 + i, m = wm * (TM / 2) + j * 32 + (lane & 31);
          const int n = n0 + wn * 32 + q * 8 + (lane >> 5) * 4;
          const uint32_t off = (s < d.S && m < d.M) ? (uint32_t(s * d.M + m) * uint32_t(d.N) + uint32_t(n)) * 4u
                                                    : kMaskedOffset;
          v[i][j][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pres, off, 0, 0));
        }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (s0 + i < d.S) {
#pragma unroll
        for (int j = 0; j < FMW; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][q * 4 + e] += v[i][j][q][e];
      }
  }

  // expand: acc += T_hi B_a^T + T_lo B_a^T, 256 rank entries per round
  if (expand) {
    for (int slot = 0; slot < d.n_used; ++slot) {
      for (int r0 = 0; r0 < d.rank; r0 += 256) {
        const int np = min(4, (d.rank - r0 + 63) / 64);
        if (slot > 0 || r0 > 0) {
          __syncthreads();             // every wave is done with the previous round's pieces
          fetch(slot, r0, np);
        }
        wait_vm<0>();
        __syncthreads();
        for (int piece = 0; piece < np; ++piece) {
#pragma unroll
          for (int sub = 0; sub < 4; ++sub) {
            const int c = 2 * sub + (lane >> 5);
            bf16x8 a = dfrag(bp + piece * PIECE_B, wn * 32 + (lane & 31), c);
            const bool past = r0 + piece * 64 + c * 8 >= d.rank;    // rank tail
            if (past) a = bf16x8{};
#pragma unroll
            for (int j = 0; j < FMW; ++j) {
              const int r = wm * (TM / 2) + j * 32 + (lane & 31);
              bf16x8 h = dfrag(thi + piece * PIECE_T, r, c), l = dfrag(tlo + piece * PIECE_T, r, c);
              if (past) h = l = bf16x8{};
              acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, h, acc[j], 0, 0, 0);
              acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, l, acc[j], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  // store: acc[j][q*4+e] is column n0 + wn*32 + q*8 + (lane/32)*4 + e of row wm*TM/2 + j*32 + lane%32
  const auto yres = make_rsrc(d.Y, d.y_bytes);
  const bool vec = (d.N & 3) == 0;
#pragma unroll
  for (int j = 0; j < FMW; ++j) {
    const int m = wm * (TM / 2) + j * 32 + (lane & 31);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + wn * 32 + q * 8 + (lane >> 5) * 4;
      const uint32_t e0 = uint32_t(m) * uint32_t(d.N) + uint32_t(n);
      if (vec) {
        const bool ok = m < d.M && n < d.N;
        if constexpr (F32_OUT) {
          const u32x4 w{__float_as_uint(acc[j][q * 4 + 0]), __float_as_uint(acc[j][q * 4 + 1]),
                        __float_as_uint(acc[j][q * 4 + 2]), __float_as_uint(acc[j][q * 4 + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(w, yres, ok ? e0 * 4u : kMaskedOffset, 0, 0);
        } else {
          const u32x2 w{pack2(acc[j][q * 4 + 0], acc[j][q * 4 + 1]), pack2(acc[j][q * 4 + 2], acc[j][q * 4 + 3])};
          __builtin_amdgcn_raw_buffer_store_b64(w, yres, ok ? e0 * 2u : kMaskedOffset, 0, 0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = m < d.M && n + e < d.N;
          if constexpr (F32_OUT)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j][q * 4 + e]), yres,
                                                  ok ? (e0 + e) * 4u : kMaskedOffset, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16(uint16_t(bf16_bits(acc[j][q * 4 + e])), yres,
                                                  ok ? (e0 + e) * 2u : kMaskedOffset, 0, 0);
        }
      }
    }
  }
}

using DGeo96 = DGeo<96>;
using DGeo128 = DGeo<128>;

}  // namespace

hipError_t launch_decode(const DecodeArgs& d, const AdapterTable& at, bool f32_out, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
  DecodeArgs da = d;
  AdapterTable aa = at;
  void* args[] = {&da, &aa};
  const int nblk = (d.n_used * d.n_atiles + d.n_wtiles) * d.S;
  const void* part = d.M <= 96 ? reinterpret_cast<const void*>(&decode_partial_kernel<DGeo96>)
                               : reinterpret_cast<const void*>(&decode_partial_kernel<DGeo128>);
  hipError_t e = hipExtLaunchKernel(part, dim3(nblk), dim3(256), args, 0, stream, ev_start, nullptr, 0);
  if (e != hipSuccess) return e;
  if (d.n_used > 0) {
    void* rargs[] = {&da};
    const int nr = (d.n_used * d.M * (d.rank / 4) + 255) / 256;
    e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_reduce_kernel), dim3(nr), dim3(256), rargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  const void* fin;
  if (d.M <= 64)
    fin = f32_out ? reinterpret_cast<const void*>(&decode_finish_kernel<64, true>)
                  : reinterpret_cast<const void*>(&decode_finish_kernel<64, false>);
  else
    fin = f32_out ? reinterpret_cast<const void*>(&decode_finish_kernel<128, true>)
                  : reinterpret_cast<const void*>(&decode_finish_kernel<128, false>);
  return hipExtLaunchKernel(fin, dim3(d.n_wtiles), dim3(256), args, 0, stream, nullptr, ev_stop, 0);
}

}  // namespace lora
