// bf16 kernels of the mixed-adapter LoRA projection for gfx950 (CDNA4).
//
// Two launches per call ("two 27B models on a single RTX 5090", section 4
// request-path figure: each changed matrix runs the base product plus the
// adapter's two thin matrices, for adapter requests only):
//
//   shrink  T = s_a X_a A_a^T on the rows of adapter segments (s_a the scale of
//           adapter a).  T is stored as
//           two bf16 halves, hi = bf16(T) and lo = bf16(T - hi), so the expand
//           can run on bf16 MFMA while keeping T to about 2^-17 relative.
//           When its tile grid is small the shrink splits K over several
//           blocks per tile, and a third launch sums their partials.
//   main    per output tile: acc = X W^T over K, then, if the tile holds adapter
//           rows, acc += T_hi B_a^T + T_lo B_a^T over the rank (rows of other
//           segments read as zero), then one round-to-nearest-even store.
//
// Both run MFMA K-loops over a ring of LDS stages: slabs of 64 elements of K
// (one whole 128-byte line per row), loaded 16 bytes per lane into registers a
// stage or two ahead and written to the ring with ds_write_b128 (the expand
// loads straight into LDS with buffer_load ... lds).  An XOR swizzle on
// 16-byte chunks keeps the ds_read_b128 fragment reads conflict-free, and
// v_mfma_f32_32x32x16_bf16 accumulates in fp32.  The main kernel runs four
// waves of 128 x 128 that keep their accumulators in AGPRs.  The MFMA "A"
// operand is the weight side (rows n) and "B" is the activation side (rows m),
// so each lane ends with four consecutive output columns of one row and
// stores them as one 8-byte write.
//
// Every global access goes through a buffer descriptor sized to its operand:
// masked or out-of-range loads return zero and out-of-range stores are
// dropped by the hardware.
#include "lora_device.h"

#include <type_traits>

namespace lora {
namespace {

// K elements per LDS stage: 128 bytes per tile row, so every row of a stage is
// one whole cache line and each load request fetches a full line (with 64-byte
// rows the same bytes took twice the requests and moved about a quarter less
// per CU per cycle).
constexpr int BK = 64;
constexpr int ROW_BYTES = BK * 2;

// One operand of a K-loop: rows of a row-major bf16 matrix whose reduction
// index is contiguous.  Tile row i is global row row0 + i; rows past the
// operand's extent (its descriptor's size) load as zeros.
struct Side {
  i32x4 res;
  uint32_t ld_bytes;
  int32_t row0;
};

// Tile shapes.  TN x TM output tile (TN weight rows, TM activation rows),
// WN x WM waves, each owning a (TN/WN) x (TM/WM) block of 32x32 MFMA tiles.
template <int TN_, int TM_, int WN_, int WM_>
struct Tile {
  static constexpr int TN = TN_, TM = TM_, WN = WN_, WM = WM_;
  static constexpr int NW = WN * WM;
  static constexpr int NT = 64 * NW;
  static constexpr int FN = TN / WN / 32;        // MFMA tiles per wave along n
  static constexpr int FM = TM / WM / 32;        // ... along m
  static constexpr int STAGE = (TN + TM) * ROW_BYTES;
  static constexpr int GROUPS = STAGE / 1024;    // 8-row groups: one wave-wide 16-byte load each
  static constexpr int PW = GROUPS / NW;         // loads per wave per stage
  static_assert(FN >= 1 && FM >= 1, "wave tile smaller than one MFMA tile");
  static_assert(TN % 16 == 0 && TM % 16 == 0 && GROUPS % NW == 0, "row groups must split evenly over waves");
};

// 16-byte chunk c of 128-byte row r sits at slot c ^ ((r >> 1) & 7).  The
// LDS has 64 four-byte banks and serves 16 lanes of a ds_read_b128 per cycle;
// those lanes read one chunk of 16 consecutive rows, which the XOR spreads over
// all 64 banks.
__device__ __forceinline__ int lds_off(int r, int c) { return r * ROW_BYTES + ((c ^ ((r >> 1) & 7)) << 4); }

constexpr uint32_t kGatherMasked = 0x80001000u;

// The shrink's activation-side load offsets for this lane, from the row map
// xrows (LDS, -1 for none): row * ld + the lane's swizzled chunk, the same for
// every stage.  A row with no X row behind it starts at kGatherMasked, past
// every operand (each under 2 GiB), so it loads zeros; with more than 128 rows
// a row of X is under 17 MB, so adding the K offset cannot wrap.  (A compare
// and select per load cost 0.6% of a 16k call.)
template <class C>
__device__ __forceinline__ void gather_offsets(uint32_t (&gx)[C::PW], const int* xrows, uint32_t ld_bytes, int wave,
                                               int lane) {
  const int g0 = wave * C::PW;
#pragma unroll
  for (int i = 0; i < C::PW; ++i) {
    const int r = (g0 + i) * 8 + (lane >> 3) - C::TN;
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int row = r >= 0 ? xrows[r] : -1;
    gx[i] = row >= 0 ? uint32_t(row) * ld_bytes + uint32_t(c) * 16u : kGatherMasked;
  }
}

__device__ __forceinline__ bf16x8 read_frag(const char* base, int r, int c) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + lds_off(r, c)));
}

// Register-staged K-loop of the shrink: a ring of two LDS slots, each lane's 8
// loads of a stage in VGPRs two stages ahead (two register sets).  In stage t
// the wave writes stage t+1 (set (t+1) & 1) into the other slot and loads
// stage t+3 into the same registers, two load pairs per substep; one barrier
// ends the stage.  The activation side's offsets come from the row map
// (gather_offsets).  The loads of stages past the last bring data that no
// stage reads: at an offset past the operands, or, for a row with no X row
// behind it, one that wraps to an offset inside X.
template <class C, class Src>
__device__ __forceinline__ void k_loop_small_reg(f32x16 (&acc)[C::FN][C::FM], int ntiles, int ntail, int kdim,
                                                 Src src, char* smem, int tid, int wn, int wm, const int* xrows) {
  static_assert(C::PW == 8 && C::FN * C::FM == 4, "128 x 128 tiles of four waves");
  if (ntiles <= 0) return;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wrow = wn * (C::TN / C::WN), xrow = wm * (C::TM / C::WM);
  const int g0 = wave * C::PW;
  const bool wside = g0 * 8 < C::TN;
  uint32_t lb[C::PW];
  __amdgpu_buffer_rsrc_t res;
  {
    Side ws, xs;
    int k0;
    src(0, ws, xs, k0);
    if (wside) {
#pragma unroll
      for (int k = 0; k < C::PW; ++k) {
        const int r = (g0 + k) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        lb[k] = uint32_t(ws.row0 + r) * ws.ld_bytes + uint32_t(c) * 16u;
      }
    } else {
      gather_offsets<C>(lb, xrows, xs.ld_bytes, wave, lane);
    }
    res = rsrc_of_words(wside ? ws.res : xs.res);
  }
  // stage t's uniform offset; past the last stage kMaskedOffset (the data is
  // never used)
  auto add = [&](int t) __attribute__((always_inline)) {
    Side ws, xs;
    int k0;
    src(t < ntiles ? t : 0, ws, xs, k0);
    return t < ntiles ? uint32_t(k0) * 2u : kMaskedOffset;
  };
  u32x4 stg[2][C::PW];
  const uint32_t wofs = uint32_t(g0) * 1024u + uint32_t(lane) * 16u;
  auto gload = [&](int set, int k, uint32_t a) __attribute__((always_inline)) {
    stg[set][k] = __builtin_amdgcn_raw_buffer_load_b128(res, lb[k] + a, 0, 0);
  };
  auto lwrite = [&](int set, int k, char* slot) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4*>(slot + wofs + k * 1024) = stg[set][k];
  };
  auto lds_sync = []() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  };
  {
    const uint32_t a0 = add(0), a1 = add(1), a2 = add(2);
#pragma unroll
    for (int k = 0; k < C::PW; ++k) gload(0, k, a0);
#pragma unroll
    for (int k = 0; k < C::PW; ++k) gload(1, k, a1);
#pragma unroll
    for (int k = 0; k < C::PW; ++k) {
      lwrite(0, k, smem);
      gload(0, k, a2);
    }
    lds_sync();
  }
  auto stage = [&](int t, auto tailc, auto par) __attribute__((always_inline)) {
    constexpr bool TAIL = decltype(tailc)::value;
    constexpr int P = decltype(par)::value;   // t & 1
    constexpr int SET = P ^ 1;                // registers of stage t+1
    Side ws, xs;
    int k0;
    src(t, ws, xs, k0);
    const uint32_t a3 = add(t + 3);
    const char* cur = smem + P * C::STAGE;
    char* const nxt = smem + (P ^ 1) * C::STAGE;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = 2 * s + (lane >> 5);
      bf16x8 fa[C::FN], fb[C::FM];
#pragma unroll
      for (int i = 0; i < C::FN; ++i) fa[i] = read_frag(cur, wrow + i * 32 + (lane & 31), c);
#pragma unroll
      for (int j = 0; j < C::FM; ++j) fb[j] = read_frag(cur + C::TN * ROW_BYTES, xrow + j * 32 + (lane & 31), c);
      if constexpr (TAIL) {
        if (k0 + c * 8 >= kdim) {
#pragma unroll
          for (int i = 0; i < C::FN; ++i) fa[i] = bf16x8{};
#pragma unroll
          for (int j = 0; j < C::FM; ++j) fb[j] = bf16x8{};
        }
      }
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0], fb[0], acc[0][0], 0, 0, 0);
      lwrite(SET, 2 * s, nxt);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0], fb[1], acc[0][1], 0, 0, 0);
      gload(SET, 2 * s, a3);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1], fb[0], acc[1][0], 0, 0, 0);
      lwrite(SET, 2 * s + 1, nxt);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1], fb[1], acc[1][1], 0, 0, 0);
      gload(SET, 2 * s + 1, a3);
    }
    lds_sync();   // stage t+1 is in its slot; no wave reads stage t's any more
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int t = 0;
  for (; t + 1 < ntail; t += 2) {
    stage(t, std::false_type{}, P0{});
    stage(t + 1, std::false_type{}, P1{});
  }
  for (; t + 1 < ntiles; t += 2) {
    stage(t, std::true_type{}, P0{});
    stage(t + 1, std::true_type{}, P1{});
  }
  if (t < ntiles) stage(t, std::true_type{}, P0{});
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
}

// ------------------------------------------------------------------ output K-loop
// Four waves, one per SIMD, each owning a 128 x 128 block of the 256 x 256
// tile: 16 MFMA tiles whose 256 accumulators per lane live in AGPRs (a wave
// alone on its SIMD may use 512 registers).  Per k16 substep a wave reads 4 + 4
// fragments for 16 MFMAs, a third less LDS reading per MFMA than waves of
// 128 x 64.  The ring holds two 64 KiB stages of BK = 64.
//
// A stage is four substeps of 16 MFMAs, each with the next substep's 8
// fragment reads among its MFMAs, and one barrier, after the first 4 MFMAs of
// substep 3 (stage t+1 is in its slot; no wave still reads stage t's).
//
// Loads go through registers.  Waves 0 and 1 load the weight rows, waves 2
// and 3 the activation rows: 16 (or, on the activation side of a shorter
// tile, 12 or 8) 16-byte loads per lane and stage, each one 8-row group of
// whole 128-byte lines.  Each load has a fixed chunk of the stage (four MFMAs),
// where the wave writes the register into the free ring slot (ds_write_b128)
// and loads it again, one stage ahead.  Chunks before the barrier write stage
// t+1 into the other slot and load stage t+2; the three after it write stage
// t+2 into stage t's slot and load stage t+3.  Every load has one stage to land,
// no load waits on a slot, and the loads spread evenly over the MFMA stream.
template <class C>
struct WideRing {
  static constexpr int STAGE = C::STAGE;        // 64 KiB for 256 x 256
  static constexpr int PWW = C::TN / 16, PWX = C::TM / 16;   // loads per lane and stage
  static_assert(C::NW == 4 && PWW == 16 && PWX >= 8 && PWX <= 16, "one load per chunk at most");
  // chunk (4 substep + chunk of substep) of load k of NL, and load of a chunk
  static constexpr int pos(int k, int nl) { return k * 16 / nl; }
  static constexpr int load_at(int p, int nl) {
    for (int k = 0; k < nl; ++k)
      if (pos(k, nl) == p) return k;
    return -1;
  }
  static constexpr int BARRIER = 12;            // chunk 0 of substep 3
};

// K-loop over `ntiles` stages; src(t, ws, xs, k0) names the operands and K
// offset of stage t, with each side's row stride the same in every stage.
// Chunks at or past kdim enter the MFMAs as zero; with MASK_ROWS so do the
// activation rows whose bit in `keep` is clear.
template <class C, bool MASK_ROWS, class Src>
__device__ __forceinline__ void k_loop_wide(f32x16 (&acc)[C::FN][C::FM], int ntiles, int kdim, Src src, char* smem,
                                            int tid, int wn, int wm, uint32_t keep = 0) {
  static_assert(C::NW == 4 && C::FN == 4 && C::FM >= 2 && C::FM <= 4, "four waves of 128 x (64, 96 or 128)");
  using R = WideRing<C>;
  if (ntiles <= 0) return;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wrow = wn * (C::TN / C::WN), xrow = wm * (C::TM / C::WM);
  const int rl = lane & 31, ch = lane >> 5;
  const bool wside = wave < 2;

  bf16x8 fa[2][C::FN], fb[2][C::FM];
  // chunks at or past kdim and masked activation rows enter as zero
  auto fix = [&](int k0, int s, int buf) __attribute__((always_inline)) {
    if (k0 + (2 * s + ch) * 8 >= kdim) {
#pragma unroll
      for (int i = 0; i < C::FN; ++i) fa[buf][i] = bf16x8{};
#pragma unroll
      for (int j = 0; j < C::FM; ++j) fb[buf][j] = bf16x8{};
    }
    if constexpr (MASK_ROWS) {
#pragma unroll
      for (int j = 0; j < C::FM; ++j)
        if (!((keep >> j) & 1u)) fb[buf][j] = bf16x8{};
    }
  };
  auto mfma = [&](int buf, int i, int j) __attribute__((always_inline)) {
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };
  auto lds_sync = []() __attribute__((always_inline)) {   // own LDS writes done, then meet
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  };

  // The waves of each side run the loop with their own number of loads, so
  // that no load sits under a run-time branch (the compiler's wait counts for
  // the staged registers stay exact).
  auto body = [&](auto nlc) __attribute__((always_inline)) {
    constexpr int NL = decltype(nlc)::value;
    const int q0 = wside ? wave * R::PWW : C::TN / 8 + (wave - 2) * R::PWX;   // first 8-row group of the wave
    // each lane's offset within a stage: row of its side, swizzled chunk
    uint32_t lb[NL];
    {
      Side w, x;
      int k0;
      src(0, w, x, k0);
      const uint32_t ld = wside ? w.ld_bytes : x.ld_bytes;
#pragma unroll
      for (int q = 0; q < NL; ++q) {
        const int r = (q0 + q) * 8 + (lane >> 3) - (wside ? 0 : C::TN);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        lb[q] = uint32_t(r) * ld + uint32_t(c) * 16u;
      }
    }
    struct Stage {
      __amdgpu_buffer_rsrc_t res;
      uint32_t add;
    };
    // stage t's operand and uniform offset; past the last stage an offset
    // beyond every operand, so the loads return zeros and move no data
    auto stage = [&](int t) __attribute__((always_inline)) {
      Side w, x;
      int k0;
      src(t < ntiles ? t : ntiles - 1, w, x, k0);
      const Side& sd = wside ? w : x;
      return Stage{rsrc_of_words(sd.res), t < ntiles ? uint32_t(sd.row0) * sd.ld_bytes + uint32_t(k0) * 2u : kMaskedOffset};
    };
    u32x4 stg[NL];
    const uint32_t wofs = uint32_t(q0) * 1024u + uint32_t(lane) * 16u;
    auto gload = [&](int k, const Stage& g) __attribute__((always_inline)) {
      stg[k] = __builtin_amdgcn_raw_buffer_load_b128(g.res, lb[k] + g.add, 0, 0);
    };
    auto lwrite = [&](int k, char* slot) __attribute__((always_inline)) {
      *reinterpret_cast<u32x4*>(slot + wofs + k * 1024) = stg[k];
    };
    // prologue: stage 0 in slot 0; stage 1 in registers, the loads after the
    // barrier already written to slot 1 and holding stage 2
    {
      const Stage g0 = stage(0);
#pragma unroll
      for (int k = 0; k < NL; ++k) gload(k, g0);
#pragma unroll
      for (int k = 0; k < NL; ++k) lwrite(k, smem);
      const Stage g1 = stage(1), g2 = stage(2);
#pragma unroll
      for (int k = 0; k < NL; ++k) gload(k, g1);
#pragma unroll
      for (int k = 0; k < NL; ++k)
        if (R::pos(k, NL) > R::BARRIER) {
          lwrite(k, smem + R::STAGE);
          gload(k, g2);
        }
      lds_sync();
    }
#pragma unroll
    for (int i = 0; i < C::FN; ++i) fa[0][i] = read_frag(smem, wrow + i * 32 + rl, ch);
#pragma unroll
    for (int j = 0; j < C::FM; ++j) fb[0][j] = read_frag(smem + C::TN * ROW_BYTES, xrow + j * 32 + rl, ch);

    auto iter = [&](int t, auto checked, auto parity) __attribute__((always_inline)) {
      constexpr bool CHECKED = decltype(checked)::value;
      constexpr int P = decltype(parity)::value;   // t & 1
      int k0 = 0;
      if constexpr (CHECKED) {
        Side w, x;
        src(t, w, x, k0);
      }
      const Stage g2 = stage(t + 2), g3 = stage(t + 3);
      char* const other = smem + (P ^ 1) * R::STAGE;
      char* const mine = smem + P * R::STAGE;
      auto substep = [&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        constexpr int buf = s & 1, ns = s < 3 ? s + 1 : 0, nb = (s + 1) & 1;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (CHECKED) fix(k0, s, buf);
        // the next substep's fragments: this stage's, or stage t+1's first (past
        // the last stage a stale slot, never used)
        const char* nx = smem + ((s < 3 ? P : P + 1) & 1) * R::STAGE;
        auto chunk = [&](auto gc) __attribute__((always_inline)) {
          constexpr int g = decltype(gc)::value;
          constexpr int p = 4 * s + g;
          constexpr int k = R::load_at(p, NL);
          constexpr bool LOAD = k >= 0;
          constexpr int kk = LOAD ? k : 0;
          auto pair_write = [&]() __attribute__((always_inline)) {
            if constexpr (LOAD) lwrite(kk, p > R::BARRIER ? mine : other);
          };
          auto pair_load = [&]() __attribute__((always_inline)) {
            if constexpr (LOAD) gload(kk, p > R::BARRIER ? g3 : g2);
          };
          if constexpr (p == R::BARRIER) {
            mfma(buf, 0, 0);
            pair_write();
            mfma(buf, 0, 1);
            pair_load();
#pragma unroll
            for (int j = 2; j < C::FM; ++j) mfma(buf, 0, j);
            __builtin_amdgcn_sched_barrier(0);
            lds_sync();   // stage t+1 is in its slot; no wave reads stage t's any more
            __builtin_amdgcn_sched_barrier(0);
            fa[nb][0] = read_frag(nx, wrow + rl, 2 * ns + ch);
            fb[nb][0] = read_frag(nx + C::TN * ROW_BYTES, xrow + rl, 2 * ns + ch);
            __builtin_amdgcn_sched_barrier(0);
            return;
          }
          // the chunk's MFMAs (one row block against the wave's FM column
          // blocks), a fragment read of the next substep after each of the
          // first two, and the chunk's load pair
          constexpr bool XREAD = g < C::FM;
          mfma(buf, g, 0);
          fa[nb][g] = read_frag(nx, wrow + g * 32 + rl, 2 * ns + ch);
          mfma(buf, g, 1);
          if constexpr (XREAD) fb[nb][g] = read_frag(nx + C::TN * ROW_BYTES, xrow + g * 32 + rl, 2 * ns + ch);
          if constexpr (C::FM > 2) mfma(buf, g, 2);
          pair_write();
          if constexpr (C::FM > 3) mfma(buf, g, 3);
          pair_load();
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if constexpr (XREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if constexpr (C::FM > 2) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if constexpr (LOAD) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS write
          if constexpr (C::FM > 3) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if constexpr (LOAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
          __builtin_amdgcn_sched_barrier(0);
        };
        chunk(std::integral_constant<int, 0>{});
        chunk(std::integral_constant<int, 1>{});
        chunk(std::integral_constant<int, 2>{});
        chunk(std::integral_constant<int, 3>{});
      };
      substep(std::integral_constant<int, 0>{});
      substep(std::integral_constant<int, 1>{});
      substep(std::integral_constant<int, 2>{});
      substep(std::integral_constant<int, 3>{});
    };
    // Stages go in pairs, so that the ring slot a fragment read addresses is a
    // compile-time constant (its address then needs no per-stage arithmetic).
    // The K tail can only fall in the last stage of the base product; the
    // expand (MASK_ROWS) checks every stage.
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int t = 0;
    if constexpr (!MASK_ROWS) {
      for (; t + 2 < ntiles; t += 2) {
        iter(t, std::false_type{}, P0{});
        iter(t + 1, std::false_type{}, P1{});
      }
    }
    for (; t + 1 < ntiles; t += 2) {
      iter(t, std::true_type{}, P0{});
      iter(t + 1, std::true_type{}, P1{});
    }
    if (t < ntiles) iter(t, std::true_type{}, P0{});
  };
  if constexpr (R::PWX == R::PWW) {
    body(std::integral_constant<int, R::PWW>{});
  } else {
    if (wside) body(std::integral_constant<int, R::PWW>{});
    else body(std::integral_constant<int, R::PWX>{});
  }
  // the loads past the last stage (zeros) and the last writes are done before
  // the ring is reused by whatever runs next
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
}

// The same K-loop with the loads written straight into LDS (buffer_load ...
// lds), for the expand: its few stages, with the row masks and a per-adapter
// operand per call, would push the register-staged loop into spills.  A wave's
// 16 (or 12, 8) loads of a stage go out in groups of four under one M0 value:
// groups 0 and 1 of stage t+2 right after the barrier in substep 3 of stage t,
// groups 2 and 3 in substep 0 of stage t+1, after its 12th and 16th MFMA.
template <class C, bool MASK_ROWS, class Src>
__device__ __forceinline__ void k_loop_wide_dma(f32x16 (&acc)[C::FN][C::FM], int ntiles, int kdim, Src src,
                                                char* smem, int tid, int wn, int wm, uint32_t keep = 0) {
  static_assert(C::NW == 4 && C::FN == 4 && C::FM >= 2 && C::FM <= 4, "four waves of 128 x (64, 96 or 128)");
  using R = WideRing<C>;
  static_assert(R::PWX % 4 == 0, "load groups of four");
  if (ntiles <= 0) return;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wrow = wn * (C::TN / C::WN), xrow = wm * (C::TM / C::WM);

  // Waves 0 and 1 load the weight rows, waves 2 and 3 the activation rows.
  // Each lane's offsets within a stage (row in the tile, swizzled chunk, group
  // bias) are fixed; a stage adds the uniform row0 * stride + 2 k0.
  const bool wside = wave < 2;
  const int q0 = wside ? wave * R::PWW : C::TN / 8 + (wave - 2) * R::PWX;   // first 8-row load of the wave
  const int ngroups = wside ? R::PWW / 4 : R::PWX / 4;
  uint32_t lb[R::PWW];
  {
    Side w, x;
    int k0;
    src(0, w, x, k0);
    const uint32_t ld = wside ? w.ld_bytes : x.ld_bytes;
#pragma unroll
    for (int q = 0; q < R::PWW; ++q) {   // past the activation side's loads: never used
      const int r = (q0 + q) * 8 + (lane >> 3) - (wside ? 0 : C::TN);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      lb[q] = uint32_t(r) * ld + uint32_t(c) * 16u - 1024u * uint32_t(q & 3);
    }
  }
  struct Dest {   // where a stage's loads go
    i32x4 res;
    uint32_t add;
    char* slot;
  };
  auto dest = [&](int t) __attribute__((always_inline)) {
    Side w, x;
    int k0;
    src(t, w, x, k0);
    const Side& sd = wside ? w : x;
    return Dest{sd.res, uint32_t(sd.row0) * sd.ld_bytes + uint32_t(k0) * 2u, smem + (t & 1) * R::STAGE};
  };
  auto group = [&](const Dest& d, int g) __attribute__((always_inline)) {
    dma16x4_biased(d.res, lb[4 * g] + d.add, lb[4 * g + 1] + d.add, lb[4 * g + 2] + d.add, lb[4 * g + 3] + d.add,
                   lds_addr(d.slot) + uint32_t(q0 + 4 * g) * 1024u);
  };
  {
    const Dest d0 = dest(0);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (g < ngroups) group(d0, g);
  }
  if (ntiles > 1) {
    const Dest d1 = dest(1);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (g < ngroups) group(d1, g);
    if (wside) wait_vm<R::PWW>();   // own loads of stage 0
    else wait_vm<R::PWX>();
  } else {
    wait_vm<0>();
  }
  __syncthreads();

  bf16x8 fa[2][C::FN], fb[2][C::FM];
  const int rl = lane & 31, ch = lane >> 5;
  {
#pragma unroll
    for (int i = 0; i < C::FN; ++i) fa[0][i] = read_frag(smem, wrow + i * 32 + rl, ch);
#pragma unroll
    for (int j = 0; j < C::FM; ++j) fb[0][j] = read_frag(smem + C::TN * ROW_BYTES, xrow + j * 32 + rl, ch);
  }
  // chunks at or past kdim and masked activation rows enter as zero
  auto fix = [&](int k0, int s, int buf) __attribute__((always_inline)) {
    if (k0 + (2 * s + ch) * 8 >= kdim) {
#pragma unroll
      for (int i = 0; i < C::FN; ++i) fa[buf][i] = bf16x8{};
#pragma unroll
      for (int j = 0; j < C::FM; ++j) fb[buf][j] = bf16x8{};
    }
    if constexpr (MASK_ROWS) {
#pragma unroll
      for (int j = 0; j < C::FM; ++j)
        if (!((keep >> j) & 1u)) fb[buf][j] = bf16x8{};
    }
  };
  auto mfma = [&](int buf, int i, int j) __attribute__((always_inline)) {
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };

  Dest held{};          // stage t+1's groups 2 and 3, issued in substep 0 of stage t
  bool held_live = false;
  auto iter = [&](int t, auto checked, auto parity) __attribute__((always_inline)) {
    constexpr bool CHECKED = decltype(checked)::value;
    constexpr int P = decltype(parity)::value;   // t & 1
    int k0 = 0;
    if constexpr (CHECKED) {
      Side w, x;
      src(t, w, x, k0);
    }
    const bool live = t + 2 < ntiles;
    Dest next{};
    auto substep = [&](auto sc) __attribute__((always_inline)) {
      constexpr int s = decltype(sc)::value;
      constexpr int buf = s & 1, ns = s < 3 ? s + 1 : 0, nb = (s + 1) & 1;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (CHECKED) fix(k0, s, buf);
      // the next substep's fragments: this stage's, or stage t+1's first (past
      // the last stage a stale slot, never used)
      const char* nx = smem + ((s < 3 ? P : P + 1) & 1) * R::STAGE;
      auto rd = [&](int g) __attribute__((always_inline)) {
        fa[nb][g] = read_frag(nx, wrow + g * 32 + rl, 2 * ns + ch);
        if (g < C::FM) fb[nb][g] = read_frag(nx + C::TN * ROW_BYTES, xrow + g * 32 + rl, 2 * ns + ch);
      };
      auto chunk = [&](auto gc) __attribute__((always_inline)) {
        constexpr int g = decltype(gc)::value;
        if constexpr (s == 3 && g == 0) {
#pragma unroll
          for (int j = 0; j < C::FM; ++j) mfma(buf, 0, j);
          __builtin_amdgcn_sched_barrier(0);
          // own loads of stage t+1 landed; after the barrier every wave's
          // have, and every wave has read all of stage t
          wait_vm<0>();
          __syncthreads();
          __builtin_amdgcn_sched_barrier(0);
          rd(0);
          next = dest(live ? t + 2 : t);
          if (live) group(next, 0);   // every wave has at least two groups
          __builtin_amdgcn_sched_barrier(0);
          return;
        }
        // the chunk's MFMAs (one row block against the wave's FM column
        // blocks) with one fragment read of the next substep after each of
        // the first two
        constexpr bool XREAD = g < C::FM;
        mfma(buf, g, 0);
        fa[nb][g] = read_frag(nx, wrow + g * 32 + rl, 2 * ns + ch);
        mfma(buf, g, 1);
        if constexpr (XREAD) fb[nb][g] = read_frag(nx + C::TN * ROW_BYTES, xrow + g * 32 + rl, 2 * ns + ch);
#pragma unroll
        for (int j = 2; j < C::FM; ++j) mfma(buf, g, j);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (XREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if constexpr (C::FM > 2) __builtin_amdgcn_sched_group_barrier(0x008, C::FM - 2, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (s == 3 && g == 1) {
          if (live) group(next, 1);
        }
        if constexpr (s == 0 && g >= 2) {
          if (held_live && g < ngroups) group(held, g);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      chunk(std::integral_constant<int, 0>{});
      chunk(std::integral_constant<int, 1>{});
      chunk(std::integral_constant<int, 2>{});
      chunk(std::integral_constant<int, 3>{});
    };
    substep(std::integral_constant<int, 0>{});
    substep(std::integral_constant<int, 1>{});
    substep(std::integral_constant<int, 2>{});
    substep(std::integral_constant<int, 3>{});
    held = next;
    held_live = live;
  };
  // Stages go in pairs, so that the ring slot a fragment read addresses is a
  // compile-time constant (its address then needs no per-stage arithmetic).
  // The K tail can only fall in the last stage of the base product; the
  // expand (MASK_ROWS) checks every stage.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int t = 0;
  if constexpr (!MASK_ROWS) {
    for (; t + 2 < ntiles; t += 2) {
      iter(t, std::false_type{}, P0{});
      iter(t + 1, std::false_type{}, P1{});
    }
  }
  for (; t + 1 < ntiles; t += 2) {
    iter(t, std::true_type{}, P0{});
    iter(t + 1, std::true_type{}, P1{});
  }
  if (t < ntiles) iter(t, std::true_type{}, P0{});
  __syncthreads();   // the ring is reused by whatever runs next
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

// Row of X behind virtual row v of adapter a: a's segments in row order,
// concatenated (-1 past its last row).
__device__ __forceinline__ int virtual_row(const SegTable& st, int a, int v) {
  for (int g = 0; g < st.n; ++g) {
    if (st.adapter[g] != a) continue;
    const int len = st.start[g + 1] - st.start[g];
    if (v < len) return st.start[g] + v;
    v -= len;
  }
  return -1;
}

// The rows of X behind a shrink tile's virtual rows v0 .. v0 + nrows - 1.
template <class C>
__device__ __forceinline__ void shrink_rows(int* phys, const SegTable& st, int a, int v0, int nrows, int tid) {
  for (int r = tid; r < C::TM; r += C::NT) phys[r] = r < nrows ? virtual_row(st, a, v0 + r) : -1;
}

// Tile `lt` of the shrink grid: its rank tile (j0), adapter, and first
// virtual row and row count.
struct ShrinkTile {
  int j0, a, v0, nrows;
};
template <class C>
__device__ __forceinline__ ShrinkTile shrink_tile(int lt, int ntn, int ntm, const ShrinkPlan& sp) {
  int tn, tv;
  tile_of_block(lt, ntn, ntm, tn, tv);
  int a = 0;                                   // the adapter whose virtual rows tile tv covers
  while (a + 1 < sp.n_adapters && sp.tile_off[a + 1] <= tv) ++a;
  const int v0 = (tv - sp.tile_off[a]) * C::TM;
  return ShrinkTile{tn * C::TN, a, v0, min(C::TM, sp.rows[a] - v0)};
}

// T = s_a acc of one 32 x 32 MFMA tile, as bf16 hi and lo parts:
// acc[r] is rank index jt + (r/4)*8 + (lane/32)*4 + r%4 on the lane's row of X
// (`row`, -1 for none).
__device__ __forceinline__ void store_t_frag(const f32x16& acc, const ProjArgs& p, float scale, int jt, int row,
                                             int lane) {
  const auto tres = make_rsrc(p.T, p.t_bytes);
  const uint32_t lo_base = uint32_t(p.M) * uint32_t(p.trank) * 2u;   // T_lo follows T_hi
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int jr = jt + q * 8 + (lane >> 5) * 4;
    float h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_hi_lo(scale * acc[q * 4 + e], h[e], l[e]);
    const uint32_t off = (row >= 0 && jr < p.trank) ? (uint32_t(row) * uint32_t(p.trank) + uint32_t(jr)) * 2u
                                                    : kMaskedOffset;
    const u32x2 hv{pack2(h[0], h[1]), pack2(h[2], h[3])};
    const u32x2 lv{pack2(l[0], l[1]), pack2(l[2], l[3])};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, hv), tres, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, lv), tres,
                                          off == kMaskedOffset ? kMaskedOffset : off + lo_base, 0, 0);
  }
}

// T = s_a acc on the tile's rows.
// acc[i][j][r]: rank index j0 + wn*(TN/WN) + i*32 + (r/4)*8 + (lane/32)*4 + r%4,
//               virtual row wm*(TM/WM) + j*32 + lane%32 of the tile
template <class C>
__device__ __forceinline__ void store_t(const f32x16 (&acc)[C::FN][C::FM], const ProjArgs& p, float scale, int j0,
                                        const int* phys, int wn, int wm, int lane) {
#pragma unroll
  for (int j = 0; j < C::FM; ++j) {
    const int row = phys[wm * (C::TM / C::WM) + j * 32 + (lane & 31)];
#pragma unroll
    for (int i = 0; i < C::FN; ++i) store_t_frag(acc[i][j], p, scale, j0 + wn * (C::TN / C::WN) + i * 32, row, lane);
  }
}

// A partial's layout: per wave, per (i, j) fragment, per quarter q, the 64
// lanes' four floats, so each store and load is one 1 KiB line per wave.
template <class C>
__device__ __forceinline__ uint32_t part_off(int wave, int i, int j, int q, int lane) {
  return uint32_t((((wave * C::FN + i) * C::FM + j) * 4 + q) * 1024 + lane * 16);
}

// ------------------------------------------------------------------ shrink
// Adapter-sorted: the rows that name adapter a, gathered from all its segments
// in row order, form a virtual row range (ShrinkPlan), and the grid has one
// block per (rank tile, virtual row tile).  A block computes
// acc = A_a[rank tile] X[its rows]^T with the activation rows loaded through an
// LDS row map, then stores T = s_a acc as bf16 hi and lo parts on those rows.
// One K loop per tile whatever the batch's interleaving of adapters, and no
// rows computed only to be dropped, except in each adapter's last tile.
//
// A grid of few tiles (a batch of few adapter rows) runs sp.splits blocks per
// tile, each over its share of K, which store their fp32 partials; the sum in
// split order (shrink_reduce_kernel) stores T, so the result does not depend
// on timing.
template <class C>
__global__ __launch_bounds__(C::NT) void shrink_kernel(ProjArgs p, SegTable st, AdapterTable at, ShrinkPlan sp, int ntn,
                                                       int ntm) {
  static_assert(C::TM == kShrinkRows && C::TN == kShrinkRows, "shrink tiles are planned in kShrinkRows rows");
  static_assert(C::NW * C::FN * C::FM * 4 * 1024 == int(kShrinkPartBytes), "partial layout");
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE];
  __shared__ int phys[C::TM];
  const int ntiles = ntn * ntm;
  const int lt = int(blockIdx.x) % ntiles, split = int(blockIdx.x) / ntiles;
  const ShrinkTile tl = shrink_tile<C>(lt, ntn, ntm, sp);
  const int atrank = p.sl.n * at.rank[tl.a];   // rows of A_a
  if (tl.j0 >= atrank) return;                 // a rank tile past this adapter's rank (whole block)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;
  shrink_rows<C>(phys, st, tl.a, tl.v0, tl.nrows, tid);
  __syncthreads();

  const Side as{make_rsrc_words(at.A[tl.a], at.a_bytes[tl.a]), uint32_t(p.K) * 2u, tl.j0};
  const Side xs{make_rsrc_words(p.X, p.x_bytes), uint32_t(p.K) * 2u, 0};
  f32x16 acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};
  // this block's stages [t0, t1) of the nk; the K tail can only fall in the last
  const int nk = (p.K + BK - 1) / BK;
  const int t0 = split * nk / sp.splits, t1 = (split + 1) * nk / sp.splits;
  const int nfull = p.K / BK;
  k_loop_small_reg<C>(acc, t1 - t0, max(0, min(t1, nfull) - t0), p.K,
                      [&](int t, Side& ws, Side& xsd, int& k0) { ws = as; xsd = xs; k0 = (t0 + t) * BK; },
                      smem, tid, wn, wm, phys);
  if (sp.splits == 1) {
    store_t<C>(acc, p, at.scale[tl.a], tl.j0, phys, wn, wm, lane);
    return;
  }
  const auto pres = make_rsrc(sp.part, sp.part_bytes);
  const uint32_t base = uint32_t(lt * sp.splits + split) * kShrinkPartBytes;
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 w{__float_as_uint(acc[i][j][q * 4 + 0]), __float_as_uint(acc[i][j][q * 4 + 1]),
                      __float_as_uint(acc[i][j][q * 4 + 2]), __float_as_uint(acc[i][j][q * 4 + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(w, pres, base + part_off<C>(wave, i, j, q, lane), 0, 0);
      }
}

// T of the split shrink's tiles: each tile's partials summed in split order,
// then stored as the unsplit shrink stores them.  One 32 x 32 MFMA tile per
// wave: block b covers the part that wave b % NW of tile b / NW computed, its
// wave w the fragment (w / FM, w % FM), with every split's loads in flight at
// once.
template <class C>
__global__ __launch_bounds__(C::NT) void shrink_reduce_kernel(ProjArgs p, SegTable st, AdapterTable at, ShrinkPlan sp,
                                                              int ntn, int ntm) {
  static_assert(C::FN * C::FM == C::NW, "one fragment per wave");
  const int lt = int(blockIdx.x) / C::NW, part = int(blockIdx.x) % C::NW;
  const ShrinkTile tl = shrink_tile<C>(lt, ntn, ntm, sp);
  if (tl.j0 >= p.sl.n * at.rank[tl.a]) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = wave / C::FM, j = wave % C::FM;
  const int wn = part % C::WN, wm = part / C::WN;
  const int r = wm * (C::TM / C::WM) + j * 32 + (lane & 31);   // the lane's virtual row in the tile
  const int row = r < tl.nrows ? virtual_row(st, tl.a, tl.v0 + r) : -1;
  const auto pres = make_rsrc(sp.part, sp.part_bytes);
  f32x4 v[kShrinkMaxSplits][4];
#pragma unroll
  for (int s_i = 0; s_i < kShrinkMaxSplits; ++s_i)
    if (s_i < sp.splits) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[s_i][q] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       pres, uint32_t(lt * sp.splits + s_i) * kShrinkPartBytes + part_off<C>(part, i, j, q, lane), 0, 0));
    }
  f32x16 acc{};
#pragma unroll
  for (int s_i = 0; s_i < kShrinkMaxSplits; ++s_i)
    if (s_i < sp.splits) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[q * 4 + e] += v[s_i][q][e];
    }
  store_t_frag(acc, p, at.scale[tl.a], tl.j0 + wn * (C::TN / C::WN) + i * 32, row, lane);
}

// ------------------------------------------------------------------ main
template <class C, bool F32_OUT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void main_kernel(
    ProjArgs p, SegTable st, AdapterTable at, int has_adapter, int ntn, int ntm) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * WideRing<C>::STAGE];
  __shared__ int8_t row_adapter[C::TM];   // adapter named by each row of the tile, -1 for none
  int tn, tm;
  tile_of_block(blockIdx.x, ntn, ntm, tn, tm);
  const int n0 = tn * C::TN, m0 = tm * C::TM;
  const int m1 = min(m0 + C::TM, p.M);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;
  if (has_adapter) {   // before the accumulators fill: the map is read by the expand only
    for (int t = tid; t < C::TM; t += C::NT) row_adapter[t] = -1;
    __syncthreads();
    for (int g = first_segment(st, m0); g < st.n && st.start[g] < m1; ++g)
      for (int t = tid; t < C::TM; t += C::NT)
        if (m0 + t >= st.start[g] && m0 + t < st.start[g + 1]) row_adapter[t] = st.adapter[g];
    __syncthreads();
  }

  f32x16 acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};

  // base product over K
  {
    const Side ws{make_rsrc_words(p.W, p.w_bytes), uint32_t(p.K) * 2u, n0};
    const Side xs{make_rsrc_words(p.X, p.x_bytes), uint32_t(p.K) * 2u, m0};
    const int nk = (p.K + BK - 1) / BK;
    auto src = [&](int t, Side& w, Side& x, int& k0) { w = ws; x = xs; k0 = t * BK; };
    k_loop_wide<C, false>(acc, nk, p.K, src, smem, tid, wn, wm);
  }

  // expand: for each adapter that rows of the tile name, stages alternate
  // T_hi and T_lo against the same 64-wide slab of B_a, with the rows that
  // name another adapter or none masked to zero: one pass per adapter however
  // many segments it has in the tile (each row's own adapter adds its term in
  // one pass, the other passes add exact zeros).  The tile's slice reads its
  // own r_a columns of T (a tile never straddles two slices).
  if (has_adapter) {
    const int slice = slice_of(p.sl, n0);
    const uint32_t tld = uint32_t(p.trank) * 2u;
    const int lo_row0 = m0 + p.M;          // T_lo rows sit M rows after T_hi rows
    uint32_t seen = 0;                     // adapters already applied to this tile
    for (int g = first_segment(st, m0); g < st.n && st.start[g] < m1; ++g) {
      const int a = st.adapter[g];
      if (a < 0 || ((seen >> a) & 1u)) continue;
      seen |= 1u << a;
      uint32_t keep = 0;                   // this lane's activation rows that name a
#pragma unroll
      for (int j = 0; j < C::FM; ++j)
        keep |= row_adapter[wm * (C::TM / C::WM) + j * 32 + (lane & 31)] == a ? 1u << j : 0u;
      // adapter a's rank: B_a's row stride, the tile's slice of T (r_a columns
      // from slice x r_a), and the number of stages
      const int ra = at.rank[a];
      const uint32_t ld = uint32_t(ra) * 2u, tcol = uint32_t(slice * ra) * 2u;
      const i32x4 tres = make_rsrc_words(static_cast<const char*>(p.T) + tcol, p.t_bytes - tcol);
      const Side bs{make_rsrc_words(at.B[a], at.b_bytes[a]), ld, n0};
      const Side th{tres, tld, m0};
      const Side tl{tres, tld, lo_row0};
      const int nr = 2 * ((ra + BK - 1) / BK);
      auto src = [&](int t, Side& w, Side& x, int& k0) { w = bs; x = (t & 1) ? tl : th; k0 = (t >> 1) * BK; };
      k_loop_wide_dma<C, true>(acc, nr, ra, src, smem, tid, wn, wm, keep);
    }
  }

  // epilogue: acc[i][j][r] is column n0 + wn*(TN/WN) + i*32 + (r/4)*8 + (lane/32)*4 + r%4
  // of row m0 + wm*(TM/WM) + j*32 + lane%32.  When N % 4 == 0 each lane writes its
  // four consecutive columns at once; otherwise one element at a time.
  const auto yres = make_rsrc(p.Y, p.y_bytes);
  const int mrow = m0 + wm * (C::TM / C::WM) + (lane & 31);
  const int ncol = n0 + wn * (C::TN / C::WN) + (lane >> 5) * 4;
  if ((p.N & 3) == 0) {
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int m = mrow + j * 32;
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = ncol + i * 32 + q * 8;
          const bool ok = m < p.M && n < p.N;
          const uint32_t e0 = uint32_t(m) * uint32_t(p.N) + uint32_t(n);
          if constexpr (F32_OUT) {
            // element values go through __float_as_uint: a bit cast applied to a vector-element
            // lvalue would read element 0
            const u32x4 w{__float_as_uint(acc[i][j][q * 4 + 0]), __float_as_uint(acc[i][j][q * 4 + 1]),
                          __float_as_uint(acc[i][j][q * 4 + 2]), __float_as_uint(acc[i][j][q * 4 + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(w, yres, ok ? e0 * 4u : kMaskedOffset, 0, 0);
          } else {
            const u32x2 w{pack2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]), pack2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3])};
            __builtin_amdgcn_raw_buffer_store_b64(w, yres, ok ? e0 * 2u : kMaskedOffset, 0, 0);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int m = mrow + j * 32;
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = ncol + i * 32 + q * 8 + e;
            const bool ok = m < p.M && n < p.N;
            const uint32_t e0 = uint32_t(m) * uint32_t(p.N) + uint32_t(n);
            if constexpr (F32_OUT) {
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][q * 4 + e]), yres,
                                                    ok ? e0 * 4u : kMaskedOffset, 0, 0);
            } else {
              __builtin_amdgcn_raw_buffer_store_b16(uint16_t(bf16_bits(acc[i][j][q * 4 + e])), yres,
                                                    ok ? e0 * 2u : kMaskedOffset, 0, 0);
            }
          }
    }
  }
}

// Tile choices.  Output: 256 weight rows by 256, 192 or 128 activation rows,
// four waves of 128 x 128, 96 or 64, one per SIMD, up to 256 fp32 accumulators
// per lane (in AGPRs), up to 128 KiB of LDS for the ring.  The host picks the
// height per call (main_tile_rows).
// Shrink: 128x128 tiles, so a 256-wide rank still gives two blocks per row
// tile.  (Batches of at most 128 rows take the decode kernel.)
using MainBig = Tile<256, 256, 2, 2>;
using Main192 = Tile<256, 192, 2, 2>;
using Main128 = Tile<256, 128, 2, 2>;
using ShrinkBig = Tile<128, 128, 2, 2>;

template <class C>
hipError_t launch_shrink_t(const ProjArgs& p, const SegTable& st, const AdapterTable& at, const ShrinkPlan& sp,
                           hipStream_t s) {
  const int ntn = (p.trank + C::TN - 1) / C::TN, ntm = sp.tile_off[sp.n_adapters];
  if (ntm == 0) return hipSuccess;
  ProjArgs pa = p;
  SegTable sa = st;
  AdapterTable aa = at;
  ShrinkPlan spa = sp;
  int a0 = ntn, a1 = ntm;
  void* args[] = {&pa, &sa, &aa, &spa, &a0, &a1};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&shrink_kernel<C>), dim3(ntn * ntm * sp.splits),
                                 dim3(C::NT), args, 0, s);
  if (e == hipSuccess && sp.splits > 1)
    e = hipLaunchKernel(reinterpret_cast<const void*>(&shrink_reduce_kernel<C>), dim3(ntn * ntm * C::NW), dim3(C::NT),
                        args, 0, s);
  return e;
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

hipError_t launch_bf16_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at, const ShrinkPlan& sp,
                              hipStream_t stream) {
  return launch_shrink_t<ShrinkBig>(p, st, at, sp, stream);
}

int main_tile_rows(int M, int N) {
  // Blocks run one per CU in whole waves of the chip, so a call takes about
  // ceil(tiles / CUs) tile times.  A tile's time shrinks far less than its
  // height, since each stage's loads, LDS traffic and barrier do not shrink
  // with it: whole calls running a single wave of tiles took about
  // 1 : 0.88 : 0.77 for 256, 192 and 128 rows.  Take the height with the
  // fewest tile times.
  constexpr int kCUs = 256;
  const int ntn = (N + 255) / 256;
  int best = 256;
  double best_cost = 0;
  for (const int tm : {256, 192, 128}) {
    const double tile_time = tm == 256 ? 1.0 : tm == 192 ? 0.88 : 0.77;
    const int64_t tiles = int64_t(ntn) * ((M + tm - 1) / tm);
    const double cost = double((tiles + kCUs - 1) / kCUs) * tile_time;
    if (tm == 256 || cost < best_cost) {
      best = tm;
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_bf16_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at, bool has_adapter,
                            bool f32_out, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  switch (main_tile_rows(p.M, p.N)) {
    case 128:
      return f32_out ? launch_main_t<Main128, true>(p, st, at, has_adapter, stream, e0, e1)
                     : launch_main_t<Main128, false>(p, st, at, has_adapter, stream, e0, e1);
    case 192:
      return f32_out ? launch_main_t<Main192, true>(p, st, at, has_adapter, stream, e0, e1)
                     : launch_main_t<Main192, false>(p, st, at, has_adapter, stream, e0, e1);
    default:
      return f32_out ? launch_main_t<MainBig, true>(p, st, at, has_adapter, stream, e0, e1)
                     : launch_main_t<MainBig, false>(p, st, at, has_adapter, stream, e0, e1);
  }
}

}  // namespace lora
