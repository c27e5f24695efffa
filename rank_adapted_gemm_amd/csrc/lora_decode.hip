// Decode-path kernel of the mixed-adapter LoRA projection (M <= 128 rows).
//
// At decode sizes the call is bound by HBM: every byte of W, A_a and B_a is read
// once and reused only M times.  One launch does the whole call:
//
//   * Work is cut into units: one unit is a 64-element K slice (128-byte rows)
//     of a 128-row tile of a weight matrix, multiplied against the same slice
//     of the activation rows.  A unit streams through an LDS ring filled by
//     buffer_load ... lds (full 128-byte lines, several units in flight), and
//     all four waves multiply on v_mfma_f32_16x16x32_bf16 (32 weight rows x
//     16*MT activation rows each).
//   * A blocks (first in the grid, a few) each take one K range of every A_a
//     tile and store one fp32 partial per tile.  When all of them are done
//     they reduce T = s_a * X A_a^T between them, each a share of the
//     (tile, 16-row) pieces, and store it as bf16 hi = bf16(T), lo =
//     bf16(T - hi), zero on rows that name another adapter or none.
//   * W blocks (one per remaining CU) split the W units evenly and in order
//     (stream-K).  The expand units of a tile (B_a's rows against T_hi and
//     T_lo) are shared out among the blocks whose W range ends in that tile,
//     and each adds its share into the same accumulators as its last W units,
//     so a tile has one partial per block and no separate expand partials.
//     The first expand unit waits for T if the A blocks are not done yet.
//   * At the end of its part of a W tile a block stores its fp32 partial
//     (fragment-major, so stores and reloads are whole 1 KiB lines) and counts
//     itself in on the tile.  The last one in sums the tile's partials in
//     block order (so the result does not depend on timing) and stores Y once.
//
// The split of the W units depends on (N, K, r) only, and the expand adds exact
// zeros on rows that name no adapter, so base-only rows come out bitwise the
// same with or without adapter rows in the batch ("two 27B models on a single
// RTX 5090", section 4 request-path figure: requests naming the base model use
// the base weights alone).
//
// Data shared between blocks (partials, T) is written and read with
// device-scope (sc1) accesses, so handing it over costs a vmcnt wait and one
// atomic add, never an L2 flush.  The counters sit in the workspace's counter
// area: zero when the workspace is first used, and put back to zero by the
// block that uses each last, so nothing has to clear them between calls.
//
// Nothing fails silently ("serving-qwen3-8-27b-on-one-rtx-3090", Installing: a
// path that silently runs wrong or slow, with nothing in the logs, is the failure
// to avoid).  Every wait is bounded; a wait that gives up, or an arrival that
// finds a count already at its expected total (a counter area left non-zero by a
// call that never finished), sets a sticky bit in the last 8 bytes of the counter
// area, which lora_workspace_status reports before it restores the area.  The
// data a lost wait would have carried is replaced by NaN, so the outputs that
// depended on it are NaN.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "lora_device.h"

namespace lora {
namespace {

constexpr int TR = kDecodeTileRows;   // 128 weight rows per tile
constexpr int UK = kDecodeUnitK;      // 64 elements per unit
constexpr int RB = UK * 2;            // 128 bytes per tile row per unit

__host__ __device__ inline int64_t pstart(int64_t b, int64_t U, int64_t G) { return b * U / G; }
// Block of a partition of U units over G blocks that holds unit u.
__host__ __device__ inline int64_t pblock(int64_t u, int64_t U, int64_t G) { return ((u + 1) * G - 1) / U; }

template <int MT_>
struct DG {
  static constexpr int MT = MT_;                   // 16-row activation tiles
  static constexpr int XR = 16 * MT;               // activation rows staged per unit
  static constexpr int STAGE = (TR + XR) * RB;
  static constexpr int NS = std::min(8, (160 * 1024) / STAGE);
  static constexpr int GT = (TR + XR) / 8;         // 8-row groups, one wave-wide 16-byte load each
  static constexpr int NA = GT % 4 == 0 ? 4 : GT % 4;
  static constexpr int PWA = (GT + 3) / 4;         // loads per unit, waves < NA
  static constexpr int PWB = GT / 4;               // loads per unit, other waves
  static constexpr int FRAG = 4 * 2 * MT * 64 * 16;   // bytes of one partial
  static_assert(NS >= 3, "ring too shallow");
};

// 16-byte chunk c of a 128-byte row r sits at slot c ^ ((r >> 1) & 7).  A
// ds_read_b128 serves 16 lanes per cycle: rows r..r+15 of one chunk, which this
// spreads over all 64 banks.
__device__ __forceinline__ int doff(int r, int c) { return r * RB + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ bf16x8 frag(const char* base, int r, int c) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + doff(r, c)));
}

template <int PW, int NS>
__device__ __forceinline__ void wait_ring(int ahead) {   // at most `ahead` later units still loading
  if constexpr (NS > 7) { if (ahead >= 6) { wait_vm<PW * 6>(); return; } }
  if constexpr (NS > 6) { if (ahead >= 5) { wait_vm<PW * 5>(); return; } }
  if constexpr (NS > 5) { if (ahead >= 4) { wait_vm<PW * 4>(); return; } }
  if constexpr (NS > 4) { if (ahead >= 3) { wait_vm<PW * 3>(); return; } }
  if constexpr (NS > 3) { if (ahead >= 2) { wait_vm<PW * 2>(); return; } }
  if (ahead >= 1) { wait_vm<PW>(); return; }
  wait_vm<0>();
}

typedef unsigned long long u64;

// Arrival counters: plain device-scope adds (one round trip, no retries).  A
// counter is zero when a call starts and the block that uses it last puts it
// back to zero.  An arrival that takes a count past `total` flags the call.
__device__ inline uint32_t arrive(u64* c, uint32_t* err, uint32_t total, uint32_t k = 1) {
  const uint32_t old = uint32_t(__hip_atomic_fetch_add(c, u64(k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (old + k > total) __hip_atomic_fetch_or(err, kDecodeErrCount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}
__device__ inline void clear(u64* c) { __hip_atomic_store(c, u64(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

enum Kind { KIND_A = 0, KIND_E = 1, KIND_W = 2 };

// Position of a unit: tile `key` and unit `st` inside it.  A units also carry
// the adapter slot and the rank tile of the key, expand units the slot and the
// hi/lo half.  Cursors step one unit at a time, so the loops never divide.
struct Cur {
  int key, st, slot, at, hl;
};

// One unit's operands: weight-side rows (128, row stride wld) and activation
// rows (XR, row stride xld), each from byte offset *base.
struct Unit {
  i32x4 wres, xres;
  uint32_t wbase, wld, xbase, xld;
};

// RANKED: adapters of different ranks; each adapter's rank, row stride and
// extents are looked up per unit, and expand units past an adapter's rank move
// no data.  Otherwise every adapter has the call's rank (the common case keeps
// its own instantiation, free of those lookups).
template <bool RANKED>
__device__ inline Unit unit_of(const Cur& c, Kind kind, const DecodeArgs& d, const AdapterTable& at) {
  Unit x;
  if (kind == KIND_E) {   // B_a's rows of the tile against the tile's slice of T (r_a columns)
    const int a = d.slot_adapter[c.slot];
    const int ra = RANKED ? at.rank[a] : d.rank;
    x.wres = make_rsrc_words(at.B[a], RANKED ? at.b_bytes[a] : d.b_bytes);
    x.wld = uint32_t(ra) * 2u;
    x.xres = make_rsrc_words(c.hl ? d.TL : d.TH, d.t_bytes);
    x.xld = uint32_t(d.trank) * 2u;
    x.wbase = uint32_t(c.key * TR) * x.wld + uint32_t(c.st) * RB;
    x.xbase = uint32_t(c.slot * d.M) * x.xld + uint32_t(slice_of(d.sl, c.key * TR) * ra) * 2u + uint32_t(c.st) * RB;
    if (RANKED && c.st * UK >= ra) {   // past this adapter's rank: no traffic (the multiply zeroes it too)
      x.wbase = kMaskedOffset;
      x.xbase = kMaskedOffset;
    }
  } else {
    x.wld = uint32_t(d.K) * 2u;
    if (kind == KIND_A) {
      const int a = d.slot_adapter[c.slot];
      x.wres = make_rsrc_words(at.A[a], RANKED ? at.a_bytes[a] : d.a_bytes);
      x.wbase = uint32_t(c.at * TR) * x.wld + uint32_t(c.st) * RB;
    } else {
      x.wres = make_rsrc_words(d.W, d.w_bytes);
      x.wbase = uint32_t(c.key * TR) * x.wld + uint32_t(c.st) * RB;
    }
    x.xres = make_rsrc_words(d.X, d.x_bytes);
    x.xld = x.wld;
    x.xbase = uint32_t(c.st) * RB;
  }
  return x;
}

// Spin (thread 0) until the counter reaches `want`; bounded, so a broken
// hand-over never hangs: after `limit` polls it flags the call and returns false.
__device__ inline bool wait_for(u64* c, u64 want, uint32_t limit, uint32_t* err) {
  for (uint32_t it = 0; it < limit; ++it) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  __hip_atomic_fetch_or(err, kDecodeErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// Q4: the base weights come as 4-bit codes plus per-group params (see
// lora_proj_q4); W units then carry 4 KiB of codes and their params instead of
// 16 KiB of bf16, and the multiply dequantizes the weight fragments to bf16.
template <int MT, bool F32_OUT, bool Q4, bool RANKED>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs d, AdapterTable at) {
  using G = DG<MT>;
  __shared__ __attribute__((aligned(1024))) char smem[G::NS * G::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lbase = lds_addr(smem);

  const int nAt = d.n_used * d.ntA;                // A tiles
  const int nEpt = d.n_used * 2 * d.nrs;           // expand units per W tile
  const int64_t UW = int64_t(d.ntW) * d.nst;
  u64* const cW = d.cnt;                           // arrivals per W tile
  u64* const cA = d.cnt + d.ntW;                   // A blocks done
  u64* const cT = cA + 1;                          // T pieces done
  u64* const cF = cA + 2;                          // W tiles finished
  const uint32_t t_total = uint32_t(nAt * MT * 2); // T pieces of the call
  // the test hook waits for one piece more than exist, with a short spin
  const uint64_t t_want = t_total + (d.fault ? 1u : 0u);
  const uint32_t spin = d.fault ? 64u : d.spin_limit;
  int t_lost = 0;                                  // (uniform) this block gave up waiting for T
  const bool ablock = int(blockIdx.x) < d.GA;
  const int b = ablock ? int(blockIdx.x) : int(blockIdx.x) - d.GA;
  const int ka0 = ablock ? int(int64_t(b) * d.nst / d.GA) : 0;        // K units of an A block
  const int ka1 = ablock ? int(int64_t(b + 1) * d.nst / d.GA) : 0;

  auto advance = [&](Cur& c, Kind kind) __attribute__((always_inline)) {
    if (kind == KIND_E) {
      if (++c.st == d.nrs) {
        c.st = 0;
        if (++c.hl == 2) {
          c.hl = 0;
          if (++c.slot == d.n_used) {
            c.slot = 0;
            ++c.key;
          }
        }
      }
    } else if (kind == KIND_W) {
      if (++c.st == d.nst) {
        c.st = 0;
        ++c.key;
      }
    } else if (++c.st == ka1) {
      c.st = ka0;
      ++c.key;
      if (++c.at == d.ntA) {
        c.at = 0;
        ++c.slot;
      }
    }
  };

  // Weight rows: wave w loads 8-row groups 4w .. 4w+3.  Activation rows: the
  // 2 MT groups are dealt out in consecutive runs, one more to each of the
  // first (2 MT) % 4 waves.  Lane l fills row l / 8, chunk l % 8.  Each run
  // goes out under one M0 value.
  constexpr int XG = 2 * MT, XQ = XG / 4, XREM = XG % 4;
  const int xcount = XQ + (wave < XREM ? 1 : 0);
  const int xfirst = wave * XQ + min(wave, XREM);
  auto issue = [&](int slot, const Cur& c, Kind kind) __attribute__((always_inline)) {
    const Unit x = unit_of<RANKED>(c, kind, d, at);
    const uint32_t dst = lbase + uint32_t(slot) * G::STAGE;
    if (Q4 && kind == KIND_W) {
      // wave w's 4 KiB: codes of its 32 rows (32 bytes each, row-major), then
      // their params words (4 bytes each); two more masked loads keep every
      // wave at four weight-side loads per unit, like the bf16 units
      const uint32_t kb = uint32_t(d.K) / 2u;                       // code bytes per row
      const uint32_t row0 = uint32_t(c.key * TR + 32 * wave);
      const uint32_t code_off[1] = {(row0 + uint32_t(lane >> 1)) * kb + uint32_t(c.st) * 32u + uint32_t(lane & 1) * 16u};
      dma16_group<1>(make_rsrc_words(d.W, d.w_bytes), code_off, dst + uint32_t(4 * wave) * 1024u);
      const uint32_t g = uint32_t(c.st) / 2u;                        // 128-wide group of the unit
      const uint32_t prm_off[3] = {lane < 8 ? (g * uint32_t(d.N) + row0 + uint32_t(lane) * 4u) * 4u : kDmaMaskedOffset,
                                   kDmaMaskedOffset, kDmaMaskedOffset};
      dma16_group<3>(make_rsrc_words(d.WP, d.wp_bytes), prm_off, dst + uint32_t(4 * wave + 1) * 1024u);
    } else {
      uint32_t off[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (4 * wave + i) * 8 + (lane >> 3);
        const int ch = (lane & 7) ^ ((r >> 1) & 7);
        off[i] = x.wbase + uint32_t(r) * x.wld + uint32_t(ch) * 16u;
      }
      dma16_group<4>(x.wres, off, dst + uint32_t(4 * wave) * 1024u);
    }
    auto xrun = [&](auto nc) __attribute__((always_inline)) {
      constexpr int NL = decltype(nc)::value;
      uint32_t off[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int r = (xfirst + i) * 8 + (lane >> 3);
        const int ch = (lane & 7) ^ ((r >> 1) & 7);
        off[i] = r < d.M ? x.xbase + uint32_t(r) * x.xld + uint32_t(ch) * 16u : kDmaMaskedOffset;
      }
      const uint32_t to = dst + uint32_t(TR / 8 + xfirst) * 1024u;
      if (kind == KIND_E) dma16_group<NL, true>(x.xres, off, to);   // T, written during this launch
      else dma16_group<NL>(x.xres, off, to);
    };
    if constexpr (XREM == 0) {
      xrun(std::integral_constant<int, XQ>{});
    } else {
      if (xcount == XQ + 1) xrun(std::integral_constant<int, XQ + 1>{});
      else xrun(std::integral_constant<int, XQ>{});
    }
  };

  f32x4 acc[2][MT];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rg][mt] = f32x4{};

  // acc[rg][mt][e] is weight row 32 wave + 16 rg + 4 (lane/16) + e of the tile,
  // activation row 16 mt + lane % 16.  A partial stores acc in that order.
  auto frag_off = [&](int rg, int mt) __attribute__((always_inline)) { return uint32_t(((wave * 2 + rg) * MT + mt) * 1024 + lane * 16); };

  // poison: NaN in place of the sums (this block's expand never got T)
  auto store_partial = [&](float* P, uint32_t pbytes, uint32_t slot, bool poison) __attribute__((always_inline)) {
    const auto pres = make_rsrc(P, pbytes);
    const f32x4 nan4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, poison ? nan4 : acc[rg][mt]), pres,
                                               slot * uint32_t(G::FRAG) + frag_off(rg, mt), 0, kDeviceScope);
  };

  // s += partial slots first .. first+n-1, in order, SB in flight (nothing else
  // is live when a tile is finished, so the loads may take most registers).
  constexpr int SB = MT <= 5 ? 8 : 4;
  auto sum_slots = [&](f32x4 (&s)[2][MT], const float* P, uint32_t pbytes, uint32_t first, int n) {
    const auto pres = make_rsrc(P, pbytes);
    for (int j = 0; j < n; j += SB) {
      f32x4 v[SB][2][MT];
#pragma unroll
      for (int h = 0; h < SB; ++h)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const uint32_t off = j + h < n ? (first + uint32_t(j + h)) * uint32_t(G::FRAG) + frag_off(rg, mt)
                                           : kMaskedOffset;
            v[h][rg][mt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pres, off, 0, kDeviceScope));
          }
#pragma unroll
      for (int h = 0; h < SB; ++h)
        if (j + h < n) {
#pragma unroll
          for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) s[rg][mt] += v[h][rg][mt];
        }
    }
  };

  // End of this block's part of W tile `key` (its W units there, and for its
  // last tile also its share of the tile's expand units).  `verdict` is a word
  // of the ring slot just consumed, free until the next barrier.
  auto tile_end = [&](int key, int& verdict) __attribute__((always_inline)) {
    const int64_t fw = int64_t(key) * d.nst;
    const int64_t bw0 = pblock(fw, UW, d.GW);
    const int nWp = int(pblock(fw + d.nst - 1, UW, d.GW) - bw0 + 1);
    store_partial(d.PW, d.pw_bytes, uint32_t(key * d.smaxW + (b - bw0)), t_lost != 0);
    wait_vm<0>();          // the partial is out (device scope) before the count
    __syncthreads();
    // 1: this block is the tile's last; 2: the count was already past the tile's
    // total (a counter area left non-zero), so this block stores NaN over the tile
    if (tid == 0) {
      const uint32_t old = arrive(cW + key, d.err, uint32_t(nWp));
      verdict = old + 1 == uint32_t(nWp) ? 1 : old + 1 > uint32_t(nWp) ? 2 : 0;
    }
    __syncthreads();
    if (verdict) {
      const int v = verdict;
      f32x4 s[2][MT];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) s[rg][mt] = f32x4{};
      if (v == 1) {
        sum_slots(s, d.PW, d.pw_bytes, uint32_t(key * d.smaxW), nWp);
      } else {
        const f32x4 nan4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) s[rg][mt] = nan4;
      }
      const auto yres = make_rsrc(d.Y, d.y_bytes);
      const bool vec = (d.N & 3) == 0;
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 16 + (lane & 15);
          const int n = key * TR + wave * 32 + rg * 16 + 4 * (lane >> 4);
          const uint32_t e0 = uint32_t(m) * uint32_t(d.N) + uint32_t(n);
          if (vec) {
            const bool ok = m < d.M && n < d.N;
            if constexpr (F32_OUT) {
              const u32x4 w{__float_as_uint(s[rg][mt][0]), __float_as_uint(s[rg][mt][1]),
                            __float_as_uint(s[rg][mt][2]), __float_as_uint(s[rg][mt][3])};
              __builtin_amdgcn_raw_buffer_store_b128(w, yres, ok ? e0 * 4u : kMaskedOffset, 0, 0);
            } else {
              const u32x2 w{pack2(s[rg][mt][0], s[rg][mt][1]), pack2(s[rg][mt][2], s[rg][mt][3])};
              __builtin_amdgcn_raw_buffer_store_b64(w, yres, ok ? e0 * 2u : kMaskedOffset, 0, 0);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool ok = m < d.M && n + e < d.N;
              if constexpr (F32_OUT)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s[rg][mt][e]), yres,
                                                      ok ? (e0 + e) * 4u : kMaskedOffset, 0, 0);
              else
                __builtin_amdgcn_raw_buffer_store_b16(uint16_t(bf16_bits(s[rg][mt][e])), yres,
                                                      ok ? (e0 + e) * 2u : kMaskedOffset, 0, 0);
            }
          }
        }
      if (tid == 0 && v == 1) {
        clear(cW + key);
        if (arrive(cF, d.err, uint32_t(d.ntW)) + 1 == uint32_t(d.ntW)) {   // the call is done: T and the A count are no longer read
          clear(cA);
          clear(cT);
          clear(cF);
        }
      }
    }
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[rg][mt] = f32x4{};
  };

  // Expand units read T: the first of them is fetched only once every T piece
  // is stored.
  bool gated = false;
  // `word` is a word of the ring slot about to be refilled: every wave reads the
  // verdict between the two barriers, before any load lands there.
  auto fetch_gate = [&](int* word) __attribute__((always_inline)) {
    if (gated) return;
    if (tid == 0) *word = wait_for(cT, t_want, spin, d.err) ? 0 : 1;
    __syncthreads();
    t_lost = *word;
    __syncthreads();
    gated = true;
  };
  // One look at the T count, taken by every wave alike: true once T is stored.
  // `word` is in a ring slot that no wave reads or refills before the second
  // barrier.
  auto try_gate = [&](int* word) __attribute__((always_inline)) {
    if (gated) return true;
    if (tid == 0) *word = __hip_atomic_load(cT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= t_want;
    __syncthreads();
    gated = *word != 0;
    __syncthreads();
    return gated;
  };

  // Stream units through the ring: n0 units of kind K0 from cursor c0, then
  // n1 expand units from cursor c1 (which continue the tile c0's units end in,
  // into the same accumulators).  The ring runs on across the change of kind;
  // each of the two loops multiplies one kind, fixed at compile time.  If T is
  // not stored when the first expand unit is due for fetching, the expand
  // fetches are deferred: the W units already in the ring are multiplied
  // meanwhile (the ring waits count only those), and after the last of them
  // the block waits for T and issues the expand units it skipped.
  auto run = [&](auto k0c, Cur c0, int n0, Cur c1, int n1) __attribute__((always_inline)) {
    constexpr Kind K0 = decltype(k0c)::value;
    const int n = n0 + n1;
    Cur ci = c0, cc = c0;   // next unit to fetch / to multiply
    bool deferred = false;  // expand fetches held back until the last W unit
    auto fetch = [&](int p) __attribute__((always_inline)) {   // unit p of the sequence into ring slot p % NS
      if (p < n0) {
        issue(p % G::NS, ci, K0);
        if (p + 1 == n0) ci = c1;
        else advance(ci, K0);
      } else {
        if (p == n0) fetch_gate(reinterpret_cast<int*>(smem + (p % G::NS) * G::STAGE));
        issue(p % G::NS, ci, KIND_E);
        advance(ci, KIND_E);
      }
    };
    auto step = [&](int i, auto kc) __attribute__((always_inline)) {   // multiply unit i (of kind kc)
      constexpr Kind K = decltype(kc)::value;
      const int ahead = min(G::NS - 2, (deferred ? n0 : n) - 1 - i);
      if (wave < G::NA) wait_ring<G::PWA, G::NS>(ahead);
      else wait_ring<G::PWB, G::NS>(ahead);
      __syncthreads();
      const int p = i + G::NS - 1;
      if (p < n) {
        if (p < n0) fetch(p);
        else if (!deferred) {
          if (p > n0 || try_gate(reinterpret_cast<int*>(smem + (p % G::NS) * G::STAGE))) fetch(p);
          else deferred = true;
        }
      }
      const char* ws = smem + (i % G::NS) * G::STAGE;
      const char* xs = ws + TR * RB;
      const int lim = K == KIND_E ? (RANKED ? at.rank[d.slot_adapter[cc.slot]] : d.rank) : d.K, e0 = cc.st * UK;
      // TAIL: zero the chunks at or past lim (a unit that reaches past it).
      // 4-bit weight units come in two versions, so that those short of lim
      // (every one when K is a multiple of 64) carry no test: as one version
      // the test became selects on every fragment register.  The bf16 units
      // keep one version with the test, which measured faster (a second
      // version cost the grouped bf16 stack 6%).
      const bool tail = lim - e0 < UK;
      auto multiply = [&](auto tail_c) __attribute__((always_inline)) {
        constexpr int TAIL = decltype(tail_c)::value;   // 0: none, 1: always, 2: if tail
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ch = 4 * j + (lane >> 4);
          bf16x8 a[2], bx[MT];
          if constexpr (Q4 && K == KIND_W) {
            // 8 codes of row 16 rg + lane % 16 (of this wave's 32), k = 32 j + 8 (lane / 16) ..,
            // dequantized with the row's group params: w = s (q - z), rounded to bf16
            const char* wq = ws + wave * 4096;
#pragma unroll
            for (int rg = 0; rg < 2; ++rg) {
              const int rr = rg * 16 + (lane & 15);
              const uint32_t codes = *reinterpret_cast<const uint32_t*>(wq + rr * 32 + j * 16 + (lane >> 4) * 4);
              const uint32_t prm = *reinterpret_cast<const uint32_t*>(wq + 1024 + rr * 4);
              const float sc = __uint_as_float(prm << 16);
              const float nsz = -sc * float((prm >> 16) & 0xFFu);     // -s z
              // even codes in the bytes of lo, odd codes in the bytes of hi;
              // code pair (2p, 2p+1) is byte p of each.  One byte-to-float
              // conversion (v_cvt_f32_ubyteN reads byte N in place) and one
              // fused multiply-add per code, one packed conversion per pair.
              // The masks are opaque to the compiler, which would otherwise
              // fold them into a shift and a mask per code.
              uint32_t lo, hi;
              asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(codes));
              asm("v_bfe_u32 %0, %1, 4, 28\n\tv_and_b32 %0, 0x0f0f0f0f, %0" : "=&v"(hi) : "v"(codes));
              u32x4 w;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float f0 = __builtin_fmaf(sc, float((lo >> (8 * q)) & 0xFFu), nsz);
                const float f1 = __builtin_fmaf(sc, float((hi >> (8 * q)) & 0xFFu), nsz);
                w[q] = __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(f0), static_cast<__bf16>(f1)});
              }
              a[rg] = __builtin_bit_cast(bf16x8, w);
            }
          } else {
#pragma unroll
            for (int rg = 0; rg < 2; ++rg) a[rg] = frag(ws, wave * 32 + rg * 16 + (lane & 15), ch);
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) bx[mt] = frag(xs, mt * 16 + (lane & 15), ch);
          if constexpr (TAIL != 0) {
            if ((TAIL == 1 || tail) && e0 + ch * 8 >= lim) {
#pragma unroll
              for (int rg = 0; rg < 2; ++rg) a[rg] = bf16x8{};
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) bx[mt] = bf16x8{};
            }
          }
#pragma unroll
          for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[rg][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rg], bx[mt], acc[rg][mt], 0, 0, 0);
        }
      };
      if constexpr (Q4 && K == KIND_W) {
        if (tail) multiply(std::integral_constant<int, 1>{});
        else multiply(std::integral_constant<int, 0>{});
      } else {
        multiply(std::integral_constant<int, 2>{});
      }
      if (deferred && i + 1 == n0) {   // the last W unit is multiplied: wait for T, issue the expand units
        deferred = false;
        for (int q = n0; q < min(n, i + G::NS); ++q) fetch(q);
      }
      const int key = cc.key;
      if (i + 1 == n0) cc = c1;
      else advance(cc, K);
      if (i + 1 == n || (i + 1 < n0 && cc.key != key)) {
        __syncthreads();   // every wave is done with this stage's slot
        if constexpr (K0 == KIND_A) {
          store_partial(d.PA, d.pa_bytes, uint32_t(key * d.GA + b), false);
#pragma unroll
          for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[rg][mt] = f32x4{};
        } else {
          tile_end(key, *reinterpret_cast<int*>(const_cast<char*>(ws)));
        }
      }
    };
#pragma unroll
    for (int p = 0; p < G::NS - 1; ++p)
      if (p < n) fetch(p);
    for (int i = 0; i < n0; ++i) step(i, k0c);
    for (int i = n0; i < n; ++i) step(i, std::integral_constant<Kind, KIND_E>{});
  };

  if (ablock) {
    // 1. this block's K range of every A tile
    if (ka1 > ka0)
      run(std::integral_constant<Kind, KIND_A>{}, Cur{0, ka0, 0, 0, 0}, nAt * (ka1 - ka0), Cur{0, 0, 0, 0, 0}, 0);
    wait_vm<0>();
    __syncthreads();
    // the ring is idle from here on: its first word carries this block's verdict
    int* word = reinterpret_cast<int*>(smem);
    if (tid == 0) *word = arrive(cA, d.err, uint32_t(d.GA)) + 1 > uint32_t(d.GA) ? 1 : 0;
    // A block with no T piece is done: it must not wait on the count either,
    // since the call's last tile clears it once every piece is in.
    if (b >= nAt * MT * 2) return;
    // every A block has stored its partials; if that never happens (or the count
    // was already past its total), this block's T pieces are stored as NaN
    if (tid == 0 && !wait_for(cA, u64(d.GA), d.spin_limit, d.err)) *word = 1;
    __syncthreads();
    const bool a_lost = *word != 0;
    // 2. T pieces (A tile g, 16-row tile mt, 16-column group rg), dealt round
    //    robin over the A blocks; each wave sums its own fragments of every A
    //    block's partial, all loads in flight at once.
    int done = 0;
    for (int item = b; item < nAt * MT * 2; item += d.GA, ++done) {
      const int g = item / (MT * 2), mt = (item / 2) % MT, rg = item & 1, sl = g / d.ntA;
      const auto pres = make_rsrc(d.PA, d.pa_bytes);
      f32x4 v[kDecodeMaxABlocks];
#pragma unroll
      for (int h = 0; h < kDecodeMaxABlocks; ++h) {
        const uint32_t off = h < d.GA ? uint32_t(g * d.GA + h) * uint32_t(G::FRAG) + frag_off(rg, mt) : kMaskedOffset;
        v[h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pres, off, 0, kDeviceScope));
      }
      f32x4 sum = f32x4{};
#pragma unroll
      for (int h = 0; h < kDecodeMaxABlocks; ++h)
        if (h < d.GA) sum += v[h];
      const auto thr = make_rsrc(d.TH, d.t_bytes), tlr = make_rsrc(d.TL, d.t_bytes);
      const int m = mt * 16 + (lane & 15);
      const bool mine = m < d.M && d.row_slot[m] == sl;
      const int j = (g % d.ntA) * TR + wave * 32 + rg * 16 + 4 * (lane >> 4);
      const bool ok = m < d.M && j < d.trank;
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float hi, lo;
        split_hi_lo(a_lost ? __builtin_nanf("") : mine ? at.scale[d.slot_adapter[sl]] * sum[e] : 0.0f, hi, lo);
        hb[e] = bf16_bits(hi);
        lb[e] = bf16_bits(lo);
      }
      const uint32_t off = ok ? (uint32_t(sl * d.M + m) * uint32_t(d.trank) + uint32_t(j)) * 2u : kMaskedOffset;
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)}, thr, off, 0,
                                            kDeviceScope);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)}, tlr, off, 0,
                                            kDeviceScope);
    }
    wait_vm<0>();           // T pieces are out before they are counted
    __syncthreads();
    if (tid == 0 && done) arrive(cT, d.err, t_total, uint32_t(done));
  } else {
    const int64_t uw0 = pstart(b, UW, d.GW), uw1 = pstart(b + 1, UW, d.GW);
    if (uw1 > uw0) {
      // Expand units: a tile this block covers whole and runs on past (no
      // other block touches it) gets all of them right after its W units; the
      // block's last tile gets this block's share, split evenly among the
      // blocks whose W units end in that tile.  Each piece of the range runs
      // as its own sequence: W units, then the expand units of the tile they
      // end in.
      const int t_last = int((uw1 - 1) / d.nst);
      int r0 = 0, r1 = 0;
      if (nEpt > 0) {
        const int64_t e_lo = pblock(int64_t(t_last) * d.nst, UW, d.GW);
        const int64_t bb = pblock(int64_t(t_last + 1) * d.nst - 1, UW, d.GW);
        const int64_t e_hi = pstart(bb + 1, UW, d.GW) == int64_t(t_last + 1) * d.nst ? bb : bb - 1;
        const int n_end = int(e_hi - e_lo + 1), idx = int(b - e_lo);
        r0 = idx * nEpt / n_end;
        r1 = (idx + 1) * nEpt / n_end;
      }
      int t = int((uw0 + d.nst - 1) / d.nst);   // first tile that starts inside the range
      for (int64_t u = uw0; u < uw1;) {
        int64_t end = uw1;
        Cur ce{t_last, r0 % d.nrs, r0 / (2 * d.nrs), 0, (r0 / d.nrs) & 1};
        int ne = r1 - r0;
        if (nEpt > 0 && t < t_last) {   // a whole tile: its W units, then all its expand units
          end = int64_t(t + 1) * d.nst;
          ce = Cur{t, 0, 0, 0, 0};
          ne = nEpt;
          ++t;
        }
        run(std::integral_constant<Kind, KIND_W>{}, Cur{int(u / d.nst), int(u % d.nst), 0, 0, 0}, int(end - u), ce, ne);
        u = end;
      }
    }
  }
}

// 4-bit calls take one rank for every adapter (lora_proj_q4), so only the bf16
// kernels come in a RANKED form.
template <int MT>
const void* pick(bool f32_out, bool q4, bool ranked) {
  if (q4)
    return f32_out ? reinterpret_cast<const void*>(&decode_kernel<MT, true, true, false>)
                   : reinterpret_cast<const void*>(&decode_kernel<MT, false, true, false>);
  if (ranked)
    return f32_out ? reinterpret_cast<const void*>(&decode_kernel<MT, true, false, true>)
                   : reinterpret_cast<const void*>(&decode_kernel<MT, false, false, true>);
  return f32_out ? reinterpret_cast<const void*>(&decode_kernel<MT, true, false, false>)
                 : reinterpret_cast<const void*>(&decode_kernel<MT, false, false, false>);
}

}  // namespace

int decode_mtiles(int64_t M) { return M <= 32 ? 2 : M <= 64 ? 4 : M <= 80 ? 5 : 8; }

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int64_t rank, int64_t trank, int64_t n_used) {
  DecodePlan p;
  p.MT = decode_mtiles(M);
  p.nst = int((K + UK - 1) / UK);
  p.nrs = int((rank + UK - 1) / UK);
  p.ntA = int((trank + TR - 1) / TR);
  p.ntW = int((N + TR - 1) / TR);
  p.n_used = int(n_used);
  const int64_t UW = int64_t(p.ntW) * p.nst;
  // A blocks: enough that one adapter's A units take each of them about 0.35
  // of a W block's units, so T is ready well before the W blocks reach the
  // expand (the A blocks also meet and reduce T after their units).  Planned
  // for one adapter of this width whatever the batch holds, so the W split
  // never depends on the adapter rows.
  const double lw = double(UW) / double(kDecodeBlocks - 16);
  int ga1 = int(std::ceil(double(p.ntA) * p.nst / (0.35 * lw)));
  ga1 = std::max(1, std::min({ga1, kDecodeMaxABlocks, p.nst}));
  // W blocks: the rest of the CUs (never more, so every block of the grid is
  // resident at once).  A tile that one block covers whole and runs past gets
  // its expand units from that block.
  p.GW = int(std::min<int64_t>(kDecodeBlocks - ga1, UW));
  p.GA = n_used > 0 ? ga1 : 0;
  // partial slots per W tile: the most blocks that share one tile
  p.smaxW = 0;
  for (int64_t t = 0; t < p.ntW; ++t)
    p.smaxW = std::max<int>(p.smaxW, int(pblock((t + 1) * p.nst - 1, UW, p.GW) - pblock(t * p.nst, UW, p.GW) + 1));
  const size_t frag = size_t(4 * 2 * p.MT * 64 * 16);
  auto r256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  p.off_cnt = 0;
  p.off_pa = LORA_WORKSPACE_COUNTER_BYTES;
  p.pa_bytes = size_t(n_used * p.ntA) * size_t(p.GA) * frag;
  p.off_pw = p.off_pa + r256(p.pa_bytes);
  p.pw_bytes = size_t(p.ntW) * size_t(p.smaxW) * frag;
  p.off_th = p.off_pw + r256(p.pw_bytes);
  p.t_bytes = size_t(n_used) * size_t(M) * size_t(trank) * 2;
  p.off_tl = p.off_th + r256(p.t_bytes);
  p.total = p.off_tl + r256(p.t_bytes);
  return p;
}

namespace {
__global__ void clear_words_kernel(uint32_t* p, int n) {
  for (int i = int(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += int(gridDim.x * blockDim.x)) p[i] = 0;
}
}  // namespace

hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  void* args[] = {&p, &n};
  return hipLaunchKernel(reinterpret_cast<const void*>(&clear_words_kernel), dim3(unsigned((n + 255) / 256)),
                         dim3(256), args, 0, stream);
}

hipError_t launch_decode(const DecodeArgs& d, const AdapterTable& at, int MT, bool f32_out, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
  const bool q4 = d.WP != nullptr, ranked = d.ranks_differ != 0;
  if (q4 && ranked) return hipErrorInvalidValue;
  const void* k = MT == 2   ? pick<2>(f32_out, q4, ranked)
                  : MT == 4 ? pick<4>(f32_out, q4, ranked)
                  : MT == 5 ? pick<5>(f32_out, q4, ranked)
                            : pick<8>(f32_out, q4, ranked);
  DecodeArgs dd = d;
  AdapterTable aa = at;
  void* args[] = {&dd, &aa};
  return hipExtLaunchKernel(k, dim3(unsigned(d.GA + d.GW)), dim3(256), args, 0, stream, ev_start, ev_stop, 0);
}

}  // namespace lora
