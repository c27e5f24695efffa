// Internal interface between the C-ABI layer (lora_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "lora_proj.h"

namespace lora {

// Segment table after host scheduling: empty segments dropped, neighbours that
// name the same adapter merged, so starts strictly increase.  Passed by value
// in the kernel arguments; each block finds the segments overlapping its rows
// with a binary search on `start`.
struct SegTable {
  int32_t n;                                  // number of segments, >= 1
  int32_t start[LORA_MAX_SEGMENTS + 1];       // start[n] == M
  int8_t adapter[LORA_MAX_SEGMENTS];          // -1 or adapter index
};

// Adapter-sorted shrink: the rows that name adapter a, over all its segments
// in row order, form one virtual row range of rows[a] rows, cut into tiles of
// kShrinkRows; tile_off[a] is the first such tile of adapter a and
// tile_off[n_adapters] the total, so every shrink tile belongs to one adapter
// however the batch interleaves them.
constexpr int kShrinkRows = 128;
struct ShrinkPlan {
  int32_t n_adapters;
  int32_t rows[LORA_MAX_ADAPTERS];
  int32_t tile_off[LORA_MAX_ADAPTERS + 1];
  // K split: `splits` blocks per tile, each over its share of the 64-wide
  // stages, store fp32 partials (kShrinkPartBytes per tile and split) at
  // `part`; a second kernel sums them in split order.  1: no split.
  int32_t splits;
  void* part;
  uint32_t part_bytes;
};
constexpr uint32_t kShrinkPartBytes = kShrinkRows * kShrinkRows * 4;
constexpr int kShrinkMaxSplits = 8;

// Adapter a has its own rank r_a (at most the call's rank r, the largest of
// them): A_a is (S r_a) x K and B_a is N x r_a, and its rows of T hold S r_a
// values (columns S r_a .. S r - 1 are never read for them).
struct AdapterTable {
  const void* A[LORA_MAX_ADAPTERS];           // (S r_a) x K each (device), S = number of slices
  const void* B[LORA_MAX_ADAPTERS];           // N x r_a each (device)
  float scale[LORA_MAX_ADAPTERS];             // s of each adapter's rows
  int32_t rank[LORA_MAX_ADAPTERS];            // r_a (0 for adapters no row names)
  uint32_t a_bytes[LORA_MAX_ADAPTERS];        // extent of A_a
  uint32_t b_bytes[LORA_MAX_ADAPTERS];        // extent of B_a
};

// Shapes and buffers of one call.  Byte extents bound every buffer access:
// loads past them read zero and stores past them are dropped by the hardware.
// Output columns are cut into slices (one slice for a plain call).  Slice s
// covers columns [slice_end[s-1], slice_end[s]) and its expand reads columns
// [s r, s r + r) of T, whose rows are trank = S r wide.
struct Slices {
  int32_t n;                                  // 1 .. LORA_MAX_SLICES
  int32_t end[LORA_MAX_SLICES];               // cumulative column ends, end[n-1] == N
};

// Slice holding output column `col`.
__host__ __device__ inline int slice_of(const Slices& sl, int col) {
  int s = 0;
  while (s + 1 < sl.n && col >= sl.end[s]) ++s;
  return s;
}

struct ProjArgs {
  const void* X;
  const void* W;
  void* Y;
  void* T;            // workspace: s_a X A_a^T for adapter rows, indexed by global row
  int32_t M, N, K, rank;   // rank: the largest adapter rank of the call
  int32_t trank;      // width of T: slices x rank
  Slices sl;
  uint32_t x_bytes, w_bytes, y_bytes, t_bytes;
};

// Byte offset used for masked accesses: past the end of every operand
// (each operand is smaller than 2 GiB).
constexpr uint32_t kMaskedOffset = 0x80000000u;

// Largest M served by the small-M (decode) path.
constexpr int kDecodeMaxRows = 128;

// Decode path (M <= kDecodeMaxRows): one launch.  Units are 64-element K slices
// of 128-row weight tiles.  A blocks (first in the grid) take one K range of
// every A_a tile each and then reduce T between them; W blocks split the W
// units evenly, each followed by its share of the expand units (B_a against T)
// of the tile its W units end in; the last block to finish a W tile sums the
// tile's fp32 partials in block order.  A wait that gives up, or a count found
// past its total, sets a sticky error bit in the last 8 bytes of the counter
// area, and the outputs that depended on the lost hand-over are stored as NaN.
constexpr int kDecodeTileRows = 128;
constexpr int kDecodeUnitK = 64;
constexpr int kDecodeBlocks = 256;      // one block per CU, all resident together
constexpr int kDecodeMaxABlocks = 32;   // blocks that compute T = s X A^T
constexpr uint32_t kDecodeErrTimeout = 1;   // a block gave up waiting for another block of its launch
constexpr uint32_t kDecodeErrCount = 2;     // a hand-over count went past its total

struct DecodeArgs {
  const void* X;
  const void* W;             // bf16 weights, or 4-bit codes when WP is set
  const void* WP;            // 4-bit params words [K/128][N], or null for bf16 weights
  void* Y;
  unsigned long long* cnt;   // counter area: arrivals per W tile, A blocks done, T pieces done, W tiles finished
  uint32_t* err;             // sticky error bits (last 8 bytes of the counter area)
  float* PA;                 // [A tile][A block] partials, fragment-major
  float* PW;                 // [W tile][slot]
  uint16_t* TH;              // [n_used][M][trank] bf16 hi part of T
  uint16_t* TL;              // [n_used][M][trank] bf16 lo part of T
  uint32_t x_bytes, w_bytes, y_bytes, t_bytes, pa_bytes, pw_bytes;
  uint32_t a_bytes, b_bytes; // extent of every A_a / B_a when all used adapters have rank `rank`
  int32_t ranks_differ;      // 1: adapters of different ranks (the kernel that reads each adapter's)
  uint32_t wp_bytes;
  int32_t M, N, K, rank;     // rank: the largest adapter rank of the call
  int32_t trank;             // width of T: slices x rank
  Slices sl;
  int32_t nst;               // units per tile along K: ceil(K / 64)
  int32_t nrs;               // expand units per tile per half: ceil(rank / 64)
  int32_t n_used;            // adapters named by at least one row
  int32_t ntA;               // A tiles per used adapter: ceil(trank / 128)
  int32_t ntW;               // W tiles: ceil(N / 128)
  int32_t GA, GW;            // A blocks, W blocks
  int32_t smaxW;             // partial slots per W tile
  uint32_t spin_limit;       // polls before a wait gives up
  int32_t fault;             // test hook: waits for T target one piece more than exist
  int8_t row_slot[kDecodeMaxRows];           // slot of each row's adapter, -1 for base-only rows
  int8_t slot_adapter[LORA_MAX_ADAPTERS];    // adapter index of each slot
};

// Grid split and workspace layout of a decode call.  Everything but the
// adapter work depends on (M, N, K, rank) only.
struct DecodePlan {
  int MT;                    // 16-row activation tiles: 2, 4, 5 or 8
  int nst, nrs, ntA, ntW, n_used;
  int GA, GW, smaxW;
  size_t off_cnt, off_pa, pa_bytes, off_pw, pw_bytes, off_th, t_bytes, off_tl, total;
};
DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int64_t rank, int64_t trank, int64_t n_used);
int decode_mtiles(int64_t M);

// Activation rows per output tile of the prefill output kernel for an M x N
// call (256, 192 or 128), chosen by whole waves of tiles over the CUs.
int main_tile_rows(int M, int N);

// Launchers (return the HIP status of the launch).
hipError_t launch_bf16_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at, const ShrinkPlan& sp,
                              hipStream_t stream);
hipError_t launch_bf16_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                            bool has_adapter, bool f32_out, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_decode(const DecodeArgs& d, const AdapterTable& at, int MT, bool f32_out, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop);
// Zero n 32-bit words on the stream (a kernel, so the fill may sit in a captured graph).
hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t stream);
// 4-bit weights: dequantize codes + params (N x K) into bf16 W (prefill path).
hipError_t launch_q4_dequant(const void* codes, const void* params, void* w, int64_t N, int64_t K, hipStream_t stream);
// Adapter extraction (lora_extract.hip).
size_t extract_workspace_bytes(int64_t N, int64_t K, int64_t l, int64_t r);
hipError_t launch_extract(const void* w_adapted, const void* w_base, int64_t N, int64_t K, const float* omega,
                          int l, int r, int power_iters, float* b_out, float* a_out, float* sigma_out,
                          void* workspace, hipStream_t s);
hipError_t launch_f32_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                             hipStream_t stream);
hipError_t launch_f32_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                           bool has_adapter, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace lora
