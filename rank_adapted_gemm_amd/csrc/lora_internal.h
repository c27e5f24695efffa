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

struct AdapterTable {
  const void* A[LORA_MAX_ADAPTERS];           // r x K each (device)
  const void* B[LORA_MAX_ADAPTERS];           // N x r each (device)
};

// Shapes and buffers of one call.  Byte extents bound every buffer access:
// loads past them read zero and stores past them are dropped by the hardware.
struct ProjArgs {
  const void* X;
  const void* W;
  void* Y;
  void* T;            // workspace: s X A^T for adapter rows, indexed by global row
  int32_t M, N, K, rank;
  float scale;
  uint32_t x_bytes, w_bytes, y_bytes, t_bytes;
  uint32_t a_bytes, b_bytes;   // extent of every A_a / B_a
};

// Byte offset used for masked accesses: past the end of every operand
// (each operand is smaller than 2 GiB).
constexpr uint32_t kMaskedOffset = 0x80000000u;

// Largest M served by the small-M (decode) path.
constexpr int kDecodeMaxRows = 128;

// Decode path (M <= kDecodeMaxRows).  Three launches:
//   partial: split-K products of X against 64-row tiles of W (fp32 partials
//            P[s][m][n]) and of each used adapter's A (partials PT[s][m][slot][j]);
//   reduce:  T = s * sum_s PT[s] on the rows of each adapter, stored as bf16
//            hi + lo (zero on other rows);
//   finish:  Y = sum_s P[s] + T B^T, one store.
// The split of W over K depends only on (N, K), never on the segment table, so
// base-only rows come out identical with or without adapter rows beside them.
constexpr int kDecodeTile = 64;         // rows of W / A per partial tile, columns per finish tile
constexpr int kDecodeStageK = 64;       // K elements per pipeline stage
constexpr int kDecodeTargetBlocks = 512;

struct DecodeArgs {
  const void* X;
  const void* W;
  void* Y;
  float* P;             // [S][M][N]
  float* PT;            // [S][M][n_used][rank]
  uint16_t* TH;         // [n_used][M][rank] bf16 hi part of T
  uint16_t* TL;         // [n_used][M][rank] bf16 lo part of T
  uint32_t x_bytes, w_bytes, y_bytes, a_bytes, b_bytes, p_bytes, pt_bytes, t_bytes;
  int32_t M, N, K, rank;
  float scale;
  int32_t nstages;      // ceil(K / kDecodeStageK)
  int32_t S, sc;        // W splits over K and stages per split
  int32_t n_wtiles;     // ceil(N / kDecodeTile)
  int32_t n_atiles;     // ceil(rank / kDecodeTile), per used adapter
  int32_t n_used;       // adapters named by at least one row
  int8_t row_slot[kDecodeMaxRows];           // slot of each row's adapter, -1 for base-only rows
  int8_t slot_adapter[LORA_MAX_ADAPTERS];    // adapter index of each slot
};

// Split factors of the decode path for a shape.
struct DecodeSplit {
  int nstages, S, sc;
};
DecodeSplit decode_split(int64_t N, int64_t K);
size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t rank, int64_t n_used);

// Launchers (return the HIP status of the launch).
hipError_t launch_bf16_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                              bool small_m, hipStream_t stream);
hipError_t launch_bf16_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                            bool has_adapter, bool f32_out, bool small_m, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_decode(const DecodeArgs& d, const AdapterTable& at, bool f32_out, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_f32_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                             hipStream_t stream);
hipError_t launch_f32_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                           bool has_adapter, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace lora
