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

// Largest M served by the small-M (decode) tiling.
constexpr int kDecodeMaxRows = 128;

// Launchers (return the HIP status of the launch).
hipError_t launch_bf16_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                              bool small_m, hipStream_t stream);
hipError_t launch_bf16_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                            bool has_adapter, bool f32_out, bool small_m, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_f32_shrink(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                             hipStream_t stream);
hipError_t launch_f32_main(const ProjArgs& p, const SegTable& st, const AdapterTable& at,
                           bool has_adapter, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace lora
