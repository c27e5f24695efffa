// 4-bit base weights on the prefill path: dequantize to bf16 once per call.
//
// "two 27B models on a single RTX 5090", section 4 memory figure: the card
// holds a 4-bit copy of the base weights beside the bf16 adapter.  Format (see
// lora_proj_q4): codes of row n packed two per byte along K, low nibble first;
// params[g][n] holds the bf16 scale s (bits 0-15) and the zero point z (bits
// 16-23) of the 128-wide group g of row n; w = s (q - z).
//
// A prefill call is bound by the MFMA pipes, so reading W as 4-bit codes saves
// nothing there; the codes are expanded into a bf16 copy in the workspace (one
// HBM pass, a few percent of the call) and the bf16 kernels run unchanged.
// Each thread turns 8 codes (4 bytes) into 8 bf16 weights (16 bytes): in fp32
// as fma(s, q, -s z) with -s z rounded once, then rounded to nearest even; the
// decode kernel computes its fragments the same way, so both paths see the
// same weights.
#include <algorithm>

#include "lora_device.h"

namespace lora {
namespace {

__global__ __launch_bounds__(256) void q4_dequant_kernel(const uint32_t* __restrict__ codes,
                                                         const uint32_t* __restrict__ params, u32x4* __restrict__ w,
                                                         int64_t N, int64_t K) {
  const int64_t per_row = K / 8;                  // 8-code words per row
  const int64_t total = N * per_row;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t n = i / per_row, k8 = i - n * per_row;
    const uint32_t c = codes[i];
    const uint32_t prm = params[(k8 * 8 / 128) * N + n];
    const float s = __uint_as_float(prm << 16);
    const float nsz = -s * float((prm >> 16) & 0xFFu);     // -s z
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __builtin_fmaf(s, float((c >> (8 * e)) & 0xFu), nsz);
      const float hi = __builtin_fmaf(s, float((c >> (8 * e + 4)) & 0xFu), nsz);
      o[e] = pack2(lo, hi);
    }
    w[i] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

}  // namespace

hipError_t launch_q4_dequant(const void* codes, const void* params, void* w, int64_t N, int64_t K,
                             hipStream_t stream) {
  const int64_t total = N * (K / 8);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 16);
  const uint32_t* c = static_cast<const uint32_t*>(codes);
  const uint32_t* p = static_cast<const uint32_t*>(params);
  u32x4* out = static_cast<u32x4*>(w);
  int64_t n = N, k = K;
  void* args[] = {&c, &p, &out, &n, &k};
  return hipLaunchKernel(reinterpret_cast<const void*>(&q4_dequant_kernel), dim3(unsigned(blocks)), dim3(256), args,
                         0, stream);
}

}  // namespace lora
