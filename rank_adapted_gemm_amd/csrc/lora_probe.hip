// Measurement probes (dense MFMA rate, streaming-read rate); see lora_probe.h.
#include <cstdint>

#include "lora_device.h"
#include "lora_probe.h"

namespace lora {
namespace {

constexpr int kProbeBlocks = 1024;   // 4 per CU, 4 waves each
constexpr int kChains = 4;           // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = __bf16(float(lane + e + 1) * (1.0f / 1024.0f));
    b[e] = __bf16(float(64 - lane + e) * (1.0f / 1024.0f));
  }
  f32x16 acc[kChains] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (s == -1.0f) sink[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         float* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i), v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride), v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= v0.x ^ v1.y ^ v2.z ^ v3.w;
  }
  for (; i < n16; i += stride) x ^= src[i].x;
  if (x == 0x9e3779b9u) sink[blockIdx.x & 1023] = 1.0f;
}

}  // namespace
}  // namespace lora

extern "C" {

lora_status lora_probe_mfma_bf16(int32_t iters, float* sink, double* flop, hipStream_t stream) {
  if (iters < 1 || iters > (1 << 24) || !sink || !flop) return LORA_EINVAL;
  hipLaunchKernelGGL(lora::mfma_probe_kernel, dim3(lora::kProbeBlocks), dim3(256), 0, stream, int(iters), sink);
  if (hipGetLastError() != hipSuccess) return LORA_EHIP;
  *flop = double(lora::kProbeBlocks) * 4 * double(iters) * lora::kChains * (32.0 * 32.0 * 16.0 * 2.0);
  return LORA_OK;
}

lora_status lora_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || bytes >= (size_t(1) << 40) ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return LORA_EINVAL;
  hipLaunchKernelGGL(lora::read_probe_kernel, dim3(lora::kProbeBlocks * 8), dim3(256), 0, stream,
                     static_cast<const lora::u32x4*>(src), int64_t(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_EHIP;
}

}  // extern "C"
