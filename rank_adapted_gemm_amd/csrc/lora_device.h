// Device helpers shared by the bf16 kernels (prefill and decode paths).
#pragma once

#include "lora_internal.h"

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // word3 0x00020000: raw 32-bit data, no swizzle (gfx9 family)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// The same descriptor as four words, for the inline-assembly loads.
__device__ __forceinline__ i32x4 make_rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return i32x4{int32_t(uint32_t(a)), int32_t(uint32_t(a >> 32) & 0xFFFFu), int32_t(bytes), 0x00020000};
}

// The descriptor of make_rsrc_words as a buffer resource, for the builtin loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of_words(const i32x4& w) {
  const uint64_t base = uint64_t(uint32_t(w[0])) | (uint64_t(uint32_t(w[1]) & 0xFFFFu) << 32);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), (short)0, w[2], 0x00020000);
}

// Global -> LDS: one buffer_load_dwordx4 with the lds flag writes 64 lanes x
// 16 bytes contiguously at M0.  Issued from inline assembly (M0 is set in the
// same statement), so completion is tracked by explicit vmcnt waits.
__device__ __forceinline__ void dma16(const i32x4& res, uint32_t voff, uint32_t lds_addr) {
  const i32x4 r{__builtin_amdgcn_readfirstlane(res[0]), __builtin_amdgcn_readfirstlane(res[1]),
                __builtin_amdgcn_readfirstlane(res[2]), __builtin_amdgcn_readfirstlane(res[3])};
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory");
}

// The same load with device-scope coherence (sc1): it reads what other CUs
// published, past any stale copy in this XCD's L2.
__device__ __forceinline__ void dma16_dev(const i32x4& res, uint32_t voff, uint32_t lds_addr) {
  const i32x4 r{__builtin_amdgcn_readfirstlane(res[0]), __builtin_amdgcn_readfirstlane(res[1]),
                __builtin_amdgcn_readfirstlane(res[2]), __builtin_amdgcn_readfirstlane(res[3])};
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen sc1 lds" : : "v"(voff), "s"(r),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory");
}

// Cache-policy operand of the buffer load/store builtins: device scope (sc1).
constexpr int kDeviceScope = 16;

// Offset for a masked lane of dma16_group: past the end of every operand even
// after subtracting the group's instruction offsets (at most 3 KiB).
constexpr uint32_t kDmaMaskedOffset = 0xFFFFF000u;

// Up to four wave-wide 16-byte global -> LDS loads under one M0 value: load i
// reads voff[i] and lands at lds_addr + 1024 * i.  The instruction offset
// (i KiB) moves the LDS destination and the memory address alike, so voff[i]
// is biased down by the same amount.  Rewriting M0 before every LDS-DMA load
// holds the wave until the previous one has left; a wave that writes M0 once
// per group of four moves about 2.6 times as many bytes.  Masked lanes pass
// kDmaMaskedOffset.  SC1 selects device-scope (sc1) loads.
template <int NL, bool SC1 = false>
__device__ __forceinline__ void dma16_group(const i32x4& res, const uint32_t (&voff)[NL], uint32_t lds_addr) {
  static_assert(NL >= 1 && NL <= 4, "one M0 covers at most four 1 KiB blocks (instruction offset < 4 KiB)");
  const i32x4 r{__builtin_amdgcn_readfirstlane(res[0]), __builtin_amdgcn_readfirstlane(res[1]),
                __builtin_amdgcn_readfirstlane(res[2]), __builtin_amdgcn_readfirstlane(res[3])};
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  const uint32_t v0 = voff[0];
  const uint32_t v1 = NL > 1 ? voff[NL > 1 ? 1 : 0] - 1024u : 0u;
  const uint32_t v2 = NL > 2 ? voff[NL > 2 ? 2 : 0] - 2048u : 0u;
  const uint32_t v3 = NL > 3 ? voff[NL > 3 ? 3 : 0] - 3072u : 0u;
  if constexpr (NL == 1) {
    if constexpr (SC1)
      asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen sc1 lds" : : "v"(v0), "s"(m0), "s"(r)
                   : "memory");
    else
      asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds" : : "v"(v0), "s"(m0), "s"(r)
                   : "memory");
  } else if constexpr (NL == 2) {
    if constexpr (SC1)
      asm volatile("s_mov_b32 m0, %2\n\t"
                   "buffer_load_dwordx4 %0, %3, 0 offen sc1 lds\n\t"
                   "buffer_load_dwordx4 %1, %3, 0 offen offset:1024 sc1 lds"
                   : : "v"(v0), "v"(v1), "s"(m0), "s"(r) : "memory");
    else
      asm volatile("s_mov_b32 m0, %2\n\t"
                   "buffer_load_dwordx4 %0, %3, 0 offen lds\n\t"
                   "buffer_load_dwordx4 %1, %3, 0 offen offset:1024 lds"
                   : : "v"(v0), "v"(v1), "s"(m0), "s"(r) : "memory");
  } else if constexpr (NL == 3) {
    if constexpr (SC1)
      asm volatile("s_mov_b32 m0, %3\n\t"
                   "buffer_load_dwordx4 %0, %4, 0 offen sc1 lds\n\t"
                   "buffer_load_dwordx4 %1, %4, 0 offen offset:1024 sc1 lds\n\t"
                   "buffer_load_dwordx4 %2, %4, 0 offen offset:2048 sc1 lds"
                   : : "v"(v0), "v"(v1), "v"(v2), "s"(m0), "s"(r) : "memory");
    else
      asm volatile("s_mov_b32 m0, %3\n\t"
                   "buffer_load_dwordx4 %0, %4, 0 offen lds\n\t"
                   "buffer_load_dwordx4 %1, %4, 0 offen offset:1024 lds\n\t"
                   "buffer_load_dwordx4 %2, %4, 0 offen offset:2048 lds"
                   : : "v"(v0), "v"(v1), "v"(v2), "s"(m0), "s"(r) : "memory");
  } else {
    if constexpr (SC1)
      asm volatile("s_mov_b32 m0, %4\n\t"
                   "buffer_load_dwordx4 %0, %5, 0 offen sc1 lds\n\t"
                   "buffer_load_dwordx4 %1, %5, 0 offen offset:1024 sc1 lds\n\t"
                   "buffer_load_dwordx4 %2, %5, 0 offen offset:2048 sc1 lds\n\t"
                   "buffer_load_dwordx4 %3, %5, 0 offen offset:3072 sc1 lds"
                   : : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(m0), "s"(r) : "memory");
    else
      asm volatile("s_mov_b32 m0, %4\n\t"
                   "buffer_load_dwordx4 %0, %5, 0 offen lds\n\t"
                   "buffer_load_dwordx4 %1, %5, 0 offen offset:1024 lds\n\t"
                   "buffer_load_dwordx4 %2, %5, 0 offen offset:2048 lds\n\t"
                   "buffer_load_dwordx4 %3, %5, 0 offen offset:3072 lds"
                   : : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(m0), "s"(r) : "memory");
  }
}

// Four wave-wide 16-byte global -> LDS loads under one M0, landing at lds_addr
// + 1024 i; voff[i] already carries the bias -1024 i that the instruction
// offsets undo (a loop that keeps its offsets across stages biases them once).
__device__ __forceinline__ void dma16x4_biased(const i32x4& res, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                               uint32_t lds_addr) {
  const i32x4 r{__builtin_amdgcn_readfirstlane(res[0]), __builtin_amdgcn_readfirstlane(res[1]),
                __builtin_amdgcn_readfirstlane(res[2]), __builtin_amdgcn_readfirstlane(res[3])};
  asm volatile("s_mov_b32 m0, %4\n\t"
               "buffer_load_dwordx4 %0, %5, 0 offen lds\n\t"
               "buffer_load_dwordx4 %1, %5, 0 offen offset:1024 lds\n\t"
               "buffer_load_dwordx4 %2, %5, 0 offen offset:2048 lds\n\t"
               "buffer_load_dwordx4 %3, %5, 0 offen offset:3072 lds"
               : : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"(r)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory"); }

// LDS byte offset of a pointer into a __shared__ array (M0 takes LDS addresses).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
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

// hi = bf16(t), lo = bf16(t - hi): t - hi is exact in fp32 (the two share
// their leading bits), so hi + lo carries t to about 2^-17 relative.
__device__ __forceinline__ void split_hi_lo(float t, float& hi, float& lo) {
  hi = static_cast<float>(static_cast<__bf16>(t));
  lo = t - hi;
}

}  // namespace lora
