// Device helpers for gfx950: MFMA fragments, bf16 rounding, coherence.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnnk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// One K chunk of a 16x16 output tile from 16-byte A and B fragments held per
// lane (lane l: row/col l%16, k-group l/16).  bf16: one 16x16x32 MFMA over 8
// consecutive k per lane; fp32: four 16x16x4 MFMAs, lane k-group q holding k =
// 4q..4q+3 of a 16-wide chunk (the same k permutation on both operands, so the
// sum is the plain dot product).
template <bool BF16>
__device__ __forceinline__ f32x4 mfma_chunk(const uint4& a, const uint4& b, f32x4 c) {
  if constexpr (BF16) {
    bf16x8 av = __builtin_bit_cast(bf16x8, a);
    bf16x8 bv = __builtin_bit_cast(bf16x8, b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
  } else {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
}

// K values per MFMA chunk: 32 (bf16) or 16 (fp32); each lane holds a quarter.
template <bool BF16> constexpr int kchunk() { return BF16 ? 32 : 16; }

__device__ __forceinline__ float sigmoidf_(float a) { return 1.0f / (1.0f + expf(-a)); }

// ---------------------------------------------------------------- coherence
// Agent-scope flags.  Producer: every wave drains its stores, the workgroup
// barrier orders them before wave 0's agent release fence, then the flag is
// stored.  Consumer: relaxed agent loads of the flags, agent acquire fence,
// workgroup barrier, then ordinary loads of the data.
__device__ __forceinline__ unsigned flag_load(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ void release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

}  // namespace rnnk
