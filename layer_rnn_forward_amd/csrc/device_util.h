// Device helpers for gfx950: MFMA fragments, bf16 rounding, coherence.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnnk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even: gfx950's v_cvt_pk_bf16_f32
// (one instruction in place of the software rounding -- add 0x7fff plus the
// lowest kept bit, keep the upper half; rnn_bf16_rounding_check compares the
// two over every fp32 pattern on the device: same bits for every non-NaN
// value, NaNs stay NaN).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
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

// Logistic and tanh from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32, about 1 ulp each): sigmoid(a) = 1 / (1 + 2^(-a log2 e));
// tanh(a) = sign(a) (1 - 2 / (1 + e^(2|a|))) for |a| >= 1/4, and its Taylor
// series through the a^11 term below that (truncation < 1e-9 relative), which
// avoids the cancellation of the identity near zero.
__device__ __forceinline__ float sigmoidf_(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * a));
}
// SELECT: evaluate both forms and pick one (no divergent branch between the
// lanes of the two ranges), else branch; which is faster depends on the
// kernel's register allocation, so the caller chooses (same results).
template <bool SELECT = true>
__device__ __forceinline__ float tanhf_(float a) {
  const float x = fabsf(a);
  if constexpr (SELECT) {
    const float z = a * a;
    float r = (-1382.0f / 155925.0f) * z + 62.0f / 2835.0f;
    r = r * z - 17.0f / 315.0f;
    r = r * z + 2.0f / 15.0f;
    r = r * z - 1.0f / 3.0f;
    float small = a + a * z * r;
    float big = copysignf(1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(2.8853900817779268f * x)), a);
    // (an empty asm statement that uses both keeps the compiler from sinking
    // either form back into a branch)
    asm volatile("" : "+v"(small), "+v"(big));
    return x < 0.25f ? small : big;
  } else {
    if (x < 0.25f) {
      const float z = a * a;
      float r = (-1382.0f / 155925.0f) * z + 62.0f / 2835.0f;
      r = r * z - 17.0f / 315.0f;
      r = r * z + 2.0f / 15.0f;
      r = r * z - 1.0f / 3.0f;
      return a + a * z * r;
    }
    return copysignf(1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(2.8853900817779268f * x)), a);
  }
}

// ---------------------------------------------------------------- coherence
// Agent-scope (sc1) loads and stores: coherent across the XCDs' L2 caches.
__device__ __forceinline__ unsigned flag_load(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace rnnk
