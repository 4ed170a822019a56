// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11) and the inter-layer dropout decision built on it.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rnnk {

struct PhiloxOut {
  uint32_t v[4];
};

// Keyed bijection of a 4-word counter.  Round: words 0 and 2 are multiplied
// by M0 and M1; the new words are (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2),
// hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); the key advances by the Weyl increments
// (W0, W1) between rounds.
__device__ __forceinline__ PhiloxOut philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                   uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = __umulhi(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return PhiloxOut{{c0, c1, c2, c3}};
}

// Dropout multiplier of element e of layer `layer`'s [T][B][D*H] input:
// word e mod 4 at counter (e div 4 mod 2^32, e div 4 div 2^32, layer, 0)
// under the key (k0, k1); kept (multiplier `scale`) when the word is at least
// `thr`, else 0.
__device__ __forceinline__ float dropout_mult(unsigned long long e, uint32_t layer, uint32_t k0,
                                              uint32_t k1, unsigned long long thr, float scale) {
  const unsigned long long q = e >> 2;
  const PhiloxOut w = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), layer, 0u, k0, k1);
  const int i = (int)(e & 3ull);
  const uint32_t word = i == 0 ? w.v[0] : i == 1 ? w.v[1] : i == 2 ? w.v[2] : w.v[3];
  return (unsigned long long)word >= thr ? scale : 0.f;
}

}  // namespace rnnk
