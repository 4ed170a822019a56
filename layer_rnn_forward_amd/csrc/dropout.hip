// Inter-layer dropout (gfx950): the keep mask of layer l's input is drawn
// from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11), a keyed bijection of a 4-word
// counter, so any kernel can recompute any element's decision and no mask is
// stored.  Element e of the [T][B][D*H] input takes word e mod 4 of the
// generator at counter (q mod 2^32, q div 2^32, l, 0), q = e div 4, under the
// key (seed mod 2^32, seed div 2^32); it is kept when that word is at least
// floor(p * 2^32) and then scaled by 1/(1-p).
//
// One thread per counter (4 consecutive elements, one 16-byte load and
// store): an HBM-bound pass, 8 bytes per element, with ~15 integer
// operations per element of generator work hidden under the memory traffic.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "philox.h"
#include "rnn_common.h"

namespace {

struct DropParams {
  const float* src;        // may equal dst
  float* dst;              // or null: write the mask instead
  uint8_t* mask;           // 1 = kept, or null
  long long n;             // elements
  uint32_t k0, k1;         // seed words
  uint32_t layer;
  unsigned long long thr;  // drop when the word is below this (0 .. 2^32)
  float scale;             // 1/(1-p), 0 when p = 1
};

template <bool VEC>
__global__ __launch_bounds__(256) void dropout_kernel(const DropParams p) {
  const long long nq = (p.n + 3) >> 2;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long q = (long long)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += stride) {
    const rnnk::PhiloxOut w = rnnk::philox4x32_10((uint32_t)q, (uint32_t)((unsigned long long)q >> 32), p.layer, 0u,
                               p.k0, p.k1);
    const long long e0 = q * 4;
    bool keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) keep[i] = (unsigned long long)w.v[i] >= p.thr;
    if (p.mask) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e0 + i < p.n) p.mask[e0 + i] = keep[i] ? 1 : 0;
    }
    if (!p.dst) continue;
    if (VEC && e0 + 3 < p.n) {
      float4 v = *reinterpret_cast<const float4*>(p.src + e0);
      v.x = keep[0] ? v.x * p.scale : 0.f;
      v.y = keep[1] ? v.y * p.scale : 0.f;
      v.z = keep[2] ? v.z * p.scale : 0.f;
      v.w = keep[3] ? v.w * p.scale : 0.f;
      *reinterpret_cast<float4*>(p.dst + e0) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e0 + i < p.n) p.dst[e0 + i] = keep[i] ? p.src[e0 + i] * p.scale : 0.f;
    }
  }
}

}  // namespace

hipError_t rnn_launch_dropout(const float* src, float* dst, uint8_t* mask, long long n,
                              unsigned long long seed, int layer, double prob, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  DropParams p{};
  p.src = src;
  p.dst = dst;
  p.mask = mask;
  p.n = n;
  p.k0 = (uint32_t)(seed & 0xFFFFFFFFull);
  p.k1 = (uint32_t)(seed >> 32);
  p.layer = (uint32_t)layer;
  // floor(p * 2^32) is exact in double (a power-of-two scaling)
  p.thr = (unsigned long long)std::floor(prob * 4294967296.0);
  p.scale = prob < 1.0 ? (float)(1.0 / (1.0 - prob)) : 0.f;
  const long long nq = (n + 3) / 4;
  const int grid = (int)std::min<long long>((nq + 255) / 256, 256LL * 16);
  const bool vec = dst && (((uintptr_t)src | (uintptr_t)dst) & 15u) == 0;
  if (vec) hipLaunchKernelGGL(dropout_kernel<true>, dim3(grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(dropout_kernel<false>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}
