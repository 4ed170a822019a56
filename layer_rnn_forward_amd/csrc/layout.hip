// Operand preparation for the time-parallel GEMMs (gfx950): element-type
// conversion and row-gather transposes, so that every product reads both
// operands K-contiguous in the compute type (the "Matrix pre-transposition"
// row of the cuDNN-5 optimisation table in Keras issue #3692).
#include <type_traits>

#include "device_util.h"
#include "rnn_common.h"

using namespace rnnk;

namespace {

template <bool BF>
__device__ __forceinline__ float ld_elem(const void* p, size_t i) {
  if constexpr (BF) return bf2f(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}
template <bool BF>
__device__ __forceinline__ void st_elem(void* p, size_t i, float v) {
  if constexpr (BF) reinterpret_cast<uint16_t*>(p)[i] = f2bf(v);
  else reinterpret_cast<float*>(p)[i] = v;
}

// 64x64 tiles through LDS; 256 threads; each thread moves 16 elements.
template <bool IN_BF, bool OUT_BF>
__global__ __launch_bounds__(256) void transpose_kernel(const TransposeParams p) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rl = ty + 4 * i;
    const int r = r0 + rl, c = c0 + tx;
    float v = 0.f;
    if (r < p.R && c < p.C) {
      int lb = -1;   // alt row of a row whose successor is past its length
      if (p.lengths) {
        const int t = r / p.len_B, b = r - t * p.len_B;
        if (t + 1 >= min(max(p.lengths[b], 0), p.len_T)) lb = b;
      }
      if (lb >= 0) {
        if (p.alt) v = ld_elem<IN_BF>(p.alt, (size_t)lb * p.ld_alt + c);
      } else if (r >= p.alt_r0 && r < p.alt_r1) {
        if (p.alt) v = ld_elem<IN_BF>(p.alt, (size_t)(r - p.alt_r0) * p.ld_alt + c);
      } else {
        v = ld_elem<IN_BF>(p.src, (size_t)((long long)(r + p.shift) * p.ld_src) + c);
      }
    }
    tile[rl][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int cl = ty + 4 * i;
    const int c = c0 + cl, r = r0 + tx;
    if (c < p.C && r < p.R) st_elem<OUT_BF>(p.out, (size_t)c * p.ld_out + r, tile[tx][cl]);
  }
}

__global__ void convert_kernel(const float* src, long long ld_src, uint16_t* dst, long long ld_dst,
                               int rows, int cols) {
  const size_t n = (size_t)rows * cols;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / cols, c = i % cols;
    dst[r * ld_dst + c] = f2bf(src[r * ld_src + c]);
  }
}

}  // namespace

hipError_t rnn_launch_transpose(const TransposeParams& p, int in_bf16, int out_bf16, hipStream_t s) {
  if (p.R <= 0 || p.C <= 0) return hipSuccess;
  dim3 grid((p.C + 63) / 64, (p.R + 63) / 64);
  if (in_bf16 && out_bf16) hipLaunchKernelGGL((transpose_kernel<true, true>), grid, dim3(256), 0, s, p);
  else if (in_bf16 && !out_bf16) hipLaunchKernelGGL((transpose_kernel<true, false>), grid, dim3(256), 0, s, p);
  else if (!in_bf16 && out_bf16) hipLaunchKernelGGL((transpose_kernel<false, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((transpose_kernel<false, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t rnn_launch_convert(const float* src, long long ld_src, void* dst, long long ld_dst, int rows,
                              int cols, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  size_t n = (size_t)rows * cols;
  unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(convert_kernel, dim3(blocks), dim3(256), 0, s, src, ld_src,
                     reinterpret_cast<uint16_t*>(dst), ld_dst, rows, cols);
  return hipGetLastError();
}
