// Operand preparation for the time-parallel GEMMs (gfx950): element-type
// conversion and row-gather transposes, so that every product reads both
// operands K-contiguous in the compute type (the "Matrix pre-transposition"
// row of the cuDNN-5 optimisation table in Keras issue #3692).
#include <algorithm>
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

// Source row of input row r (null: a row of zeros).  With lengths, row
// r = t*len_B + b reads alt row b once t + 1 reaches the row's clamped length;
// rows in [alt_r0, alt_r1) read alt rows from 0; every other row reads src row
// r + shift.
template <bool BF>
__device__ __forceinline__ const char* src_row(const TransposeParams& p, int r) {
  constexpr int ES = BF ? 2 : 4;
  int lb = -1;
  if (p.lengths) {
    const int t = r / p.len_B, b = r - t * p.len_B;
    if (t + 1 >= min(max(p.lengths[b], 0), p.len_T)) lb = b;
  }
  if (lb >= 0) return p.alt ? reinterpret_cast<const char*>(p.alt) + (size_t)lb * p.ld_alt * ES : nullptr;
  if (r >= p.alt_r0 && r < p.alt_r1)
    return p.alt ? reinterpret_cast<const char*>(p.alt) + (size_t)(r - p.alt_r0) * p.ld_alt * ES : nullptr;
  return reinterpret_cast<const char*>(p.src) + (size_t)((long long)(r + p.shift) * p.ld_src) * ES;
}

// 64x64 tiles through LDS, 256 threads.  Loads: a thread reads 4 consecutive
// columns of one row (one 16-byte fp32 or 8-byte bf16 access when p.vec_in);
// stores: a thread writes 8 consecutive rows of one output row (one 16-byte
// bf16 or two 16-byte fp32 accesses when p.vec_out).  Both flags are set by
// the host only when every row start and the tile edges keep the accesses
// aligned and inside the matrix; otherwise element accesses are used.
// Up to four independent transposes in one launch (blockIdx.z selects one);
// a z slice past them, if present, sets the fill ranges instead.
struct TransposeBatch {
  TransposeParams p[4];
  int n;          // transposes
  FillJob fill;   // fill.count > 0: one more z slice
};

template <bool IN_BF, bool OUT_BF>
__global__ __launch_bounds__(256) void transpose_kernel(const TransposeBatch batch) {
  __shared__ float tile[64][65];
  if ((int)blockIdx.z >= batch.n) {
    const size_t nb = (size_t)gridDim.x * gridDim.y;
    const size_t t0 = ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    for (int j = 0; j < batch.fill.count; ++j) {
      uint32_t* q = reinterpret_cast<uint32_t*>(batch.fill.p[j]);
      const size_t nw = batch.fill.bytes[j] / 4;
      for (size_t i = t0; i < nw; i += nb * blockDim.x) q[i] = batch.fill.v[j];
    }
    return;
  }
  const TransposeParams& p = batch.p[blockIdx.z];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (r0 >= p.R || c0 >= p.C) return;   // the grid covers the largest job
  const int tid = threadIdx.x;
  const int cg = (tid & 15) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = (tid >> 4) + 16 * i;
    const int r = r0 + rl, c = c0 + cg;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    // the input row of output index r (a permuted reduction index: map)
    int rn = r;
    if (p.map == 1) rn = gg_col_source(r, p.mU, p.mG, p.mH, p.mNwg);
    else if (p.map == 2) rn = tb_k_source(r, p.mBc, p.mT, p.mB);
    const char* row = (r < p.R && rn >= 0) ? src_row<IN_BF>(p, rn) : nullptr;
    if (row) {
      if (p.vec_in && c + 3 < p.C) {
        if constexpr (IN_BF) {
          const uint2 u = *reinterpret_cast<const uint2*>(row + (size_t)c * 2);
          v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
          v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
          const float4 f = *reinterpret_cast<const float4*>(row + (size_t)c * 4);
          v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < p.C) v[e] = ld_elem<IN_BF>(row, (size_t)(c + e));
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[rl][cg + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int item = tid + 256 * j;
    const int cl = item >> 3, rg = (item & 7) * 8;
    const int c = c0 + cl, r = r0 + rg;
    if (c >= p.C) continue;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[rg + e][cl];
    if (p.vec_out && r + 7 < p.R) {
      if constexpr (OUT_BF) {
        const uint4 u = make_uint4(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]), pack2bf(v[4], v[5]),
                                   pack2bf(v[6], v[7]));
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + (size_t)c * p.ld_out + r) = u;
      } else {
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + (size_t)c * p.ld_out + r);
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (r + e < p.R) st_elem<OUT_BF>(p.out, (size_t)c * p.ld_out + r + e, v[e]);
    }
  }
}

// fp32 -> bf16 (round to nearest even).  Vector path (cols % 8 == 0 and every
// row start 16-byte aligned on both sides): a thread converts 8 consecutive
// elements with two 16-byte loads and one 16-byte store.
// The first `fill_blocks` blocks of the launch set the fill ranges instead.
__global__ void convert_kernel(const float* src, long long ld_src, uint16_t* dst, long long ld_dst,
                               int rows, int cols, int vec, const FillJob fill, int fill_blocks) {
  if ((int)blockIdx.x < fill_blocks) {
    const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (size_t)fill_blocks * blockDim.x;
    for (int j = 0; j < fill.count; ++j) {
      uint32_t* q = reinterpret_cast<uint32_t*>(fill.p[j]);
      const size_t nw = fill.bytes[j] / 4;
      for (size_t i = t0; i < nw; i += stride) q[i] = fill.v[j];
    }
    return;
  }
  const size_t bid = blockIdx.x - fill_blocks, nblk = gridDim.x - fill_blocks;
  if (vec) {
    const int cv = cols >> 3;
    const size_t n = (size_t)rows * cv;
    for (size_t i = bid * blockDim.x + threadIdx.x; i < n; i += nblk * blockDim.x) {
      const int r = (int)(i / (unsigned)cv), c = (int)(i - (size_t)r * cv) * 8;
      const float4* s4 = reinterpret_cast<const float4*>(src + (size_t)r * ld_src + c);
      const float4 a = s4[0], b = s4[1];
      *reinterpret_cast<uint4*>(dst + (size_t)r * ld_dst + c) =
          make_uint4(pack2bf(a.x, a.y), pack2bf(a.z, a.w), pack2bf(b.x, b.y), pack2bf(b.z, b.w));
    }
    return;
  }
  const size_t n = (size_t)rows * cols;
  for (size_t i = bid * blockDim.x + threadIdx.x; i < n; i += nblk * blockDim.x) {
    const size_t r = i / cols, c = i % cols;
    dst[r * ld_dst + c] = f2bf(src[r * ld_src + c]);
  }
}

// Achievable dense MFMA throughput: every wave runs `iters` rounds of eight
// independent accumulations (v_mfma_f32_16x16x32_bf16, or four
// v_mfma_f32_16x16x4_f32 per round and chain for fp32) on constant operands,
// so the matrix pipes never wait for data or for one another.  Operands are
// powers of two (a = 2^-4, b = 2^-5 in every element) so that each thread's
// output, the sum of its 32 accumulator values, is exact:
// 32 * iters * K * 2^-9 with K = 32 (bf16) or 16 (fp32) per round.
template <bool BF16>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* out) {
  uint4 a, b;
  if constexpr (BF16) {
    a = make_uint4(0x3D803D80u, 0x3D803D80u, 0x3D803D80u, 0x3D803D80u);   // bf16 2^-4
    b = make_uint4(0x3D003D00u, 0x3D003D00u, 0x3D003D00u, 0x3D003D00u);   // bf16 2^-5
  } else {
    a = make_uint4(0x3D800000u, 0x3D800000u, 0x3D800000u, 0x3D800000u);   // fp32 2^-4
    b = make_uint4(0x3D000000u, 0x3D000000u, 0x3D000000u, 0x3D000000u);   // fp32 2^-5
  }
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = mfma_chunk<BF16>(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// v_mfma_f32_16x16x32_bf16 with the operands converted once, outside the
// loop; this file is compiled with VGPR accumulators (with AGPR ones the
// compiler rotated some chains through accumulator moves between the MFMAs,
// which halved the measured rate): each thread's sum of its 32 accumulator
// values is 32 * iters * 32 * 2^-9.
__global__ __launch_bounds__(256) void mfma_peak_16_bf16_kernel(int iters, float* out) {
  const uint4 a = make_uint4(0x3D803D80u, 0x3D803D80u, 0x3D803D80u, 0x3D803D80u);
  const uint4 b = make_uint4(0x3D003D00u, 0x3D003D00u, 0x3D003D00u, 0x3D003D00u);
  const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same with v_mfma_f32_32x32x16_bf16 (32768 flop each; a lane holds 8
// consecutive k of one row and 16 accumulators): each thread's sum of its
// 128 accumulator values is 128 * iters * 16 * 2^-9.
__global__ __launch_bounds__(256) void mfma_peak_32_kernel(int iters, float* out) {
  const uint4 a = make_uint4(0x3D803D80u, 0x3D803D80u, 0x3D803D80u, 0x3D803D80u);
  const uint4 b = make_uint4(0x3D003D00u, 0x3D003D00u, 0x3D003D00u, 0x3D003D00u);
  const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Check of the library's fp32 -> bf16 rounding (f2bf, the hardware
// conversion) against round-to-nearest-even written out on the bit pattern:
// add 0x7fff plus the lowest kept bit, keep the upper 16 bits; a NaN must
// stay a NaN.  Patterns [first, first + count) (count <= 2^32), grid-stride;
// each thread adds its mismatch count to *mism once.
__global__ __launch_bounds__(256) void bf16_round_check_kernel(unsigned long long first, unsigned long long count,
                                                               unsigned long long* mism) {
  unsigned long long bad = 0;
  const unsigned long long stride = (unsigned long long)gridDim.x * blockDim.x;
  for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const uint32_t u = (uint32_t)(first + i);
    const uint16_t got = f2bf(__uint_as_float(u));
    const bool nan = (u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u;
    if (nan) {
      bad += ((got & 0x7f80u) != 0x7f80u || (got & 0x007fu) == 0u) ? 1u : 0u;
    } else {
      const uint16_t want = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
      bad += got != want ? 1u : 0u;
    }
  }
  if (bad) atomicAdd(mism, bad);
}

}  // namespace

hipError_t rnn_launch_bf16_round_check(unsigned long long first, unsigned long long count, unsigned long long* mism,
                                       hipStream_t s) {
  hipLaunchKernelGGL(bf16_round_check_kernel, dim3(2048), dim3(256), 0, s, first, count, mism);
  return hipGetLastError();
}

hipError_t rnn_launch_mfma_peak(int kind, int blocks, int iters, float* out, hipStream_t s) {
  if (kind == 2) hipLaunchKernelGGL(mfma_peak_32_kernel, dim3(blocks), dim3(256), 0, s, iters, out);
  else if (kind == 1) hipLaunchKernelGGL(mfma_peak_16_bf16_kernel, dim3(blocks), dim3(256), 0, s, iters, out);
  else hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3(blocks), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

hipError_t rnn_launch_transpose_batch(const TransposeParams* ps, int n, int in_bf16, int out_bf16, hipStream_t s,
                                      const FillJob* fill) {
  if (n < 1 || n > 4) return hipErrorInvalidValue;
  if (fill && (fill->count < 0 || fill->count > 4)) return hipErrorInvalidValue;
  TransposeBatch b{};
  b.n = n;
  if (fill) b.fill = *fill;
  int gx = 0, gy = 0;
  const uintptr_t ia = in_bf16 ? 8 : 16, es_in = in_bf16 ? 2 : 4, es_out = out_bf16 ? 2 : 4;
  auto al = [](const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; };
  for (int i = 0; i < 4; ++i) {
    // slots past n stay empty (the grid's z extent is n)
    TransposeParams q = i < n ? ps[i] : TransposeParams{};
    // vector accesses only where every row start they can touch is aligned
    q.vec_in = al(q.src, ia) && (q.ld_src * es_in) % ia == 0 &&
               (!q.alt || (al(q.alt, ia) && (q.ld_alt * es_in) % ia == 0));
    q.vec_out = al(q.out, 16) && (q.ld_out * es_out) % 16 == 0;
    b.p[i] = q;
    if (i < n && q.R > 0 && q.C > 0) {
      gx = std::max(gx, (q.C + 63) / 64);
      gy = std::max(gy, (q.R + 63) / 64);
    }
  }
  const int nz = n + (b.fill.count > 0 ? 1 : 0);
  if (b.fill.count > 0) {   // the fill slice needs a grid of at least one block
    gx = std::max(gx, 1);
    gy = std::max(gy, 1);
  }
  if (gx == 0 || gy == 0) return hipSuccess;
  dim3 grid(gx, gy, nz);
  if (in_bf16 && out_bf16) hipLaunchKernelGGL((transpose_kernel<true, true>), grid, dim3(256), 0, s, b);
  else if (in_bf16 && !out_bf16) hipLaunchKernelGGL((transpose_kernel<true, false>), grid, dim3(256), 0, s, b);
  else if (!in_bf16 && out_bf16) hipLaunchKernelGGL((transpose_kernel<false, true>), grid, dim3(256), 0, s, b);
  else hipLaunchKernelGGL((transpose_kernel<false, false>), grid, dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t rnn_launch_transpose(const TransposeParams& p, int in_bf16, int out_bf16, hipStream_t s,
                                const FillJob* fill) {
  return rnn_launch_transpose_batch(&p, 1, in_bf16, out_bf16, s, fill);
}

hipError_t rnn_launch_convert(const float* src, long long ld_src, void* dst, long long ld_dst, int rows,
                              int cols, hipStream_t s, const FillJob* fill) {
  FillJob f{};
  size_t fill_bytes = 0;
  if (fill) {
    if (fill->count < 0 || fill->count > 4) return hipErrorInvalidValue;
    f = *fill;
    for (int j = 0; j < f.count; ++j) fill_bytes += f.bytes[j];
  }
  // enough fill blocks for the ranges (each thread sets a few words)
  const int fill_blocks = fill_bytes ? (int)std::min<size_t>((fill_bytes / 4 + 1023) / 1024, 256) : 0;
  if ((rows <= 0 || cols <= 0) && fill_blocks == 0) return hipSuccess;
  const int vec = cols % 8 == 0 && (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0 && ld_src % 4 == 0 &&
                  ld_dst % 8 == 0;
  const size_t n = (rows > 0 && cols > 0) ? (size_t)rows * cols / (vec ? 8 : 1) : 0;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(convert_kernel, dim3(blocks + fill_blocks), dim3(256), 0, s, src, ld_src,
                     reinterpret_cast<uint16_t*>(dst), ld_dst, rows, cols, vec, f, fill_blocks);
  return hipGetLastError();
}
