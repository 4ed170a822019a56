// MFMA GEMM for the time-parallel products of the fused RNN (gfx950):
//   * the hoisted input projection  GX = X W_ih^T + b   (all steps, both directions)
//   * the data gradient             dX = dG W_ih
//   * the weight gradients          dW = dG^T [X | 1]  (bias gradient as the ones column)
// Computing every time step of the input projection in one product is the
// "Combining Inputs" / "Combined GEMMs" rows of the cuDNN-5 optimisation table
// in Keras issue #3692; the weight gradients batch all steps the same way.
//
// Tile 128x128, K step 32, 256 threads (2x2 waves of 64x64), 16x16 MFMA
// tiles; operands converted to the compute type while staged into LDS
// (double-buffered, one barrier per K step).
#include <type_traits>

#include "device_util.h"
#include "rnn_common.h"

using namespace rnnk;

namespace {

constexpr int BM = 128, BN = 128, BK = 32, NTHR = 256;

template <bool BF16>
struct LdsT {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int STR = BF16 ? (BK + 8) : (BK + 4);  // padded row stride (elements)
};

// Stage 4 consecutive values (along k) of one row into LDS.
template <bool BF16>
__device__ __forceinline__ void lds_put4(typename LdsT<BF16>::T* dst, const float (&v)[4]) {
  if constexpr (BF16) {
    uint2 w = make_uint2(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]));
    *reinterpret_cast<uint2*>(dst) = w;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}
template <bool BF16>
__device__ __forceinline__ void lds_put1(typename LdsT<BF16>::T* dst, float v) {
  if constexpr (BF16) *dst = f2bf(v); else *dst = v;
}

template <bool BF16, bool B_BF16, bool A_KMAJ, bool B_KN, int EPI>
__global__ __launch_bounds__(NTHR) void gemm_kernel(const GemmParams p) {
  static_assert(!B_BF16 || BF16, "bf16 B operand needs the bf16 path");
  using ET = typename LdsT<BF16>::T;
  constexpr int STR = LdsT<BF16>::STR;
  __shared__ __attribute__((aligned(16))) ET As[2][BM * STR];
  __shared__ __attribute__((aligned(16))) ET Bs[2][BN * STR];

  const int z = blockIdx.z;
  const float* __restrict__ A = p.A[z];
  const int M = p.M, N = p.N, K = p.K;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const long long lda = p.lda, ldb = p.ldb;
  const int n_ones = p.n_ones;
  const int shift = p.b_shift[z], ak0 = p.b_alt_k0[z], ak1 = p.b_alt_k1[z];
  const float* __restrict__ balt = p.b_alt[z];

  // --- staging registers
  float ra[4][4];
  float rbf[4][4];   // fp32 B
  uint4 rbh[2];      // bf16 B (8 values each)

  auto b_row_ptr = [&](int k) -> const float* {  // fp32 KN source row (remapped); null = zero row
    if (k >= ak0 && k < ak1) return balt ? balt + (long long)(k - ak0) * p.ld_alt : nullptr;
    return reinterpret_cast<const float*>(p.B[z]) + (long long)(k + shift) * ldb;
  };

  auto load_tile = [&](int k0) {
    // A: 128 x 32 fp32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int idx = tid + i * NTHR;
      if constexpr (A_KMAJ) {
        int r = idx >> 3, kq = (idx & 7) * 4;
        int m = m0 + r, k = k0 + kq;
        const float* src = A + (long long)m * lda + k;
        if (p.a_vec && m < M && k + 3 < K) {
          float4 v = *reinterpret_cast<const float4*>(src);
          ra[i][0] = v.x; ra[i][1] = v.y; ra[i][2] = v.z; ra[i][3] = v.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) ra[i][e] = (m < M && k + e < K) ? src[e] : 0.f;
        }
      } else {
        int kr = idx >> 5, mq = (idx & 31) * 4;
        int k = k0 + kr, m = m0 + mq;
        const float* src = A + (long long)k * lda + m;
        if (p.a_vec && k < K && m + 3 < M) {
          float4 v = *reinterpret_cast<const float4*>(src);
          ra[i][0] = v.x; ra[i][1] = v.y; ra[i][2] = v.z; ra[i][3] = v.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) ra[i][e] = (k < K && m + e < M) ? src[e] : 0.f;
        }
      }
    }
    // B
    if constexpr (B_BF16) {
      const uint16_t* Bh = reinterpret_cast<const uint16_t*>(p.B[z]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int idx = tid + i * NTHR;
        uint16_t v8[8];
        if constexpr (!B_KN) {
          int n = n0 + (idx >> 2), k = k0 + (idx & 3) * 8;
          const uint16_t* src = Bh + (long long)n * ldb + k;
          if (p.b_vec && n < N && k + 7 < K) {
            rbh[i] = *reinterpret_cast<const uint4*>(src);
            continue;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] = (n < N && k + e < K) ? src[e] : (uint16_t)0;
        } else {
          int k = k0 + (idx >> 4), n = n0 + (idx & 15) * 8;
          const uint16_t* src = Bh + (long long)k * ldb + n;
          if (p.b_vec && k < K && n + 7 < N) {
            rbh[i] = *reinterpret_cast<const uint4*>(src);
            continue;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] = (k < K && n + e < N) ? src[e] : (uint16_t)0;
        }
        rbh[i] = make_uint4(v8[0] | (v8[1] << 16), v8[2] | (v8[3] << 16), v8[4] | (v8[5] << 16),
                            v8[6] | (v8[7] << 16));
      }
    } else {
      const float* Bf = reinterpret_cast<const float*>(p.B[z]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int idx = tid + i * NTHR;
        if constexpr (!B_KN) {
          int n = n0 + (idx >> 3), k = k0 + (idx & 7) * 4;
          const float* src = Bf + (long long)n * ldb + k;
          if (p.b_vec && n < N && k + 3 < K) {
            float4 v = *reinterpret_cast<const float4*>(src);
            rbf[i][0] = v.x; rbf[i][1] = v.y; rbf[i][2] = v.z; rbf[i][3] = v.w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) rbf[i][e] = (n < N && k + e < K) ? src[e] : 0.f;
          }
        } else {
          int k = k0 + (idx >> 5), n = n0 + (idx & 31) * 4;
          const float* row = (k < K) ? b_row_ptr(k) : nullptr;
          bool ones_in = (n_ones >= n && n_ones < n + 4);
          if (p.b_vec && row && n + 3 < N && !ones_in) {
            float4 v = *reinterpret_cast<const float4*>(row + n);
            rbf[i][0] = v.x; rbf[i][1] = v.y; rbf[i][2] = v.z; rbf[i][3] = v.w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              int nn = n + e;
              float v = 0.f;
              if (k < K && nn < N) v = (nn == n_ones) ? 1.f : (row ? row[nn] : 0.f);
              rbf[i][e] = v;
            }
          }
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    ET* as = As[buf];
    ET* bs = Bs[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int idx = tid + i * NTHR;
      if constexpr (A_KMAJ) {
        int r = idx >> 3, kq = (idx & 7) * 4;
        lds_put4<BF16>(as + r * STR + kq, ra[i]);
      } else {
        int kr = idx >> 5, mq = (idx & 31) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) lds_put1<BF16>(as + (mq + e) * STR + kr, ra[i][e]);
      }
    }
    if constexpr (B_BF16) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int idx = tid + i * NTHR;
        if constexpr (!B_KN) {
          int n = idx >> 2, k8 = (idx & 3) * 8;
          *reinterpret_cast<uint4*>(bs + n * STR + k8) = rbh[i];
        } else {
          int kr = idx >> 4, n8 = (idx & 15) * 8;
          const uint32_t w[4] = {rbh[i].x, rbh[i].y, rbh[i].z, rbh[i].w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            bs[(n8 + e) * STR + kr] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int idx = tid + i * NTHR;
        if constexpr (!B_KN) {
          int n = idx >> 3, kq = (idx & 7) * 4;
          lds_put4<BF16>(bs + n * STR + kq, rbf[i]);
        } else {
          int kr = idx >> 5, nq = (idx & 31) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) lds_put1<BF16>(bs + (nq + e) * STR + kr, rbf[i][e]);
        }
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  if (nk > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  const int fr = lane & 15, fq = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
    const ET* as = As[buf];
    const ET* bs = Bs[buf];
    constexpr int CH = BF16 ? 1 : 2;           // MFMA chunks per K step
    constexpr int CW = BF16 ? 32 : 16;         // k per chunk
    constexpr int PER = CW / 4;                // k per lane per chunk
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      uint4 af[4], bfr[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        af[mt] = *reinterpret_cast<const uint4*>(as + (wm + mt * 16 + fr) * STR + ch * CW + fq * PER);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        bfr[nt] = *reinterpret_cast<const uint4*>(bs + (wn + nt * 16 + fr) * STR + ch * CW + fq * PER);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_chunk<BF16>(af[mt], bfr[nt], acc[mt][nt]);
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

  // --- epilogue
  float* __restrict__ C = p.C[z];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = n0 + wn + nt * 16 + fr;
      if (n >= N) continue;
      float badd = 0.f;
      if constexpr (EPI == EPI_BIAS) {
        badd = p.bias1 ? p.bias1[n] : 0.f;
        if (p.bias2 && ((n % p.gh) / p.hh) != p.bias2_skip_gate) badd += p.bias2[n];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + mt * 16 + fq * 4 + r;
        if (m >= M) continue;
        const float v = acc[mt][nt][r];
        if constexpr (EPI == EPI_DW) {
          if (n == n_ones) p.cbias[z][m] = v;
          else C[(long long)m * p.ldc + n] = v;
        } else {
          C[(long long)m * p.ldc + n] = v + badd;
        }
      }
    }
  }
}

template <bool BF16, bool B_BF16, bool A_KMAJ, bool B_KN, int EPI>
hipError_t launch_one(const GemmParams& p, int batches, hipStream_t s) {
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM, batches);
  hipLaunchKernelGGL((gemm_kernel<BF16, B_BF16, A_KMAJ, B_KN, EPI>), grid, dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t rnn_launch_gemm(const GemmParams& p, int bf16_compute, int b_bf16, int a_kmajor,
                           int b_kn, int epi, int batches, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || batches <= 0) return hipSuccess;
  if (batches > 2) return hipErrorInvalidValue;
  // The combinations the operator uses.
  if (bf16_compute && b_bf16 && a_kmajor && !b_kn && epi == EPI_BIAS)
    return launch_one<true, true, true, false, EPI_BIAS>(p, batches, s);
  if (!bf16_compute && !b_bf16 && a_kmajor && !b_kn && epi == EPI_BIAS)
    return launch_one<false, false, true, false, EPI_BIAS>(p, batches, s);
  if (bf16_compute && b_bf16 && a_kmajor && b_kn && epi == EPI_STORE)
    return launch_one<true, true, true, true, EPI_STORE>(p, batches, s);
  if (!bf16_compute && !b_bf16 && a_kmajor && b_kn && epi == EPI_STORE)
    return launch_one<false, false, true, true, EPI_STORE>(p, batches, s);
  if (bf16_compute && !b_bf16 && !a_kmajor && b_kn && epi == EPI_DW)
    return launch_one<true, false, false, true, EPI_DW>(p, batches, s);
  if (!bf16_compute && !b_bf16 && !a_kmajor && b_kn && epi == EPI_DW)
    return launch_one<false, false, false, true, EPI_DW>(p, batches, s);
  return hipErrorInvalidValue;
}
