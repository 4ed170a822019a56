// MFMA GEMM for the time-parallel products of the fused RNN (gfx950):
//   * the hoisted input projection  GX = X W_ih^T + b   (all steps, both directions)
//   * the data gradient             dX = dG W_ih        (B = W_ih^T, pre-transposed)
//   * the weight gradients          dW = dG^T [X | 1]   (A = dG^T, B = X^T, pre-transposed;
//                                                        the bias gradient is the ones row of B)
// Computing every time step of a projection in one product is the "Combining
// Inputs" / "Combined GEMMs" rows of the cuDNN-5 optimisation table in Keras
// issue #3692; giving every product the same operand layout is its "Matrix
// pre-transposition" row.
//
// One layout only: C[m, n] = sum_k A[m, k] * B[n, k], both operands
// K-contiguous, both in the compute type (bf16 with fp32 accumulation, or
// fp32).  Default tile 128x128, K step 32 (fp32) / 64 (bf16) -- 128 bytes of
// every tile row per step -- 256 threads as 2x2 waves of 64x64 built from
// 16x16 MFMA tiles (the direct-to-LDS kernel also runs other wave grids and
// 64 x 16*FN wave tiles, below).  Tiles are numbered m-major and dealt to the 8 XCDs in
// contiguous runs so that the tiles sharing an A row-block share an L2.
// Optional split-K writes fp32 partials that a second kernel sums in a fixed
// order (deterministic).
//
// Two kernels share that structure:
//  * gemm_lds_kernel, used whenever every operand row is 16-byte aligned and
//    K is a whole number of 16-byte vectors: operands go straight from global
//    memory into LDS (global_load_lds, no register staging) through a
//    multi-stage pipeline (one barrier per K step; the loads of step k+NS-1
//    are issued as soon as every wave has finished step k-1), tiles visited
//    in groups of 8 tile rows for L2 reuse, in an XOR-swizzled layout (16-byte slot s of row r
//    holds k-vector s ^ (r & 7)) so that the fragment reads of 8 consecutive
//    rows hit distinct banks.  Addressing is branch-free: rows past M re-read
//    the last row of A, rows past N and the ones row of the bias gradient
//    read a 16-byte ones vector (results of rows past M or N are not
//    stored), and vectors past K read a 16-byte zero vector.
//  * gemm_nt_kernel, the general fallback (any alignment and K), staging
//    through registers with element-wise edge handling.
#include <cstdlib>
#include <type_traits>

#include "device_util.h"
#include "rnn_common.h"

using namespace rnnk;

namespace {

constexpr int BM = 128, BN = 128, NTHR = 256;

template <bool BF16>
struct Cfg {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int BK = BF16 ? 64 : 32;          // k per LDS stage
  static constexpr int EPV = 16 / sizeof(T);         // elements per 16-byte vector
  static constexpr int STR = BK + EPV;               // padded LDS row (elements)
  static constexpr int VPR = BK / EPV;               // 16-byte vectors per tile row
  static constexpr int LPT = BM * VPR / NTHR;        // vectors per thread per operand
};

template <bool BF16>
__device__ __forceinline__ uint4 load_vec(const typename Cfg<BF16>::T* row, int k, int K, bool rv,
                                          bool vec_ok) {
  using T = typename Cfg<BF16>::T;
  constexpr int EPV = Cfg<BF16>::EPV;
  if (rv && vec_ok && k + EPV <= K) return *reinterpret_cast<const uint4*>(row + k);
  T v[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) v[e] = (rv && k + e < K) ? row[k + e] : (T)0;
  return *reinterpret_cast<const uint4*>(v);
}

// Ones row for the bias gradient: EPV ones in the compute type, zero past K.
template <bool BF16>
__device__ __forceinline__ uint4 ones_vec(int k, int K) {
  using T = typename Cfg<BF16>::T;
  constexpr int EPV = Cfg<BF16>::EPV;
  T v[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    if constexpr (BF16) v[e] = (k + e < K) ? (uint16_t)0x3f80 : (uint16_t)0;
    else v[e] = (k + e < K) ? 1.f : 0.f;
  }
  return *reinterpret_cast<const uint4*>(v);
}

// Store one wave's 64 x 16*FN accumulator tile (rows mw0.., columns nw0..):
// the fp32 split-K partial, or C with the epilogue EPI.
template <int EPI, int FN = 4>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p, const f32x4 (&acc)[4][FN], int z,
                                              int split, int mw0, int nw0, int fr, int fq) {
  const int M = p.M, N = p.N;
  if (p.split_k > 1) {
    float* part = p.partial + ((size_t)z * p.split_k + split) * (size_t)M * N;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < FN; ++nt) {
        const int n = nw0 + nt * 16 + fr;
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mw0 + mt * 16 + fq * 4 + r;
          if (m < M) part[(size_t)m * N + n] = acc[mt][nt][r];
        }
      }
    return;
  }
  float* __restrict__ C = p.C[z];
  float badd[FN] = {};
  if constexpr (EPI == EPI_BIAS) {
#pragma unroll
    for (int nt = 0; nt < FN; ++nt) {
      const int n = min(nw0 + nt * 16 + fr, N - 1);
      float b = p.bias1 ? p.bias1[n] : 0.f;
      if (p.bias2 && ((n % p.gh) / p.hh) != p.bias2_skip_gate) b += p.bias2[n];
      badd[nt] = b;
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < FN; ++nt) {
      const int n = nw0 + nt * 16 + fr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mw0 + mt * 16 + fq * 4 + r;
        if (m >= M || n >= N) continue;
        const float v = acc[mt][nt][r];
        if constexpr (EPI == EPI_DW) {
          if (n == p.n_ones) p.cbias[z][m] = v;
          else C[(long long)m * p.ldc + n] = v;
        } else {
          C[(long long)m * p.ldc + n] = v + badd[nt];
        }
      }
    }
  }
}

template <bool BF16, int EPI>
__global__ __launch_bounds__(NTHR) void gemm_nt_kernel(const GemmParams p) {
  using T = typename Cfg<BF16>::T;
  constexpr int BK = Cfg<BF16>::BK, EPV = Cfg<BF16>::EPV, STR = Cfg<BF16>::STR;
  constexpr int VPR = Cfg<BF16>::VPR, LPT = Cfg<BF16>::LPT;
  __shared__ __attribute__((aligned(16))) T As[2][BM * STR];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * STR];

  const int z = blockIdx.z;
  const int M = p.M, N = p.N, K = p.K;
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int ntiles = tm * tn;
  const int nsplit = p.split_k;
  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a contiguous
  // run of m-major tiles.
  const int total = ntiles * nsplit;
  const int bid = blockIdx.x;
  const int per = (total + 7) / 8;
  const int lin = (bid % 8) * per + bid / 8;
  if (lin >= total) return;
  const int split = lin % nsplit;
  const int tile = lin / nsplit;
  const int m0 = (tile / tn) * BM, n0 = (tile % tn) * BN;
  const int kper = ((K + nsplit - 1) / nsplit + BK - 1) / BK * BK;
  const int kbeg = split * kper, kend = min(K, kbeg + kper);

  const T* __restrict__ A = reinterpret_cast<const T*>(p.A[z]);
  const T* __restrict__ Bm = reinterpret_cast<const T*>(p.B[z]);
  const long long lda = p.lda, ldb = p.ldb;
  // the wave index in a scalar register (the same in every lane)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int fr = lane & 15, fq = lane >> 4;
  const bool avec = p.a_vec, bvec = p.b_vec;

  uint4 ra[LPT], rb[LPT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int idx = tid + i * NTHR;
      const int r = idx / VPR, kv = (idx % VPR) * EPV;
      const int m = m0 + r, n = n0 + r, k = k0 + kv;
      const bool mv = m < M, nv = n < N;
      ra[i] = load_vec<BF16>(A + (long long)(mv ? m : 0) * lda, k, kend, mv, avec);
      if (n == p.n_ones) rb[i] = ones_vec<BF16>(k, kend);
      else rb[i] = load_vec<BF16>(Bm + (long long)(nv ? n : 0) * ldb, k, kend, nv && n != p.n_ones, bvec);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int idx = tid + i * NTHR;
      const int r = idx / VPR, kv = (idx % VPR) * EPV;
      *reinterpret_cast<uint4*>(&As[buf][r * STR + kv]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][r * STR + kv]) = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    load_tile(kbeg);
    store_tile(0);
  }
  __syncthreads();
  constexpr int CW = BF16 ? 32 : 16;        // k per MFMA chunk
  constexpr int PER = CW / 4;               // k per lane per chunk
  constexpr int CH = BK / CW;               // chunks per stage
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile(kbeg + (kt + 1) * BK);
    const T* as = As[buf];
    const T* bs = Bs[buf];
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

  gemm_epilogue<EPI>(p, acc, z, split, m0 + wm, n0 + wn, fr, fq);
}

// --------------------------------------------------------------- fast path
constexpr int kRowBytes = 128;                  // bytes of one tile row per K step
constexpr int kStageBytes = BM * kRowBytes;     // one operand, one stage

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint4 lds_read16(const lds_char* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector memory
// and `lgkm` LDS/scalar operations are outstanding; export count not waited on.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (((vm >> 4) & 3) << 14) | ((lgkm & 15) << 8) | (7 << 4) | (vm & 15);
}

// Block tile (64*WM) x (16*FN*WN), WM x WN waves of 64 x 16*FN (4 x FN MFMA
// tiles); NS pipeline stages of (64*WM + 16*FN*WN) rows x 128 bytes of LDS; GM: tiles are visited in
// groups of GM tile rows, column by column inside a group, so that the
// workgroups running at the same time on one XCD share few A and B row
// blocks (0: row-major).
template <bool BF16, int EPI, int NS, int GM, int WM, int WN, int FN = 4>
__global__ __launch_bounds__(64 * WM * WN) void gemm_lds_kernel(const GemmParams p) {
  using T = typename Cfg<BF16>::T;
  constexpr int BK = Cfg<BF16>::BK, EPV = Cfg<BF16>::EPV;
  constexpr int NW = WM * WN;
  constexpr int TBM = 64 * WM, TBN = 16 * FN * WN;   // waves of 64 x 16*FN
  constexpr int SA = TBM * kRowBytes, SB = TBN * kRowBytes;   // one stage of A / of B
  constexpr int LA = TBM / (8 * NW), LB = TBN / (8 * NW);     // 1 KB loads per wave per stage
  static_assert(LA * 8 * NW == TBM && LB * 8 * NW == TBN, "whole 8-row load groups per wave");
  static_assert(BK * sizeof(T) == kRowBytes, "one K step is 128 bytes of a row");
  __shared__ __attribute__((aligned(1024))) char smem[NS * (SA + SB)];
  lds_char* const lds = (lds_char*)smem;

  const int z = blockIdx.z;
  const int M = p.M, N = p.N, K = p.K;
  const int tm = (M + TBM - 1) / TBM, tn = (N + TBN - 1) / TBN;
  const int nsplit = p.split_k;
  const int total = tm * tn * nsplit;
  const int bid = blockIdx.x;
  const int per = (total + 7) / 8;
  const int lin = (bid % 8) * per + bid / 8;
  if (lin >= total) return;
  const int split = lin % nsplit;
  int tile = lin / nsplit;
  int mi = tile / tn, ni = tile % tn;
  if (GM > 0) {
    const int g = tile / (GM * tn), in = tile - g * GM * tn;
    const int gm = min(GM, tm - g * GM);
    mi = g * GM + in % gm;
    ni = in / gm;
  }
  const int m0 = mi * TBM, n0 = ni * TBN;
  const int kper = ((K + nsplit - 1) / nsplit + BK - 1) / BK * BK;
  const int kbeg = split * kper, kend = min(K, kbeg + kper);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  // the wave index in a scalar register (the same in every lane)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave / WN) * 64, wn = (wave % WN) * (16 * FN);
  const int fr = lane & 15, fq = lane >> 4;

  // ---- loader: load j of wave w fills rows 8*(NW*j + w) .. +7 of a stage
  // (64 lanes x 16 bytes); lane l takes row 8*(NW*j+w) + l/8, slot l%8,
  // i.e. k-vector (l%8) ^ (row & 7)
  const char* zero = reinterpret_cast<const char*>(p.zero16);
  const char* ones = reinterpret_cast<const char*>(p.ones16);
  const char* arow[LA];
  const char* brow[LB];
  const int kvo = ((lane & 7) ^ ((lane >> 3) & 7)) * EPV;   // rows 8*g + lane/8: row & 7 == lane/8
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int r = 8 * (NW * j + wave) + (lane >> 3);
    arow[j] = reinterpret_cast<const char*>(reinterpret_cast<const T*>(p.A[z]) +
                                            (long long)min(m0 + r, M - 1) * p.lda);
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int r = 8 * (NW * j + wave) + (lane >> 3);
    // the ones row reads the ones vector, and so do rows past N (B may have
    // no real row to re-read when its last row is the ones row)
    const int n = n0 + r;
    brow[j] = (n == p.n_ones || n >= N)
                  ? nullptr
                  : reinterpret_cast<const char*>(reinterpret_cast<const T*>(p.B[z]) + (long long)n * p.ldb);
  }
  auto issue = [&](int st, int k0) {
    lds_char* sa = lds + st * SA;
    lds_char* sb = lds + NS * SA + st * SB;
    const int k = k0 + kvo;
    const bool kv = k < kend;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const char* ga = kv ? arow[j] + (size_t)k * sizeof(T) : zero;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)ga,
                                       (void __attribute__((address_space(3)))*)(sa + (NW * j + wave) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const char* gb = kv ? (brow[j] ? brow[j] + (size_t)k * sizeof(T) : ones) : zero;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)gb,
                                       (void __attribute__((address_space(3)))*)(sb + (NW * j + wave) * 1024), 16, 0, 0);
    }
  };

  // fragment offsets: row r, k-vector v sits at r*128 + ((v ^ (r & 7)) * 16);
  // for the rows a lane reads, r & 7 == fr & 7
  constexpr int CH = BK * (int)sizeof(T) / 64;   // MFMA chunks (4 vectors) per step
  int fo[CH];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) fo[ch] = fr * kRowBytes + (((ch * 4 + fq) ^ (fr & 7)) * 16);

  f32x4 acc[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the bias gradient's row sums (the 64 x 80 wave tiles only, so the other
  // instances compile without it): the waves of the first column tile whose
  // columns start at 0 also multiply their A fragments by ones (A reads
  // zeros past K, and rows past M are never stored)
  constexpr bool BIAS_MFMA = EPI == EPI_DW && FN == 5;
  const bool bias_wave = BIAS_MFMA && p.bias_mfma && ni == 0 && wn == 0;
  f32x4 accb[4] = {};
  const unsigned one2 = BF16 ? 0x3f803f80u : 0x3f800000u;
  const uint4 ones_frag = {one2, one2, one2, one2};

#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < nk) issue(i, kbeg + i * BK);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % NS;
    // this thread's loads of step kt are complete once only those of the
    // steps issued after it (LA + LB each) remain outstanding, and its LDS
    // reads of step kt-1 once lgkmcnt is 0; the barrier extends both to all
    // threads.  A bare barrier: __syncthreads() would also wait for the
    // later steps' loads (its fence drains every memory operation).
    const int ahead = min(nk - 1 - kt, NS - 2);
    __builtin_amdgcn_sched_barrier(0);
    if (NS >= 4 && ahead >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * (LA + LB), 0));
    else if (NS >= 3 && ahead >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_imm(LA + LB, 0));
    else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // every wave has finished step kt-1, so its buffer can be refilled
    if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kbeg + (kt + NS - 1) * BK);
    const lds_char* sa = lds + st * SA + wm * kRowBytes;
    const lds_char* sb = lds + NS * SA + st * SB + wn * kRowBytes;
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      uint4 af[4], bfr[FN];
#pragma unroll
      for (int t = 0; t < 4; ++t) af[t] = lds_read16(sa + t * 16 * kRowBytes + fo[ch]);
#pragma unroll
      for (int t = 0; t < FN; ++t) bfr[t] = lds_read16(sb + t * 16 * kRowBytes + fo[ch]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < FN; ++nt) acc[mt][nt] = mfma_chunk<BF16>(af[mt], bfr[nt], acc[mt][nt]);
      if (bias_wave) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) accb[mt] = mfma_chunk<BF16>(af[mt], ones_frag, accb[mt]);
      }
    }
  }
  gemm_epilogue<EPI, FN>(p, acc, z, split, m0 + wm, n0 + wn, fr, fq);
  if (bias_wave && fr == 0) {   // every column of accb holds the row sums
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + mt * 16 + fq * 4 + r;
        if (m < M) p.cbias[z][m] = accb[mt][r];
      }
  }
}

// Fixed-order sum of the split-K partials, then the dW epilogue.
__global__ void splitk_reduce_kernel(const GemmParams p) {
  const int z = blockIdx.y;
  const size_t MN = (size_t)p.M * p.N;
  const float* part = p.partial + (size_t)z * p.split_k * MN;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += (size_t)gridDim.x * blockDim.x) {
    float v = 0.f;
    for (int s = 0; s < p.split_k; ++s) v += part[(size_t)s * MN + i];
    const int m = (int)(i / p.N), n = (int)(i % p.N);
    if (n == p.n_ones) p.cbias[z][m] = v;
    else p.C[z][(long long)m * p.ldc + n] = v;
  }
}

// One configuration of the direct-to-LDS kernel: waves WM x WN of 64 x 16*FN,
// stages NS.
template <bool BF16, int EPI, int NS, int GM, int WM, int WN, int FN = 4>
void launch_lds(const GemmParams& p, int batches, hipStream_t s) {
  const int tbn = 16 * FN * WN;
  const int tiles = ((p.M + 64 * WM - 1) / (64 * WM)) * ((p.N + tbn - 1) / tbn) * p.split_k;
  const int grid = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_lds_kernel<BF16, EPI, NS, GM, WM, WN, FN>), dim3(grid, 1, batches), dim3(64 * WM * WN), 0,
                     s, p);
}

template <bool BF16, int EPI>
hipError_t launch_one(const GemmParams& p, int batches, hipStream_t s) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.split_k;
  const int grid = (tiles + 7) / 8 * 8;
  const bool fast = p.a_vec && p.b_vec && p.zero16 && (p.n_ones < 0 || p.ones16) &&
                    p.K % Cfg<BF16>::EPV == 0 && !p.force_general;
  // tuning: the direct-to-LDS kernel's shape (waves, stages)
  static const int variant = [] {
    const char* v = std::getenv("RNN_GEMM_VARIANT");
    return v ? std::atoi(v) : 0;
  }();
  if (fast) {
    const bool g8 = p.split_k == 1;   // groups of 8 tile rows help the single-pass products
    int v = variant;
    if (v == 0 && BF16 && EPI == EPI_BIAS && p.split_k == 1) {
      // the input projection: 256x256 tiles on sixteen waves (one workgroup
      // per CU) do a unit of work in 2/3 of the time of two 128x128
      // workgroups per CU (measured: 33 us per round of 256x256 tiles vs
      // 25 us per round of 2 x 128x128 per CU at K = 800), but come in
      // rounds of 256 tiles instead of 512: take them when the rounds they
      // need cost less
      const int r128 = (((p.M + 127) / 128) * ((p.N + 127) / 128) + 511) / 512;
      const int r256 = (((p.M + 255) / 256) * ((p.N + 255) / 256) + 255) / 256;
      if (33.2 * r256 < 25.0 * r128) v = 3;
    }
    if (v == 0 && BF16 && EPI == EPI_STORE && p.split_k == 1) {
      // the data gradient: 128 x 160 tiles (waves of 64 x 80) when one round
      // of them, one per CU or two, replaces more than one round of 128 x 128
      // tiles at the same occupancy (the 800-wide DS2 product splits into 5
      // column tiles instead of 6.25: measured 46.4 -> 41.9 us, three or four
      // stages 44.7 / 43.6 us; the 1600-wide inner layers of a bidirectional
      // stack, 470 tiles instead of 611: 143.8 -> 107 us)
      const int tm = (p.M + 127) / 128;
      const int t160 = tm * ((p.N + 159) / 160) * batches, t128 = tm * ((p.N + 127) / 128) * batches;
      if ((t160 <= 256 && t128 > 256) || (t160 <= 512 && t128 > 512)) v = 7;
    }
    if (v == 0 && BF16 && EPI == EPI_DW && p.split_k == 1 && p.n_ones == p.N - 1 && p.N > 1) {
      // a weight gradient: the bias row sums by MFMA against ones, so that
      // the product is N - 1 wide, on 128 x 160 tiles, when one round of
      // them at two per CU replaces more than one round of 128 x 128 tiles
      // with the ones row
      const int tm = (p.M + 127) / 128;
      const int t160 = tm * ((p.N - 1 + 159) / 160) * batches, t128 = tm * ((p.N + 127) / 128) * batches;
      if (t160 <= 512 && t128 > 512) {
        GemmParams q = p;
        q.N = p.N - 1;
        q.n_ones = -1;
        q.bias_mfma = 1;
        g8 ? launch_lds<BF16, EPI, 2, 8, 2, 2, 5>(q, batches, s) : launch_lds<BF16, EPI, 2, 0, 2, 2, 5>(q, batches, s);
        return hipGetLastError();
      }
    }
    switch (v) {
      case 1: g8 ? launch_lds<BF16, EPI, 3, 8, 4, 2>(p, batches, s) : launch_lds<BF16, EPI, 3, 0, 4, 2>(p, batches, s); break;
      case 2: g8 ? launch_lds<BF16, EPI, 3, 8, 2, 4>(p, batches, s) : launch_lds<BF16, EPI, 3, 0, 2, 4>(p, batches, s); break;
      case 3: g8 ? launch_lds<BF16, EPI, 2, 8, 4, 4>(p, batches, s) : launch_lds<BF16, EPI, 2, 0, 4, 4>(p, batches, s); break;
      case 4: g8 ? launch_lds<BF16, EPI, 4, 8, 2, 2>(p, batches, s) : launch_lds<BF16, EPI, 4, 0, 2, 2>(p, batches, s); break;
      case 5: g8 ? launch_lds<BF16, EPI, 3, 8, 2, 2>(p, batches, s) : launch_lds<BF16, EPI, 3, 0, 2, 2>(p, batches, s); break;
      case 6: g8 ? launch_lds<BF16, EPI, 2, 8, 4, 2>(p, batches, s) : launch_lds<BF16, EPI, 2, 0, 4, 2>(p, batches, s); break;
      case 7: g8 ? launch_lds<BF16, EPI, 2, 8, 2, 2, 5>(p, batches, s) : launch_lds<BF16, EPI, 2, 0, 2, 2, 5>(p, batches, s); break;
      case 8: g8 ? launch_lds<BF16, EPI, 3, 8, 2, 2, 5>(p, batches, s) : launch_lds<BF16, EPI, 3, 0, 2, 2, 5>(p, batches, s); break;
      case 9: g8 ? launch_lds<BF16, EPI, 4, 8, 2, 2, 5>(p, batches, s) : launch_lds<BF16, EPI, 4, 0, 2, 2, 5>(p, batches, s); break;
      default:
        // two stages (64 KB of LDS, two workgroups per CU) measured faster
        // than three or four with one workgroup per CU
        g8 ? launch_lds<BF16, EPI, 2, 8, 2, 2>(p, batches, s) : launch_lds<BF16, EPI, 2, 0, 2, 2>(p, batches, s);
    }
  } else {
    hipLaunchKernelGGL((gemm_nt_kernel<BF16, EPI>), dim3(grid, 1, batches), dim3(NTHR), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.split_k <= 1) return e;
  size_t mn = (size_t)p.M * p.N;
  unsigned blocks = (unsigned)std::min<size_t>((mn + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks, batches), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t rnn_launch_gemm(const GemmParams& p, int bf16, int epi, int batches, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || batches <= 0) return hipSuccess;
  // split-K: the weight gradients and the plain store (the partials' sum is
  // written by splitk_reduce_kernel); never with the bias epilogue
  if (batches > 2 || p.split_k < 1 || (p.split_k > 1 && (epi == EPI_BIAS || !p.partial)))
    return hipErrorInvalidValue;
  if (bf16) {
    if (epi == EPI_BIAS) return launch_one<true, EPI_BIAS>(p, batches, s);
    if (epi == EPI_STORE) return launch_one<true, EPI_STORE>(p, batches, s);
    if (epi == EPI_DW) return launch_one<true, EPI_DW>(p, batches, s);
  } else {
    if (epi == EPI_BIAS) return launch_one<false, EPI_BIAS>(p, batches, s);
    if (epi == EPI_STORE) return launch_one<false, EPI_STORE>(p, batches, s);
    if (epi == EPI_DW) return launch_one<false, EPI_DW>(p, batches, s);
  }
  return hipErrorInvalidValue;
}
