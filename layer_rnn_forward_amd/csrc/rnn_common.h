// Shared host/device definitions of the fused RNN library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnnk {

constexpr int kMaxLayersPerLaunch = 8;   // layers resident in one wavefront launch
constexpr int kFlagStride = 32;          // u32 per flag slot (128 bytes)
constexpr int kMaxWaitFlags = 512;       // flags one workgroup may poll per step
constexpr int kWaitPerLane = kMaxWaitFlags / 64;
constexpr int kXcds = 8;                 // XCDs of one MI355X (SPX mode), each with its own L2

// Grid of a sweep with `groups` groups of `nwg` workgroups: linear (place
// 0), XCD-local (place 1) or runs of `place` consecutive workgroups per XCD
// (place >= 2); logical_wg in recurrent_util.h maps them, idle slots exit at
// once.
__host__ __device__ constexpr int sweep_grid(int place, int nwg, int groups) {
  return place == 1   ? kXcds * ((groups + kXcds - 1) / kXcds) * nwg
         : place >= 2 ? (nwg * groups + kXcds * place - 1) / (kXcds * place) * (kXcds * place)
                      : nwg * groups;
}

enum Mode { MODE_TANH = 0, MODE_LSTM = 1, MODE_GRU = 2 };

// Reserve slots per (layer, direction, step, batch row, unit):
//   LSTM: i f g o c     GRU: r z n gh_n     tanh: none
__host__ __device__ constexpr int reserve_slots(int mode) {
  return mode == MODE_LSTM ? 5 : (mode == MODE_GRU ? 4 : 0);
}
__host__ __device__ constexpr int gates_of(int mode) {
  return mode == MODE_LSTM ? 4 : (mode == MODE_GRU ? 3 : 1);
}

// ------------------------------------------------------------------ GEMM
// C[m, n] = sum_k A[m*lda + k] * B[n*ldb + k]   (batched over blockIdx.z < 2)
// A and B in the compute type (bf16 or fp32), both K-contiguous.  Row n_ones
// of B is all ones (it yields the bias gradient), or -1.
// Epilogue: EPI_STORE  C[m*ldc + n] = acc
//           EPI_BIAS   C[m*ldc + n] = acc + bias1[n] + bias2[n] (bias2 skipped
//                      for columns whose gate (n % gh) / hh == bias2_skip_gate)
//           EPI_DW     n == n_ones ? cbias[m] = acc : C[m*ldc + n] = acc
// split_k > 1 (EPI_DW only): fp32 partials [batch][split][M][N] in `partial`,
// summed in split order by a second kernel.
enum Epi { EPI_STORE = 0, EPI_BIAS = 1, EPI_DW = 2 };

struct GemmParams {
  int M, N, K;
  const void* A[2];
  long long lda;
  const void* B[2];
  long long ldb;
  int n_ones;
  float* C[2];
  long long ldc;
  float* cbias[2];
  const float* bias1;
  const float* bias2;
  int bias2_skip_gate, gh, hh;
  int a_vec, b_vec;   // 1: 16-byte vector loads are legal (aligned bases and strides)
  int split_k;
  float* partial;
  const void* zero16;  // 16 bytes of zeros (device), or null: general kernel only
  const void* ones16;  // 16 bytes of ones in the compute type (device)
  int force_general;   // 1: always use the general kernel
  // set by the launcher only (direct-to-LDS kernel, EPI_DW, no split):
  // cbias[z][m] = sum_k A[m,k], from extra MFMAs against a ones fragment in
  // the first column tile, instead of a ones row of B
  int bias_mfma;
};

// Row-gather transpose: out[c * ld_out + r] = src_row(r)[c] for r < R, c < C,
// where src_row(r) = src + (r + shift) * ld_src, except rows r in
// [alt_r0, alt_r1) which read alt + (r - alt_r0) * ld_alt (zeros if alt is
// null).  Converts the element type on the way.
struct TransposeParams {
  const void* src;
  long long ld_src;
  int shift;
  const void* alt;
  long long ld_alt;
  int alt_r0, alt_r1;
  void* out;
  long long ld_out;
  int R, C;
  // with lengths: row r = t*len_B + b also reads alt row b whenever
  // t + 1 >= the row's length clamped to [0, len_T] (a reverse-direction
  // step whose successor is past the row's end starts from h0)
  const int* lengths;
  int len_B, len_T;
  // set by the launcher: 16-byte (fp32) / 8-byte (bf16) row loads and
  // 16-byte stores of 8 output elements are aligned
  int vec_in, vec_out;
  // the output's contiguous index r is a permuted reduction index of a
  // product (gg_col / tb_k below); the input row it gathers is
  //   map 1: gg_col_source(r, mU, mG, mH, mNwg)   (W_ih^T for the dX product)
  //   map 2: tb_k_source(r, mBc, mT, mB)           (X^T, H_prev^T for dW)
  // a hole (no input row) reads zeros; map 0: row r
  int map;
  int mU, mG, mH, mNwg;
  int mBc, mT, mB;
};

// Reduction-index orders of the gate gradients, chosen so that each
// workgroup of the backward sweep writes whole cache lines that no other
// workgroup (on another XCD) shares:
//  * dG [T*B][dg_ld], the A operand of the dX product: column
//    gg_col(d, slice, g, j) = d*nwg*G*U + slice*G*U + g*U + j for unit
//    slice*U + j of gate g, direction d -- the G*U values a workgroup makes
//    for one row are contiguous;
//  * dG^T [D*G*H][tb_ld] (rows in the natural gate order), the A operand of
//    the weight-gradient products: column tb_k(c, t, bl) = c*T*Bc + t*Bc + bl
//    for batch row c*Bc + bl of chunk c at step t -- one workgroup's values of
//    a row at successive steps are adjacent.
// The other operand of each product (W_ih^T; X^T, H_prev^T) is gathered in
// the same order; positions of units past H or batch rows past B are zero in
// both.
__host__ __device__ inline long long gg_col(int d, int slice, int g, int j, int U, int G, int nwg) {
  return (long long)d * nwg * G * U + (long long)slice * G * U + (long long)g * U + j;
}
__host__ __device__ inline long long tb_k(int c, int t, int bl, int T, int Bc) {
  return (long long)c * T * Bc + (long long)t * Bc + bl;
}
// Natural row (d*G*H + g*H + u) of column r of dG, or -1 past H.
__host__ __device__ inline int gg_col_source(int r, int U, int G, int H, int nwg) {
  const int CG = nwg * G * U;
  const int d = r / CG, rem = r - d * CG;
  const int slice = rem / (G * U), r2 = rem - slice * G * U;
  const int g = r2 / U, j = r2 - g * U;
  const int u = slice * U + j;
  return u < H ? d * G * H + g * H + u : -1;
}
// Natural row (t*B + b) of column k of dG^T, or -1 past B.
__host__ __device__ inline int tb_k_source(int k, int Bc, int T, int B) {
  const int c = k / (T * Bc), rem = k - c * T * Bc;
  const int t = rem / Bc, bl = rem - t * Bc;
  const int b = c * Bc + bl;
  return b < B ? t * B + b : -1;
}

// ------------------------------------------------------------- recurrence
// One forward launch covers `nlayers` layers (a wavefront when > 1) or one
// layer with both directions; groups are (layer, direction, batch chunk);
// each group has `nwg` workgroups owning `U` hidden units each.
struct FwdParams {
  int T, B, H, D;
  int nlayers;            // layers in this launch
  int nchunk, Bc;         // batch chunks of Bc rows
  int U, nwg;             // units per workgroup, workgroups per group
  int slice;              // bytes of one producer's slice in a ring entry (multiple of 128)
  int gran;               // bytes of one granule: padded rows x 16 (U/PER granules per slice)
  long long ring_step;    // bytes of one ring entry (nwg * slice)
  long long ring_group;   // bytes of one group's ring (entries * ring_step)
  int stage;              // 1: copy each consumed ring entry into LDS first
  int group_poll;         // 1: one wave polls every producer; 0: each wave its own
  int s_begin, s_end;     // global steps [s_begin, s_end); -1 is the prologue
  int s_total;            // T + nlayers - 1
  int persistent, training, wavefront;
  int probe;              // 1: exchange only (waits, ring stores, flags); no weights, math or outputs
  int place, ngroups;     // workgroup placement (sweep_grid) and the launch's group count
  const int* lengths;     // [B] valid steps per row (clamped to [0, T]), or null: all T
  void* xch2;             // GRU with (r*h) W_hn: rings of r*h, laid out as xch
  int paper;              // GRU with (r*h) W_hn: 1 for h = (1-z) h_prev + z n
  // wavefront training with inter-layer dropout: rings (laid out as xch) of
  // each layer's h times its dropout multiplier, read by the layer above; or
  // null.  Multiplier of element e of layer l's input: philox.h dropout_mult
  void* xch_drop;
  unsigned long long drop_thr;
  float drop_scale;
  unsigned drop_k0, drop_k1;
  int first_layer;        // index of layer 0 of this launch in the network
  const void* w_ih[kMaxLayersPerLaunch];   // layer block [D*G*H, I_l]
  const void* w_hh[kMaxLayersPerLaunch];   // layer block [D*G*H, H]
  const float* b_ih[kMaxLayersPerLaunch];  // [D*G*H]
  const float* b_hh[kMaxLayersPerLaunch];
  int in_l[kMaxLayersPerLaunch];           // input width of each layer
  const float* gx;        // hoisted projection of the launch's first layer [T*B, D*G*H]
  float* y[kMaxLayersPerLaunch];           // [T, B, D*H]
  float* reserve[kMaxLayersPerLaunch];     // [D][T][B][R][H] (training)
  const float* h0;        // [L*D, B, H] of the whole network, or null
  const float* c0;
  float* hy;
  float* cy;
  float* st_h;            // carried state between stepped launches [nlayers*D][B][H]
  float* st_c;
  void* xch;              // exchange rings: per group [s_total + 1][nwg][slice]
  unsigned* flags;        // per workgroup, kFlagStride apart
  unsigned* err;
  unsigned spin_limit;
};

struct BwdParams {
  int T, B, H, D;
  int nchunk, Bc, U, nwg;
  int slice;              // bytes of one producer's slice (G*U/PER granules, a multiple of 128)
  int gran;               // bytes of one granule: padded rows x 16
  long long ring_step, ring_group;
  int stage;              // 1: copy each consumed ring entry into LDS first
  int group_poll;         // 1: one wave polls every producer; 0: each wave its own
  int s_begin, s_end;     // processing steps; s == T is the final dh0 phase
  int persistent;
  int place, ngroups;     // workgroup placement (sweep_grid) and the launch's group count
  const int* lengths;     // [B] valid steps per row (clamped to [0, T]), or null: all T
  // GRU with (r*h) W_hn: xch carries da_n (one gate per slice, gran/slice
  // above) and xch2 carries [da_r, da_z] (two gates per slice)
  void* xch2;
  int gran2, slice2;
  long long ring_step2, ring_group2;
  int paper;
  const void* w_hh;       // layer block [D*G*H, H]
  const float* reserve;   // [D][T][B][R][H]
  const float* y;         // layer output [T, B, D*H]
  const float* h0;        // this layer's rows [D, B, H] or null
  const float* c0;
  const float* dy;        // [T, B, D*H]
  const float* dhy;       // [D, B, H] or null
  const float* dcy;
  void* dg;               // dG_i [T*B][dg_ld] in the compute type, columns gg_col (dX operand)
  void* dgT;              // dG_i^T [D*G*H][tb_ld], columns tb_k (dW_ih operand)
  void* dghT;             // GRU: dG_h^T, as dgT (dW_hh operand)
  int dg_ld;              // row stride of dg (>= D*nwg*G*U)
  int tb_ld;              // row stride of dgT / dghT (>= nchunk*T*Bc)
  float* dh0;             // [D, B, H] or null
  float* dc0;
  float* st_dh;           // carries between stepped launches [D*nchunk... ] laid out [D][B][H]
  float* st_dc;
  void* xch;              // exchange rings: per group [T + 1][nwg][slice]
  unsigned* flags;
  unsigned* err;
  unsigned spin_limit;
};

}  // namespace rnnk

// Kernel configuration chosen by the host planner.
struct RecConfig {
  int nt;      // 16-column MFMA tiles per workgroup
  int mt;      // 16-row batch tiles (Bc <= 16*mt)
  int kpw;     // K chunks per wave held in registers (upper bound)
  int nwaves;  // waves per workgroup
};

// Launchers (defined in the .hip files).  Return hipSuccess or the launch error.
hipError_t rnn_launch_gemm(const rnnk::GemmParams& p, int bf16, int epi, int batches, hipStream_t s);
// Dense MFMA throughput probe: `blocks` workgroups of 256 threads, `iters`
// rounds of eight independent MFMA chains per wave; one float per thread.
// kind 0: fp32 16x16x4, 1: bf16 16x16x32, 2: bf16 32x32x16.
hipError_t rnn_launch_mfma_peak(int kind, int blocks, int iters, float* out, hipStream_t s);
hipError_t rnn_launch_bf16_round_check(unsigned long long first, unsigned long long count, unsigned long long* mism,
                                       hipStream_t s);
// Up to four ranges to fill with 32-bit patterns in the same launch as
// another job (bytes: multiples of 4; count 0: none).
struct FillJob {
  void* p[4];
  unsigned long long bytes[4];
  uint32_t v[4];
  int count;
};
// Transposes; in_bf16 / out_bf16: element types of src (and alt) / out;
// `fill` (optional): ranges set by one more z slice of the same launch,
// complete when the launch is.
hipError_t rnn_launch_transpose(const rnnk::TransposeParams& p, int in_bf16, int out_bf16, hipStream_t s,
                                const FillJob* fill = nullptr);
// One launch for 1..4 transposes of the same element types.
hipError_t rnn_launch_transpose_batch(const rnnk::TransposeParams* ps, int n, int in_bf16, int out_bf16,
                                      hipStream_t s, const FillJob* fill = nullptr);
// fp32 -> bf16 (round to nearest even); `fill` (optional): ranges set by
// the same launch (its first blocks), complete when the launch is
hipError_t rnn_launch_convert(const float* src, long long ld_src, void* dst, long long ld_dst, int rows,
                              int cols, hipStream_t s, const FillJob* fill = nullptr);
// lds: dynamic LDS bytes (the ring-entry staging buffer, 0 when not staging)
hipError_t rnn_launch_fwd(const rnnk::FwdParams& p, int mode, int bf16, const RecConfig& c,
                          int grid, size_t lds, hipStream_t s);
hipError_t rnn_launch_bwd(const rnnk::BwdParams& p, int mode, int bf16, const RecConfig& c,
                          int grid, size_t lds, hipStream_t s);
// Fill ranges with 32-bit patterns (values null: zeros).  bytes: multiples of 4.
hipError_t rnn_launch_fill(void* const* ptrs, const size_t* bytes, const uint32_t* values, int n,
                           hipStream_t s);
hipError_t rnn_copy_state(float* dst, const float* src, size_t n, hipStream_t s);
// Inter-layer dropout of n fp32 elements (dst = src * keep / (1 - prob),
// in place allowed) and/or its keep mask (bytes, 1 = kept); either output
// may be null.  Mask of element e: Philox4x32-10 word e mod 4 at counter
// (e div 4, layer) under the 64-bit seed, kept when >= floor(prob * 2^32).
hipError_t rnn_launch_dropout(const float* src, float* dst, uint8_t* mask, long long n,
                              unsigned long long seed, int layer, double prob, hipStream_t s);
// Maximum co-resident workgroups of the fwd/bwd kernel for this config (0 if unsupported).
int rnn_fwd_max_resident(int mode, int bf16, const RecConfig& c, size_t lds);
// GRU flavours whose n reads (r*h) W_hn: two exchanges per step, persistent only.
hipError_t rnn_launch_gru2_fwd(const rnnk::FwdParams& p, int bf16, const RecConfig& c, int grid,
                               hipStream_t s);
hipError_t rnn_launch_gru2_bwd(const rnnk::BwdParams& p, int bf16, const RecConfig& c, int grid,
                               hipStream_t s);
int rnn_gru2_fwd_max_resident(int bf16, const RecConfig& c);
int rnn_gru2_bwd_max_resident(int bf16, const RecConfig& c);
bool rnn_gru2_fwd_config_supported(int bf16, const RecConfig& c);
bool rnn_gru2_bwd_config_supported(int bf16, const RecConfig& c);
int rnn_bwd_max_resident(int mode, int bf16, const RecConfig& c, size_t lds);
bool rnn_fwd_config_supported(int mode, int bf16, const RecConfig& c);
bool rnn_bwd_config_supported(int mode, int bf16, const RecConfig& c);

// Per-mode entry points of the recurrent sweeps (recurrent_<mode>_<fwd|bwd>.hip).
#define RNN_SWEEP_DECLS(NAME)                                                                         \
  hipError_t rnn_fwd_launch_##NAME(const rnnk::FwdParams& p, int bf16, const RecConfig& c, int grid,   \
                                   size_t lds, hipStream_t s);                                        \
  int rnn_fwd_resident_##NAME(int bf16, const RecConfig& c, size_t lds);                              \
  bool rnn_fwd_supported_##NAME(int bf16, const RecConfig& c);                                        \
  hipError_t rnn_bwd_launch_##NAME(const rnnk::BwdParams& p, int bf16, const RecConfig& c, int grid,   \
                                   size_t lds, hipStream_t s);                                        \
  int rnn_bwd_resident_##NAME(int bf16, const RecConfig& c, size_t lds);                              \
  bool rnn_bwd_supported_##NAME(int bf16, const RecConfig& c);
RNN_SWEEP_DECLS(tanh)
RNN_SWEEP_DECLS(lstm)
RNN_SWEEP_DECLS(gru)
