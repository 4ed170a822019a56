// Dispatch of the persistent recurrent sweeps by cell mode, and the small
// fill and copy kernels of the library (gfx950).  The sweep kernels are
// in recurrent_sweeps.h, instantiated per mode in recurrent_<mode>_<fwd|bwd>.hip.
#include "rnn_common.h"

using namespace rnnk;

namespace {

// ===================================================================== misc
struct FillArgs {
  void* p[8];
  size_t n[8];      // bytes (multiple of 4)
  uint32_t v[8];    // 32-bit fill pattern
  int count;
};

__global__ void fill_kernel(const FillArgs a) {
  for (int i = 0; i < a.count; ++i) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.p[i]);
    const size_t nw = a.n[i] / 4;
    const uint32_t v = a.v[i];
    for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < nw; k += (size_t)gridDim.x * blockDim.x)
      dst[k] = v;
  }
}

__global__ void copy_kernel(float* dst, const float* src, size_t n) {
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (size_t)gridDim.x * blockDim.x)
    dst[k] = src ? src[k] : 0.f;
}
}  // namespace

#define RNN_BY_MODE(PREFIX, DFLT, ...)                              \
  switch (mode) {                                                   \
    case MODE_TANH: return PREFIX##tanh(__VA_ARGS__);               \
    case MODE_LSTM: return PREFIX##lstm(__VA_ARGS__);               \
    case MODE_GRU: return PREFIX##gru(__VA_ARGS__);                 \
    default: return DFLT;                                           \
  }

hipError_t rnn_launch_fwd(const FwdParams& p, int mode, int bf16, const RecConfig& c, int grid,
                          size_t lds, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  RNN_BY_MODE(rnn_fwd_launch_, hipErrorInvalidValue, p, bf16, c, grid, lds, s)
}
int rnn_fwd_max_resident(int mode, int bf16, const RecConfig& c, size_t lds) {
  RNN_BY_MODE(rnn_fwd_resident_, 0, bf16, c, lds)
}
bool rnn_fwd_config_supported(int mode, int bf16, const RecConfig& c) {
  RNN_BY_MODE(rnn_fwd_supported_, false, bf16, c)
}
hipError_t rnn_launch_bwd(const BwdParams& p, int mode, int bf16, const RecConfig& c, int grid,
                          size_t lds, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  RNN_BY_MODE(rnn_bwd_launch_, hipErrorInvalidValue, p, bf16, c, grid, lds, s)
}
int rnn_bwd_max_resident(int mode, int bf16, const RecConfig& c, size_t lds) {
  RNN_BY_MODE(rnn_bwd_resident_, 0, bf16, c, lds)
}
bool rnn_bwd_config_supported(int mode, int bf16, const RecConfig& c) {
  RNN_BY_MODE(rnn_bwd_supported_, false, bf16, c)
}

hipError_t rnn_launch_fill(void* const* ptrs, const size_t* bytes, const uint32_t* values, int n,
                           hipStream_t s) {
  FillArgs a{};
  size_t total = 0;
  int k = 0;
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i] || bytes[i] == 0) continue;
    if (k == 8) return hipErrorInvalidValue;
    a.p[k] = ptrs[i];
    a.n[k] = bytes[i];
    a.v[k] = values ? values[i] : 0u;
    total += bytes[i];
    ++k;
  }
  a.count = k;
  if (k == 0) return hipSuccess;
  size_t blocks = (total / 4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t rnn_copy_state(float* dst, const float* src, size_t n, hipStream_t s) {
  if (!dst || n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}
