/*
 * rnn.h -- C ABI of the fused stacked RNN operator for AMD Instinct MI355X
 * (gfx950): vanilla tanh RNN, LSTM and GRU (PyTorch/cuDNN equations), forward
 * inference, forward training that fills a caller-owned reserved workspace,
 * and backward through time that reuses it.
 *
 * Sources (web pages, cited by title and section):
 *  - "fused RNN operator" design page (Apache MXNet wiki), *Problem
 *    Statement*: one fused operator for multi-layer, bidirectional vanilla /
 *    LSTM / GRU networks, inference and training; *Operator Registration*:
 *    forward intermediates are kept in a reserved workspace, reused by the
 *    backward pass and across iterations, released with the operator.
 *  - oneDNN issue #218 "rnn training example?": the workspace protocol (create
 *    a forward-training descriptor, query the workspace size, allocate it,
 *    pass it as a forward output and as a backward input); the PyTorch GRU
 *    snippet (two biases, gate chunks r, z, n); hx/cx/hy/cy shaped
 *    (num_layers*num_directions, batch, hidden); TNC input layout.
 *  - Keras issue #3692 "Exposing Cudnn v5 RNN models": the descriptor
 *    CudnnLSTM(num_layers, num_units, input_size).
 *  - The GRU flavours of oneDNN issue #218 ("GRU flavours": PyTorch/cuDNN,
 *    TensorFlow, and the original paper).  The TensorFlow and paper flavours
 *    need r for every unit before the n product, so their recurrent sweeps
 *    exchange twice per step and run only as persistent launches: with
 *    RNN_SCHED_STEPPED, or when the sweep's workgroups cannot all be resident,
 *    their compute calls return RNN_STATUS_NOT_CORESIDENT.  Layers always
 *    run one after another (no layer wavefront).
 *
 * General rules for every call
 *  - Every call returns rnn_status_t: 0 on success, a negative code otherwise.
 *    No call throws; no call prints.
 *  - Device pointers are plain HIP device addresses on the current device.
 *    The caller owns and allocates every device buffer, including the
 *    workspace.  The handle owns only host-side state and never allocates
 *    device memory.
 *  - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *    Compute calls only enqueue work on that stream and return; device-side
 *    faults surface at the next synchronisation.  A bounded wait inside the
 *    persistent kernels that expires (for example when another process keeps
 *    CUs busy so that the kernel's workgroups cannot all be resident) sets an
 *    error word in the workspace, makes every workgroup exit, and is reported
 *    by rnn_device_status().
 *  - All floating-point activations are fp32.  Matrices are fp32 or bf16
 *    (rnn_wtype_t); biases are always fp32; weight gradients are always fp32.
 *  - Calls on one handle are not thread-safe; distinct handles are
 *    independent.  Two calls that share a workspace must not run
 *    concurrently.
 */
#ifndef RNN_MI355X_H
#define RNN_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rnn_desc* rnn_handle_t;
typedef int rnn_status_t;

/* The enums below are passed as ints.  C++ gives them an int underlying type,
 * so that a value outside the listed ones (which the calls reject with
 * INVALID_ARG) is still a valid value of the type. */
#ifdef __cplusplus
#define RNN_ENUM_BASE : int
#else
#define RNN_ENUM_BASE
#endif

typedef enum RNN_ENUM_BASE {
  RNN_TANH = 0,      /* h' = tanh(W_ih x + b_ih + W_hh h + b_hh) */
  RNN_LSTM = 1,      /* gates i, f, g, o in this memory order */
  RNN_GRU = 2,       /* gates r, z, n; n = tanh(W_in x + b_in + r*(W_hn h + b_hn)),
                        h' = (1-z)*n + z*h (PyTorch / cuDNN flavour) */
  RNN_GRU_TF = 3,    /* gates r, z, n; n = tanh(W_in x + b_in + W_hn (r*h) + b_hn),
                        h' = (1-z)*n + z*h (TensorFlow flavour) */
  RNN_GRU_PAPER = 4  /* as RNN_GRU_TF with h' = (1-z)*h + z*n (original-paper flavour) */
} rnn_mode_t;

typedef enum RNN_ENUM_BASE { RNN_W_F32 = 0, RNN_W_BF16 = 1 } rnn_wtype_t;

/* Which parameter tensor of one (layer, direction), for rnn_weight_offset. */
typedef enum RNN_ENUM_BASE { RNN_W_IH = 0, RNN_W_HH = 1, RNN_B_IH = 2, RNN_B_HH = 3 } rnn_param_t;

/* Recurrent-sweep schedule (rnn_set_schedule). */
typedef enum RNN_ENUM_BASE {
  RNN_SCHED_AUTO = 0,       /* persistent when every workgroup fits on the GPU at once, else stepped */
  RNN_SCHED_PERSISTENT = 1, /* one launch per sweep; error RNN_STATUS_NOT_CORESIDENT if it cannot fit */
  RNN_SCHED_STEPPED = 2     /* one launch per time step (no device-wide waits) */
} rnn_schedule_t;

#define RNN_STATUS_SUCCESS 0
#define RNN_STATUS_INVALID_ARG (-1)
#define RNN_STATUS_UNSUPPORTED (-2)
#define RNN_STATUS_WORKSPACE_TOO_SMALL (-3)
#define RNN_STATUS_BAD_CALL_ORDER (-4)
#define RNN_STATUS_NOT_CORESIDENT (-5)
#define RNN_STATUS_DEVICE (-6)
#define RNN_STATUS_DEVICE_TIMEOUT (-7)

/* Create a descriptor of a stacked RNN: `num_layers` layers, `num_dirs`
 * directions (1 or 2), layer-0 input width `input_size`, hidden width
 * `hidden_size` per direction (the (num_layers, num_units, input_size)
 * descriptor of Keras issue #3692 plus mode and direction count).  Layers
 * l > 0 take the concatenation [forward | backward] of the layer below
 * (width num_dirs*hidden_size).  Errors: INVALID_ARG for a NULL `out`,
 * non-positive sizes, num_dirs not 1 or 2, unknown mode or wtype.  On error
 * *out is set to NULL. */
rnn_status_t rnn_create(rnn_handle_t* out, rnn_mode_t mode, int num_layers, int num_dirs,
                        int input_size, int hidden_size, rnn_wtype_t wtype);

/* Release the descriptor (host memory only).  NULL is accepted. */
rnn_status_t rnn_destroy(rnn_handle_t h);

/* Choose how the recurrent sweeps are launched (default RNN_SCHED_AUTO).
 * Results are bitwise identical across schedules.  The TensorFlow and
 * original-paper GRU flavours run only persistently: with RNN_SCHED_STEPPED
 * their compute calls return RNN_STATUS_NOT_CORESIDENT. */
rnn_status_t rnn_set_schedule(rnn_handle_t h, rnn_schedule_t s);

/* Variable-length (packed) batches: the packed-sequence question of oneDNN
 * issue #218, with the semantics of PyTorch's packed sequences (the pages
 * fix none).  `lengths` is a DEVICE pointer to int32 [B] (B of every later
 * compute call) giving each batch row's number of valid steps; values are
 * clamped to [0, T].  Row b is processed only at steps t < lengths[b]: at the
 * other steps its state (h, and c for LSTM) is carried unchanged and its y is
 * 0, so direction 0 stops and direction 1 starts at t = lengths[b] - 1 and
 * hy/cy are the states after each direction's last valid step.  The backward
 * pass ignores dy at those steps, passes dh/dc through them, and gives zero dx
 * there; dW/db collect only valid steps.  Rows of length 0 return h0/c0 and
 * dhy/dcy unchanged.  NULL (the default) means every row has T steps.  The
 * pointer is stored in the handle (the caller keeps the buffer alive and
 * unchanged while calls that use it run) and applies to the compute calls
 * that follow; rnn_backward_data and rnn_backward_weights return
 * BAD_CALL_ORDER if it changed since the rnn_forward_training they follow.
 * Errors: INVALID_ARG for a NULL handle. */
rnn_status_t rnn_set_sequence_lengths(rnn_handle_t h, const int* lengths);

/* Inter-layer dropout in training (the MKL-DNN issue thread on the "fused
 * RNN" pages asks for it as cuDNN offers it; the pages fix no semantics, so
 * cuDNN's and PyTorch's are taken).  In rnn_forward_training the input of
 * every layer l >= 1 is y_{l-1} * keep / (1 - p); x, the recurrent state and
 * the top layer's y are never dropped, and rnn_forward_inference never drops.
 * The backward calls apply the same multiplier to the gradient of y_{l-1}
 * and use the dropped input for dW_ih, with the p and seed of the forward
 * they follow.  The keep mask is not stored: element e of layer l's
 * [T][B][D*H] input is kept when word (e mod 4) of Philox4x32-10 (Salmon et
 * al., "Parallel random numbers: as easy as 1, 2, 3", SC'11) at counter
 * (e div 4 mod 2^32, e div 4 div 2^32, l, 0) under the key (seed mod 2^32,
 * seed div 2^32) is at least floor(p * 2^32); p = 1 drops everything.  A
 * different seed per training step gives fresh masks.  p > 0 enlarges the
 * training workspace (one fp32 [T][B][D*H] slot per dropped layer), so size
 * it after this call.  Errors: INVALID_ARG for a NULL handle or p outside
 * [0, 1] (or NaN).  Default p = 0. */
rnn_status_t rnn_set_dropout(rnn_handle_t h, double p, unsigned long long seed);

/* The keep mask a training pass with the current dropout setting applies to
 * layer `layer`'s input (1 <= layer < num_layers): T*B*num_dirs*hidden_size
 * bytes at the DEVICE pointer `mask`, 1 = kept, 0 = dropped, TNC order,
 * written on `stream`.  Errors: INVALID_ARG for a NULL handle, a layer out of
 * range, negative sizes or a NULL mask with a non-empty shape; DEVICE for a
 * failed launch. */
rnn_status_t rnn_dropout_mask(rnn_handle_t h, void* stream, int T, int B, int layer,
                              unsigned char* mask);

/* Bytes of the packed weight buffer (grad = 0: matrices in the handle's
 * wtype, biases fp32) or of the packed weight-gradient buffer (grad = 1: all
 * fp32). */
rnn_status_t rnn_weights_size(rnn_handle_t h, int grad, size_t* bytes);

/* Byte offset and element count of one parameter tensor inside the packed
 * (grad = 0) or gradient (grad = 1) buffer.  Each tensor is stored row-major
 * in the PyTorch layout: W_ih [G*H, I_l], W_hh [G*H, H], b_ih [G*H],
 * b_hh [G*H], G = 1 (tanh), 4 (LSTM, rows i,f,g,o), 3 (GRU, rows r,z,n) --
 * the chunk order of the PyTorch GRU snippet in oneDNN issue #218.  The two
 * directions of one tensor kind of a layer are adjacent (direction 1 right
 * after direction 0); each such block starts on 256 bytes.  Element type: matrices rnn_wtype_t of the
 * handle (fp32 when grad = 1), biases fp32.  Errors: INVALID_ARG for
 * out-of-range layer/dir/which or NULL outputs. */
rnn_status_t rnn_weight_offset(rnn_handle_t h, int grad, int layer, int dir, rnn_param_t which,
                               size_t* byte_offset, size_t* elem_count);

/* Source: oneDNN issue #218, the workspace protocol (query the size, then
 * allocate).
 * Workspace bytes for T steps and batch B: training = 0 for
 * rnn_forward_inference, training = 1 for the forward_training /
 * backward_data / backward_weights sequence (the size query of the oneDNN
 * workspace protocol).  The size depends on (handle, T, B, training) only.
 * Errors: INVALID_ARG for T < 0, B < 0 or NULL bytes; UNSUPPORTED when the
 * recurrent sweeps have no kernel configuration for the shape (the compute
 * calls return the same status): each workgroup keeps its slice of W_hh in
 * registers, which bounds the hidden size.  Hidden sizes up to 1024 with
 * fp32 weights and 2048 with bf16 weights are supported for every mode,
 * stack and batch; larger ones only where the mode, the pass and the batch
 * chunking leave room (at most 2048 / 4096). */
rnn_status_t rnn_workspace_size(rnn_handle_t h, int T, int B, int training, size_t* bytes);

/* Forward pass without saving intermediates.  Source: the MXNet "fused RNN
 * operator" page, Problem Statement (one fused call for stacked, optionally
 * bidirectional vanilla / LSTM / GRU layers, inference); oneDNN issue #218 for
 * the TNC input layout and the (num_layers*num_directions, batch, hidden)
 * state shape; the GRU equations of its PyTorch snippet.
 *   x   [T, B, I] fp32 (TNC)             y   [T, B, D*H] fp32; direction 0 in
 *   h0  [L*D, B, H] fp32 or NULL (zeros)      columns [0,H), direction 1 in [H,2H)
 *   c0  [L*D, B, H] fp32 or NULL; LSTM only (must be NULL otherwise)
 *   W   packed weights (rnn_weight_offset)
 *   hy  [L*D, B, H] or NULL (not written); cy likewise, LSTM only
 *   ws  at least rnn_workspace_size(h, T, B, 0) bytes, 256-byte aligned
 * Index l*D + d of h0/hy is layer l, direction d.  Direction 1 walks
 * t = T-1 .. 0 and its hy is the state after t = 0.  T = 0 or B = 0 is
 * valid: hy/cy are copied from h0/c0 (zeros if NULL) and y is empty.
 * Using a workspace here invalidates a pending training sequence on the same
 * workspace.  Errors: INVALID_ARG (NULL required pointers, c0/cy given for a
 * non-LSTM mode, misaligned ws), WORKSPACE_TOO_SMALL, UNSUPPORTED (hidden
 * size beyond the kernels' limit, rnn_workspace_size), NOT_CORESIDENT (with
 * RNN_SCHED_PERSISTENT, or for the two-exchange GRU flavours with
 * RNN_SCHED_STEPPED or when the sweep's workgroups cannot all be resident), DEVICE (launch failure). */
rnn_status_t rnn_forward_inference(rnn_handle_t h, void* stream, int T, int B, const float* x,
                                   const float* h0, const float* c0, const void* W, float* y,
                                   float* hy, float* cy, void* ws, size_t ws_bytes);

/* Source: oneDNN issue #218, the workspace protocol (the forward-training
 * call takes the workspace as an output); the MXNet "fused RNN operator" page,
 * Operator Registration (forward intermediates kept for backward, the buffer
 * reused across iterations).
 * As rnn_forward_inference, and additionally fills the workspace (at least
 * rnn_workspace_size(h, T, B, 1) bytes) with what backward_data reuses:
 * post-activation gates and cell states per (layer, direction, step), GRU's
 * W_hn h + b_hn, and every inner layer's output.  The outputs y, hy, cy are
 * bitwise equal to rnn_forward_inference's. */
rnn_status_t rnn_forward_training(rnn_handle_t h, void* stream, int T, int B, const float* x,
                                  const float* h0, const float* c0, const void* W, float* y,
                                  float* hy, float* cy, void* ws, size_t ws_bytes);

/* Source: oneDNN issue #218, the workspace protocol (the backward call takes
 * the forward's workspace as an input); the MXNet "fused RNN operator" page,
 * Operator Registration (backward reuses the saved intermediates).  The split
 * into a data part and a weight part is this library's.
 * Backward through time, data part.  Must follow rnn_forward_training on the
 * same handle with the same T, B and workspace (else BAD_CALL_ORDER).
 *   y    the forward's y; dy [T, B, D*H]; dhy, dcy [L*D, B, H] or NULL (zeros;
 *        dcy LSTM only); W, h0, c0 as given to the forward.
 *   dx   [T, B, I] written; dh0, dc0 [L*D, B, H] or NULL (not written; dc0
 *        LSTM only).
 * Stores the gate gradients of every layer in the workspace for
 * rnn_backward_weights.  Same error codes as the forward. */
rnn_status_t rnn_backward_data(rnn_handle_t h, void* stream, int T, int B, const float* y,
                               const float* dy, const float* dhy, const float* dcy, const void* W,
                               const float* h0, const float* c0, float* dx, float* dh0,
                               float* dc0, void* ws, size_t ws_bytes);

/* Source: as rnn_backward_data; the weight gradients of all time steps as
 * single products follow the "Combined GEMMs" and "Combining Inputs" rows of
 * the cuDNN-5 optimisation table in Keras issue #3692.
 * Backward through time, weight part.  Must follow rnn_backward_data with the
 * same T, B and workspace (else BAD_CALL_ORDER).  x, h0 and y are the
 * forward's.  dW (rnn_weights_size(h, 1, .) bytes, layout of
 * rnn_weight_offset with grad = 1) is OVERWRITTEN with dLoss/dW, dLoss/db.
 * The gate gradients backward_data left in the workspace are only read; its
 * operand scratch (transposed inputs and states, split-K partials) is
 * overwritten, so the workspace is an in/out argument.  May be called again
 * without repeating backward_data. */
rnn_status_t rnn_backward_weights(rnn_handle_t h, void* stream, int T, int B, const float* x,
                                  const float* h0, const float* y, void* ws, size_t ws_bytes,
                                  float* dW);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * rnn_forward_inference with the workspace replaced by a fixed device array
 * of the library, rnn_static_workspace_bytes() bytes (128 MiB: the
 * single-layer Deep Speech 2 shape, T = 300, B = 20, input = hidden = 800,
 * needs about 94 MiB), one per device, placed when the library's code is
 * loaded on that device and held until the process ends.  Arguments and
 * results as rnn_forward_inference (bitwise equal outputs).  The call
 * allocates nothing (per-launch profiling events are not recorded in it) and
 * sets what must start at zero (flags, error word) itself; nothing else
 * carries over from one call to the next.  Every call on one device shares
 * that device's array: calls that overlap in time on one device (two host
 * threads, two streams) race and give undefined results.  An expired bounded
 * wait (see rnn_device_status) is recorded in that array, where no call
 * reports it.  Errors: as rnn_forward_inference, and
 * WORKSPACE_TOO_SMALL when rnn_workspace_size(h, T, B, 0) exceeds the
 * array. */
rnn_status_t rnn_forward_inference_static(rnn_handle_t h, void* stream, int T, int B, const float* x,
                                          const float* h0, const float* c0, const void* W, float* y,
                                          float* hy, float* cy);
size_t rnn_static_workspace_bytes(void);

/* Diagnostic: the latency floor of the persistent forward sweep.  Runs the
 * launch that rnn_forward_inference (training = 0) or rnn_forward_training
 * (training = 1) would use for its first recurrent sweep -- the two passes
 * may plan different batch chunks -- with the same grid, the same per-step
 * waits on the producers' flags and the same exchange-ring stores and flag
 * publication (the step-wise grid synchronisation of the persistent-RNN
 * design discussed in the TVM thread "Persist RNN Implementation"), but no
 * weights, arithmetic or outputs, so that its time divided by the steps is
 * the cost of the exchange alone.  Writes only the workspace (at least
 * rnn_workspace_size(h, T, B, training) bytes); invalidates a pending
 * training sequence on it.  Timed like the other launches by
 * rnn_set_profiling (kernel id 7).  Errors: as rnn_forward_inference, and
 * NOT_CORESIDENT when the sweep could not run persistently. */
rnn_status_t rnn_exchange_floor(rnn_handle_t h, void* stream, int T, int B, int training, void* ws,
                                size_t ws_bytes);

/* Diagnostic: the device's achievable dense MFMA throughput, the measured
 * denominator next to the published peak when the time-parallel products
 * are rated against the matrix roofline.  Enqueues on `stream` one launch of
 * `blocks` workgroups of 256 threads (four waves); every wave runs `iters`
 * rounds of eight independent MFMA accumulations on register operands:
 *   kind 0: four v_mfma_f32_16x16x4_f32 per round and chain (8192 flop),
 *   kind 1: v_mfma_f32_16x16x32_bf16 (16384 flop),
 *   kind 2: v_mfma_f32_32x32x16_bf16 (32768 flop),
 * so the launch performs blocks * 4 * iters * 8 * (that many) flop; time it
 * with events on `stream`.  Writes one float per thread to `out` (device
 * memory of the caller, at least blocks * 256 floats), exactly
 * A * iters * K / 512 with (A, K) = (32, 16), (32, 32), (128, 16) for kinds
 * 0, 1, 2 -- a check that no work was skipped.  Touches nothing else; needs
 * no handle.  Errors: INVALID_ARG for an unknown kind, blocks <= 0,
 * iters <= 0 or a null `out`; DEVICE for a launch error. */
rnn_status_t rnn_mfma_peak_probe(void* stream, int kind, int blocks, int iters, float* out);

/* Diagnostic: checks the fp32 -> bf16 rounding that every bf16 product
 * operand and exchanged value goes through (round to nearest even, the
 * rounding the bf16-weight path states) on the device: for every fp32 bit
 * pattern in
 * [first, first + count) (within 0 .. 2^32) the library's conversion is
 * compared with round-to-nearest-even written out on the bits, and a NaN
 * must stay a NaN.  Adds the number of mismatches to *mismatches (a device
 * pointer to one unsigned 64-bit integer that the caller initialises);
 * enqueues on `stream` and returns.  Touches nothing else; needs no handle.
 * Errors: INVALID_ARG for a NULL pointer or a range past 2^32; DEVICE for a
 * launch error. */
rnn_status_t rnn_bf16_rounding_check(void* stream, unsigned long long first, unsigned long long count,
                                     unsigned long long* mismatches);

/* Diagnostic: the launch plan of the recurrent sweeps for (T, B, training)
 * as the compute calls would make it now (environment and device included).
 * Writes 16 ints to `out` (host memory): out[0..7] the forward sweep and
 * out[8..15] the backward sweep (zeros when training = 0), each as: batch
 * chunks, rows per chunk, hidden units per workgroup, workgroups per group,
 * groups, grid (workgroups launched), placement (0: linear, 1: XCD-local
 * recurrence groups, r >= 2: runs of r consecutive workgroups per XCD),
 * persistent (1) or stepped (0).  Host only; touches no
 * device memory.  Errors: INVALID_ARG for a NULL handle or out, T < 0 or
 * B < 0; UNSUPPORTED when no kernel configuration fits. */
rnn_status_t rnn_plan_info(rnn_handle_t h, int T, int B, int training, int* out);

/* Synchronise `stream` and report whether a kernel that used `ws` hit an
 * expired bounded wait since the workspace was last handed to a compute
 * call: RNN_STATUS_SUCCESS or RNN_STATUS_DEVICE_TIMEOUT (or DEVICE if the
 * synchronisation itself failed). */
rnn_status_t rnn_device_status(rnn_handle_t h, void* stream, const void* ws, size_t ws_bytes);

/* Per-kernel timing with HIP events recorded on the caller's stream around
 * every launch (off by default; adds one event pair per launch).  Kernel ids:
 * 0 input-projection GEMM, 1 recurrent forward sweep, 2 recurrent backward
 * sweep, 3 dX GEMM, 4 dW GEMMs, 5 workspace fill, 6 operand preparation
 * (bf16 conversion and transposes for the GEMMs), 7 exchange probe
 * (rnn_exchange_floor), 8 inter-layer dropout passes.  rnn_profile_read
 * synchronises, accumulates the elapsed times of finished launches and
 * returns the launch count and total milliseconds for `kernel` since the last
 * reset (rnn_set_profiling(h, 1) resets). */
rnn_status_t rnn_set_profiling(rnn_handle_t h, int enable);
rnn_status_t rnn_profile_read(rnn_handle_t h, int kernel, long long* launches, double* total_ms);

/* Static text for a status code. */
const char* rnn_status_string(rnn_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* RNN_MI355X_H */
