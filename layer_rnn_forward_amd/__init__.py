"""MI355X-native fused stacked RNN operator (vanilla tanh RNN, LSTM, GRU).

A thin ctypes binding over ``librnn_mi355x.so`` (HIP kernels for gfx950 plus
a C ABI, declared in ``include/rnn.h``).  Functions carry the C names and only
marshal arguments: torch tensors become device pointers, the current torch
stream becomes the HIP stream.  Every step of the computation runs in the
library's kernels; there is no fallback.  Loading fails loudly if the library
has not been built.
"""

from __future__ import annotations

import ctypes
import os

from ._binding import (  # noqa: F401
    MODES,
    RNNError,
    Handle,
    lib_path,
    load_library,
    rnn_create,
    rnn_destroy,
    rnn_set_schedule,
    rnn_set_sequence_lengths,
    rnn_set_dropout,
    rnn_dropout_mask,
    rnn_weights_size,
    rnn_weight_offset,
    rnn_workspace_size,
    rnn_forward_inference,
    rnn_forward_training,
    rnn_forward_inference_static,
    rnn_static_workspace_bytes,
    rnn_backward_data,
    rnn_exchange_floor,
    rnn_mfma_peak_probe,
    rnn_bf16_rounding_check,
    MFMA_PROBES,
    rnn_plan_info,
    PLAN_FIELDS,
    rnn_backward_weights,
    rnn_device_status,
    rnn_set_profiling,
    rnn_profile_read,
    rnn_status_string,
    pack_weights,
    unpack_weights,
    SCHED_AUTO,
    SCHED_PERSISTENT,
    SCHED_STEPPED,
    KERNEL_NAMES,
)

__all__ = [n for n in dir() if n.startswith("rnn_")] + [
    "MODES", "RNNError", "Handle", "pack_weights", "unpack_weights", "load_library", "lib_path",
]
