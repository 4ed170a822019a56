"""ctypes binding of include/rnn.h.  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

MODES = {"rnn_tanh": 0, "lstm": 1, "gru": 2, "gru_tf": 3, "gru_paper": 4}
WTYPES = {"f32": 0, "bf16": 1}
SCHED_AUTO, SCHED_PERSISTENT, SCHED_STEPPED = 0, 1, 2
KERNEL_NAMES = ["gemm_input", "recurrent_fwd", "recurrent_bwd", "gemm_dx", "gemm_dw", "fill", "prep",
                "exchange_probe", "dropout"]
STATUS_DEVICE_TIMEOUT = -7

_LIB = None


class RNNError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {rnn_status_string(status)} ({status})")


def lib_path() -> str:
    """The in-tree library, or the build named by RNN_LIB (e.g. the
    host-sanitizer build of build.build_sanitized)."""
    return os.environ.get("RNN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "librnn_mi355x.so")


def load_library():
    """Load the HIP library; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP extension first "
            "(python -m layer_rnn_forward_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    psz = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "rnn_create": [ctypes.POINTER(vp), i, i, i, i, i, i],
        "rnn_destroy": [vp],
        "rnn_set_schedule": [vp, i],
        "rnn_set_sequence_lengths": [vp, vp],
        "rnn_set_dropout": [vp, ctypes.c_double, ctypes.c_ulonglong],
        "rnn_dropout_mask": [vp, vp, i, i, i, vp],
        "rnn_weights_size": [vp, i, psz],
        "rnn_weight_offset": [vp, i, i, i, i, psz, psz],
        "rnn_workspace_size": [vp, i, i, i, psz],
        "rnn_forward_inference": [vp, vp, i, i, vp, vp, vp, vp, vp, vp, vp, vp, sz],
        "rnn_forward_training": [vp, vp, i, i, vp, vp, vp, vp, vp, vp, vp, vp, sz],
        "rnn_forward_inference_static": [vp, vp, i, i, vp, vp, vp, vp, vp, vp, vp],
        "rnn_backward_data": [vp, vp, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz],
        "rnn_backward_weights": [vp, vp, i, i, vp, vp, vp, vp, sz, vp],
        "rnn_device_status": [vp, vp, vp, sz],
        "rnn_exchange_floor": [vp, vp, i, i, i, vp, sz],
        "rnn_mfma_peak_probe": [vp, i, i, i, vp],
        "rnn_bf16_rounding_check": [vp, ctypes.c_ulonglong, ctypes.c_ulonglong, vp],
        "rnn_plan_info": [vp, i, i, i, ctypes.POINTER(ctypes.c_int)],
        "rnn_set_profiling": [vp, i],
        "rnn_profile_read": [vp, i, ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_double)],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.rnn_status_string.argtypes = [ctypes.c_int]
    lib.rnn_status_string.restype = ctypes.c_char_p
    lib.rnn_static_workspace_bytes.argtypes = []
    lib.rnn_static_workspace_bytes.restype = ctypes.c_size_t
    _LIB = lib
    return lib


def rnn_status_string(s: int) -> str:
    return load_library().rnn_status_string(int(s)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise RNNError(status, where)


class Handle:
    """Owns an ``rnn_handle_t``; remembers the descriptor for marshalling."""

    def __init__(self, ptr, mode, num_layers, num_dirs, input_size, hidden_size, wtype):
        self.ptr = ptr
        self.mode, self.L, self.D = mode, num_layers, num_dirs
        self.I, self.H, self.wtype = input_size, hidden_size, wtype
        self.G = {"rnn_tanh": 1, "lstm": 4, "gru": 3, "gru_tf": 3, "gru_paper": 3}[mode]
        self.lengths = None

    def __del__(self):
        try:
            if self.ptr is not None and _LIB is not None:
                _LIB.rnn_destroy(self.ptr)
                self.ptr = None
        except Exception:
            pass


def _ptr(t, name, dtype=torch.float32):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or None")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else ctypes.c_void_p(t.data_ptr() or 0)


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def rnn_create(mode, num_layers, num_dirs, input_size, hidden_size, wtype="f32") -> Handle:
    lib = load_library()
    out = ctypes.c_void_p()
    _check(lib.rnn_create(ctypes.byref(out), MODES[mode], num_layers, num_dirs, input_size,
                          hidden_size, WTYPES[wtype]), "rnn_create")
    return Handle(out, mode, num_layers, num_dirs, input_size, hidden_size, wtype)


def rnn_destroy(h: Handle):
    if h.ptr is not None:
        _check(load_library().rnn_destroy(h.ptr), "rnn_destroy")
        h.ptr = None


def rnn_set_schedule(h: Handle, sched: int):
    _check(load_library().rnn_set_schedule(h.ptr, int(sched)), "rnn_set_schedule")


def rnn_set_sequence_lengths(h: Handle, lengths):
    """Per-row valid step counts (int32 device tensor [B]) for the calls that
    follow, or None for full-length rows.  The handle keeps a reference so the
    tensor outlives its use."""
    _check(load_library().rnn_set_sequence_lengths(h.ptr, _ptr(lengths, "lengths", torch.int32)),
           "rnn_set_sequence_lengths")
    h.lengths = lengths


def rnn_set_dropout(h: Handle, p: float, seed: int = 0):
    """Inter-layer dropout probability and 64-bit seed of the training passes
    that follow (p = 0 switches it off)."""
    _check(load_library().rnn_set_dropout(h.ptr, float(p), int(seed) & ((1 << 64) - 1)),
           "rnn_set_dropout")


def rnn_dropout_mask(h: Handle, T: int, B: int, layer: int, mask):
    """Write the keep mask (uint8 device tensor, T*B*D*H elements) a training
    pass applies to layer ``layer``'s input."""
    _check(load_library().rnn_dropout_mask(h.ptr, _stream(), T, B, layer,
                                           _ptr(mask, "mask", torch.uint8)), "rnn_dropout_mask")


def rnn_weights_size(h: Handle, grad: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(load_library().rnn_weights_size(h.ptr, int(grad), ctypes.byref(n)), "rnn_weights_size")
    return n.value


def rnn_weight_offset(h: Handle, grad: int, layer: int, direction: int, which: int):
    off, cnt = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().rnn_weight_offset(h.ptr, int(grad), layer, direction, which,
                                            ctypes.byref(off), ctypes.byref(cnt)),
           "rnn_weight_offset")
    return off.value, cnt.value


def rnn_workspace_size(h: Handle, T: int, B: int, training: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().rnn_workspace_size(h.ptr, T, B, int(training), ctypes.byref(n)),
           "rnn_workspace_size")
    return n.value


def _fwd(fn, h, T, B, x, h0, c0, W, y, hy, cy, ws, name):
    lib = load_library()
    _check(getattr(lib, fn)(h.ptr, _stream(), T, B, _ptr(x, "x"), _ptr(h0, "h0"), _ptr(c0, "c0"),
                            _ptr(W, "W", None), _ptr(y, "y"), _ptr(hy, "hy"), _ptr(cy, "cy"),
                            _ptr(ws, "ws", None), _nbytes(ws)), name)


def rnn_forward_inference(h, T, B, x, h0, c0, W, y, hy, cy, ws):
    _fwd("rnn_forward_inference", h, T, B, x, h0, c0, W, y, hy, cy, ws, "rnn_forward_inference")


def rnn_forward_training(h, T, B, x, h0, c0, W, y, hy, cy, ws):
    _fwd("rnn_forward_training", h, T, B, x, h0, c0, W, y, hy, cy, ws, "rnn_forward_training")


def rnn_forward_inference_static(h, T, B, x, h0, c0, W, y, hy, cy):
    """rnn_forward_inference on the library's fixed device array instead of a
    caller workspace (allocates nothing; calls on one device must not overlap)."""
    lib = load_library()
    _check(lib.rnn_forward_inference_static(h.ptr, _stream(), T, B, _ptr(x, "x"), _ptr(h0, "h0"),
                                            _ptr(c0, "c0"), _ptr(W, "W", None), _ptr(y, "y"),
                                            _ptr(hy, "hy"), _ptr(cy, "cy")), "rnn_forward_inference_static")


def rnn_static_workspace_bytes() -> int:
    return int(load_library().rnn_static_workspace_bytes())


def rnn_backward_data(h, T, B, y, dy, dhy, dcy, W, h0, c0, dx, dh0, dc0, ws):
    _check(load_library().rnn_backward_data(
        h.ptr, _stream(), T, B, _ptr(y, "y"), _ptr(dy, "dy"), _ptr(dhy, "dhy"), _ptr(dcy, "dcy"),
        _ptr(W, "W", None), _ptr(h0, "h0"), _ptr(c0, "c0"), _ptr(dx, "dx"), _ptr(dh0, "dh0"),
        _ptr(dc0, "dc0"), _ptr(ws, "ws", None), _nbytes(ws)), "rnn_backward_data")


def rnn_backward_weights(h, T, B, x, h0, y, ws, dW):
    _check(load_library().rnn_backward_weights(
        h.ptr, _stream(), T, B, _ptr(x, "x"), _ptr(h0, "h0"), _ptr(y, "y"), _ptr(ws, "ws", None),
        _nbytes(ws), _ptr(dW, "dW", None)), "rnn_backward_weights")


def rnn_device_status(h, ws) -> int:
    """0, or -7 (a bounded device wait expired); raises on other errors."""
    s = load_library().rnn_device_status(h.ptr, _stream(), _ptr(ws, "ws", None), _nbytes(ws))
    if s not in (0, STATUS_DEVICE_TIMEOUT):
        raise RNNError(s, "rnn_device_status")
    return s


def rnn_exchange_floor(h, T, B, ws, training=False):
    """Run the forward sweep's exchange alone (same launch, no arithmetic),
    with the plan of the training (True) or inference (False) pass."""
    _check(load_library().rnn_exchange_floor(h.ptr, _stream(), T, B, 1 if training else 0,
                                             _ptr(ws, "ws", None), _nbytes(ws)),
           "rnn_exchange_floor")


PLAN_FIELDS = ("nchunk", "rows", "units", "nwg", "groups", "grid", "place", "persistent")


def rnn_plan_info(h, T: int, B: int, training: bool):
    """The recurrent sweeps' launch plan: ``{"fwd": {...}, "bwd": {...}}``
    with the fields of PLAN_FIELDS (``bwd`` only for training)."""
    out = (ctypes.c_int * 16)()
    _check(load_library().rnn_plan_info(h.ptr, T, B, 1 if training else 0, out), "rnn_plan_info")
    r = {"fwd": dict(zip(PLAN_FIELDS, out[0:8]))}
    if training:
        r["bwd"] = dict(zip(PLAN_FIELDS, out[8:16]))
    return r


MFMA_PROBES = {"f32_16x16x4": 0, "bf16_16x16x32": 1, "bf16_32x32x16": 2}


def rnn_mfma_peak_probe(kind: str, blocks: int, iters: int, out):
    """Enqueue the dense MFMA throughput probe (`kind` a key of MFMA_PROBES)
    on the current stream; `out` is a float32 device tensor of at least
    blocks*256 elements."""
    if out.numel() < blocks * 256:
        raise ValueError("out holds fewer than blocks*256 floats")
    _check(load_library().rnn_mfma_peak_probe(_stream(), MFMA_PROBES[kind], blocks, iters,
                                              _ptr(out, "out")), "rnn_mfma_peak_probe")


def rnn_bf16_rounding_check(first: int, count: int, mismatches):
    """Enqueue the device check of the fp32 -> bf16 rounding over the bit
    patterns [first, first + count); adds the mismatch count to
    `mismatches`, an int64 device tensor of one element the caller zeroes."""
    _check(load_library().rnn_bf16_rounding_check(_stream(), first, count,
                                                  _ptr(mismatches, "mismatches", torch.int64)),
           "rnn_bf16_rounding_check")


def rnn_set_profiling(h, enable: bool):
    _check(load_library().rnn_set_profiling(h.ptr, int(bool(enable))), "rnn_set_profiling")


def rnn_profile_read(h, kernel: int):
    n, ms = ctypes.c_longlong(), ctypes.c_double()
    _check(load_library().rnn_profile_read(h.ptr, int(kernel), ctypes.byref(n), ctypes.byref(ms)),
           "rnn_profile_read")
    return n.value, ms.value


# ------------------------------------------------------------ weight packing
def pack_weights(h: Handle, params, device="cuda") -> torch.Tensor:
    """Place ``params[l][d] = {w_ih, w_hh, b_ih, b_hh}`` (arrays) into the
    packed buffer at the offsets the library reports; matrices in the handle's
    element type (round to nearest even for bf16), biases fp32."""
    buf = torch.zeros(rnn_weights_size(h, 0), dtype=torch.uint8)
    for l in range(h.L):
        for d in range(h.D):
            for which, name in enumerate(("w_ih", "w_hh", "b_ih", "b_hh")):
                off, cnt = rnn_weight_offset(h, 0, l, d, which)
                a = torch.as_tensor(np.ascontiguousarray(params[l][d][name]), dtype=torch.float64)
                assert a.numel() == cnt, (l, d, name, a.numel(), cnt)
                dt = torch.bfloat16 if (which < 2 and h.wtype == "bf16") else torch.float32
                raw = a.reshape(-1).to(dt).view(torch.uint8)
                buf[off:off + raw.numel()] = raw
    return buf.to(device)


def unpack_weights(h: Handle, buf: torch.Tensor, grad: int = 1):
    """Inverse of :func:`pack_weights` (``grad=1``: the fp32 gradient buffer)
    -> ``[l][d]{name: float64 numpy array}``."""
    cpu = buf.detach().to("cpu").contiguous().view(-1).view(torch.uint8)
    out = []
    for l in range(h.L):
        I_l = h.I if l == 0 else h.D * h.H
        row = []
        for d in range(h.D):
            p = {}
            for which, name in enumerate(("w_ih", "w_hh", "b_ih", "b_hh")):
                off, cnt = rnn_weight_offset(h, grad, l, d, which)
                bf = (not grad) and which < 2 and h.wtype == "bf16"
                nb = cnt * (2 if bf else 4)
                t = cpu[off:off + nb].view(torch.bfloat16 if bf else torch.float32).to(torch.float64)
                shape = {0: (h.G * h.H, I_l), 1: (h.G * h.H, h.H)}.get(which, (h.G * h.H,))
                p[name] = t.reshape(shape).numpy()
            row.append(p)
        out.append(row)
    return out
