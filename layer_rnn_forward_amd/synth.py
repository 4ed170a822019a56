"""Seeded synthetic inputs for the fused RNN operator.

This module only draws random numbers and rounds them to the working
precision; it holds none of the operator's arithmetic.  Both the GPU tests
and the fp64 oracle are fed from it, so the two sides see bit-identical
values (the oracle receives them widened exactly to fp64).

Workload shapes follow the Deep Speech 2 sizes quoted on the MXNet "fused
RNN operator" page (Performance > LSTM and > GRU: sequence length 300, batch
20, input 800, hidden 800) and its 5-layer bidirectional variants.  No data
set is involved: the inputs are Gaussian stand-ins for speech features.

Draw order (fixed): one ``torch.Generator('cpu')`` per role, seeded
``1000*N + k`` for workload ``N``: ``k = 0`` weights (layer -> direction ->
W_ih, W_hh, b_ih, b_hh, each U(-1/sqrt(H), 1/sqrt(H))), ``k = 1`` x ~ N(0,1),
``k = 2`` h0 then c0, ``k = 3`` dy then dhy then dcy.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

GATES = {"rnn_tanh": 1, "lstm": 4, "gru": 3, "gru_tf": 3, "gru_paper": 3}


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str
    layers: int
    dirs: int
    T: int
    B: int
    input_size: int
    hidden: int
    wtype: str            # "f32" or "bf16" (matrix element type)
    state_std: float      # 0.0 -> h0 = c0 = 0; else N(0, state_std) (std)
    seed_base: int
    init_scale_hidden: int = 0   # U(+-1/sqrt(this)); 0 -> hidden
    notes: str = field(default="")


def _w(name, mode, L, D, T, B, I, H, wtype, std, n, notes=""):
    return Workload(name, mode, L, D, T, B, I, H, wtype, std, 1000 * n, 0, notes)


# The five workloads, numbered 1..5, plus the unidirectional 5-layer stack.
WORKLOADS = {
    "lstm_small_f32": _w("lstm_small_f32", "lstm", 1, 1, 16, 4, 32, 32, "f32", 0.0, 1),
    "lstm_ds2_f32": _w("lstm_ds2_f32", "lstm", 1, 1, 300, 20, 800, 800, "f32", 0.1, 2),
    "lstm_ds2_bf16": _w("lstm_ds2_bf16", "lstm", 1, 1, 300, 20, 800, 800, "bf16", 0.1, 2),
    "gru_ds2_f32": _w("gru_ds2_f32", "gru", 1, 1, 300, 20, 800, 800, "f32", 0.1, 3),
    "lstm_ds2_l5_bi_bf16": _w("lstm_ds2_l5_bi_bf16", "lstm", 5, 2, 300, 20, 800, 800, "bf16", 0.0, 4),
    "gru_ds2_l5_bi_bf16": _w("gru_ds2_l5_bi_bf16", "gru", 5, 2, 300, 20, 800, 800, "bf16", 0.0, 5),
    "tanh_ds2_l5_bi_bf16": _w("tanh_ds2_l5_bi_bf16", "rnn_tanh", 5, 2, 300, 20, 800, 800, "bf16", 0.0, 5),
    "lstm_ds2_l5_uni_bf16": _w("lstm_ds2_l5_uni_bf16", "lstm", 5, 1, 300, 20, 800, 800, "bf16", 0.0, 6),
    # the GRU flavours at the same shape (two exchanges per step)
    "gru_ds2_bf16": _w("gru_ds2_bf16", "gru", 1, 1, 300, 20, 800, 800, "bf16", 0.1, 3),
    "gru_tf_ds2_bf16": _w("gru_tf_ds2_bf16", "gru_tf", 1, 1, 300, 20, 800, 800, "bf16", 0.1, 7),
    "gru_tf_ds2_f32": _w("gru_tf_ds2_f32", "gru_tf", 1, 1, 300, 20, 800, 800, "f32", 0.1, 7),
    "gru_paper_ds2_bf16": _w("gru_paper_ds2_bf16", "gru_paper", 1, 1, 300, 20, 800, 800, "bf16", 0.1, 8),
}


def round_matrix(t: torch.Tensor, wtype: str) -> torch.Tensor:
    """Round an fp64 tensor to the matrix element type (round to nearest
    even), returned widened back to fp64 so that it is exact in either
    precision."""
    if wtype == "bf16":
        return t.to(torch.bfloat16).to(torch.float64)
    if wtype == "f32":
        return t.to(torch.float32).to(torch.float64)
    raise ValueError(wtype)


def make_params(mode, layers, dirs, input_size, hidden, wtype, seed, scale_hidden=None):
    """``params[l][d] = {w_ih, w_hh, b_ih, b_hh}`` as fp64 numpy arrays whose
    values are exactly representable in the working precision (matrices in
    ``wtype``, biases in fp32)."""
    G = GATES[mode]
    g = torch.Generator("cpu").manual_seed(seed)
    k = 1.0 / math.sqrt(scale_hidden or hidden)
    out = []
    for l in range(layers):
        I_l = input_size if l == 0 else dirs * hidden
        row = []
        for _ in range(dirs):
            shapes = {"w_ih": (G * hidden, I_l), "w_hh": (G * hidden, hidden),
                      "b_ih": (G * hidden,), "b_hh": (G * hidden,)}
            p = {}
            for name in ("w_ih", "w_hh", "b_ih", "b_hh"):
                t = torch.empty(shapes[name], dtype=torch.float64).uniform_(-k, k, generator=g)
                t = round_matrix(t, wtype) if name.startswith("w_") else round_matrix(t, "f32")
                p[name] = t.numpy()
            row.append(p)
        out.append(row)
    return out


def make_inputs(mode, layers, dirs, T, B, input_size, hidden, seed_x, seed_state, state_std):
    """``x [T, B, I]``, ``h0``/``c0`` ``[L*D, B, H]`` (``c0`` None unless
    LSTM) as fp64 numpy arrays of fp32-representable values."""
    gx = torch.Generator("cpu").manual_seed(seed_x)
    x = torch.randn((T, B, input_size), dtype=torch.float64, generator=gx)
    x = x.to(torch.float32).to(torch.float64).numpy()
    shape = (layers * dirs, B, hidden)
    if state_std > 0.0:
        gs = torch.Generator("cpu").manual_seed(seed_state)
        h0 = (torch.randn(shape, dtype=torch.float64, generator=gs) * state_std)
        h0 = h0.to(torch.float32).to(torch.float64).numpy()
        c0 = None
        if mode == "lstm":
            c0 = (torch.randn(shape, dtype=torch.float64, generator=gs) * state_std)
            c0 = c0.to(torch.float32).to(torch.float64).numpy()
    else:
        h0 = np.zeros(shape)
        c0 = np.zeros(shape) if mode == "lstm" else None
    return x, h0, c0


def make_grads(mode, layers, dirs, T, B, hidden, seed, with_state_grads=False, std=1.0):
    """Upstream gradients: ``dy [T, B, D*H] ~ N(0,1)``; ``dhy``/``dcy``
    ``[L*D, B, H]`` ~ N(0, std) if ``with_state_grads`` else zeros (``dcy``
    None unless LSTM)."""
    g = torch.Generator("cpu").manual_seed(seed)
    dy = torch.randn((T, B, dirs * hidden), dtype=torch.float64, generator=g)
    dy = dy.to(torch.float32).to(torch.float64).numpy()
    shape = (layers * dirs, B, hidden)
    if with_state_grads:
        dhy = (torch.randn(shape, dtype=torch.float64, generator=g) * std)
        dhy = dhy.to(torch.float32).to(torch.float64).numpy()
        dcy = None
        if mode == "lstm":
            dcy = (torch.randn(shape, dtype=torch.float64, generator=g) * std)
            dcy = dcy.to(torch.float32).to(torch.float64).numpy()
    else:
        dhy = np.zeros(shape)
        dcy = np.zeros(shape) if mode == "lstm" else None
    return dy, dhy, dcy


def make_workload(w: Workload, with_state_grads=False):
    """All inputs of a workload: ``dict(params, x, h0, c0, dy, dhy, dcy)``."""
    params = make_params(w.mode, w.layers, w.dirs, w.input_size, w.hidden, w.wtype,
                         w.seed_base + 0, w.init_scale_hidden or None)
    x, h0, c0 = make_inputs(w.mode, w.layers, w.dirs, w.T, w.B, w.input_size, w.hidden,
                            w.seed_base + 1, w.seed_base + 2, w.state_std)
    dy, dhy, dcy = make_grads(w.mode, w.layers, w.dirs, w.T, w.B, w.hidden,
                              w.seed_base + 3, with_state_grads)
    return dict(params=params, x=x, h0=h0, c0=c0, dy=dy, dhy=dhy, dcy=dcy)


def make_case(mode, layers, dirs, T, B, input_size, hidden, wtype="f32", seed=7,
              state_std=0.5, with_state_grads=True, scale=None):
    """A small ad-hoc case (tests): same draw order as :func:`make_workload`
    with ``seed_base = seed``."""
    params = make_params(mode, layers, dirs, input_size, hidden, wtype, seed, scale)
    x, h0, c0 = make_inputs(mode, layers, dirs, T, B, input_size, hidden, seed + 1,
                            seed + 2, state_std)
    dy, dhy, dcy = make_grads(mode, layers, dirs, T, B, hidden, seed + 3, with_state_grads)
    return dict(params=params, x=x, h0=h0, c0=c0, dy=dy, dhy=dhy, dcy=dcy)
