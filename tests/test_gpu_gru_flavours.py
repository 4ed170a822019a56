"""The TensorFlow and original-paper GRU flavours on the GPU against the oracle.

Both read the candidate as n = tanh(W_in x + b_in + W_hn (r*h) + b_hn); the
TensorFlow flavour updates h = (1-z) n + z h, the paper's h = (1-z) h + z n
(oneDNN issue #218, "GRU flavours").  Their sweeps run two exchanges per step
and need every workgroup resident at once.
"""

from __future__ import annotations

import itertools
import sys

import numpy as np
import pytest
import torch

import layer_rnn_forward_amd as R
from layer_rnn_forward_amd import synth
from tests.gpu_harness import check, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

FLAVOURS = ("gru_tf", "gru_paper")
TOL = {"f32": (1e-4, 1e-3), "bf16": (2e-2, 2e-2)}


def _case(mode, L, D, T, B, I, H, wtype, seed):
    return synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=seed, state_std=0.5,
                           with_state_grads=True)


def _announce(*a):
    print("CASE", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("mode,L,D,wtype",
                         list(itertools.product(FLAVOURS, (1, 2), (1, 2), ("f32", "bf16"))))
def test_flavour_parity(mode, L, D, wtype):
    # several workgroups and a ragged last slice (H = 40 is not a multiple of
    # the slice width), a ragged batch chunk (B = 19)
    T, B, I, H = 9, 19, 37, 40
    _announce("flavour", mode, L, D, wtype)
    case = _case(mode, L, D, T, B, I, H, wtype, seed=11)
    g = run_gpu(mode, L, D, case, wtype)
    o = run_oracle(mode, L, D, case)
    check(compare(g, o, mode, L, D), *TOL[wtype])


@pytest.mark.parametrize("mode,wtype", list(itertools.product(FLAVOURS, ("f32", "bf16"))))
def test_flavour_wide(mode, wtype):
    # many producer slices per wave, two batch chunks in the backward sweep
    T, B, I, H = 6, 40, 64, 264
    _announce("flavour-wide", mode, wtype)
    case = _case(mode, 1, 2, T, B, I, H, wtype, seed=12)
    g = run_gpu(mode, 1, 2, case, wtype)
    o = run_oracle(mode, 1, 2, case)
    check(compare(g, o, mode, 1, 2), *TOL[wtype])


@pytest.mark.parametrize("mode,D", list(itertools.product(FLAVOURS, (1, 2))))
def test_flavour_packed(mode, D):
    T, B, I, H = 8, 11, 24, 32
    lengths = [8, 0, 1, 5, 8, 3, 7, 2, 6, 4, 8]
    _announce("flavour-packed", mode, D, lengths)
    case = _case(mode, 2, D, T, B, I, H, "f32", seed=13)
    g = run_gpu(mode, 2, D, case, "f32", lengths=lengths)
    o = run_oracle(mode, 2, D, case, lengths=lengths)
    check(compare(g, o, mode, 2, D), *TOL["f32"])
    for b, n in enumerate(lengths):
        assert np.all(g["y"][n:, b] == 0.0)
        assert np.all(g["dx"][n:, b] == 0.0)


@pytest.mark.parametrize("mode", FLAVOURS)
def test_flavour_inference_and_no_state(mode):
    T, B, I, H = 7, 5, 16, 24
    _announce("flavour-inference", mode)
    case = _case(mode, 2, 2, T, B, I, H, "f32", seed=14)
    g = run_gpu(mode, 2, 2, case, "f32", training=False, pass_state=False)
    o = run_oracle(mode, 2, 2, case, backward=False, pass_state=False)
    check(compare(g, o, mode, 2, 2), *TOL["f32"])


@pytest.mark.parametrize("mode", FLAVOURS)
def test_flavour_stepped_schedule_is_refused(mode):
    _announce("flavour-stepped", mode)
    h = R.rnn_create(mode, 1, 1, 8, 16)
    R.rnn_set_schedule(h, R.SCHED_STEPPED)
    T, B = 3, 2
    W = torch.zeros(R.rnn_weights_size(h, 0) // 4, device="cuda")
    ws = torch.empty(R.rnn_workspace_size(h, T, B, 0), dtype=torch.uint8, device="cuda")
    x = torch.zeros(T, B, 8, device="cuda")
    y = torch.empty(T, B, 16, device="cuda")
    with pytest.raises(R.RNNError) as e:
        R.rnn_forward_inference(h, T, B, x, None, None, W, y, None, None, ws)
    assert e.value.status == -5   # RNN_STATUS_NOT_CORESIDENT
    R.rnn_destroy(h)


def test_flavours_differ_from_pytorch_gru():
    # the same weights give different outputs in the three GRU flavours
    T, B, I, H = 5, 4, 8, 16
    _announce("flavour-distinct")
    case = _case("gru", 1, 1, T, B, I, H, "f32", seed=15)
    ys = {m: run_gpu(m, 1, 1, case, "f32", training=False)["y"] for m in ("gru",) + FLAVOURS}
    assert np.max(np.abs(ys["gru"] - ys["gru_tf"])) > 1e-3
    assert np.max(np.abs(ys["gru_tf"] - ys["gru_paper"])) > 1e-3
