"""Variable-length (packed) batches on the GPU against the fp64 oracle.

Each batch row runs only its first ``lengths[b]`` steps (past them its state
is carried and its output is zero); see ``rnn_set_sequence_lengths`` in
``include/rnn.h``.  Lengths include 0 and T.
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

MODES = ("rnn_tanh", "lstm", "gru")
TOL = {"f32": (1e-4, 1e-3), "bf16": (2e-2, 2e-2)}


def _case(mode, L, D, T, B, I, H, wtype, seed):
    return synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=seed, state_std=0.5,
                           with_state_grads=True)


def _lengths(T, B, seed):
    rng = np.random.default_rng(seed)
    n = rng.integers(0, T + 1, size=B)
    n[0], n[1] = T, 0
    if B > 2:
        n[2] = 1
    return [int(v) for v in n]


def _announce(*a):
    print("CASE", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("mode,L,D,wtype", list(itertools.product(MODES, (1, 2), (1, 2), ("f32", "bf16"))))
def test_packed_parity(mode, L, D, wtype):
    T, B, I, H = 9, 19, 37, 40
    lengths = _lengths(T, B, seed=L * 10 + D)
    _announce("packed", mode, L, D, wtype, lengths)
    case = _case(mode, L, D, T, B, I, H, wtype, seed=7)
    g = run_gpu(mode, L, D, case, wtype, lengths=lengths)
    o = run_oracle(mode, L, D, case, lengths=lengths)
    check(compare(g, o, mode, L, D), *TOL[wtype])
    # outputs and input gradients past each row's length are exactly zero
    for b, n in enumerate(lengths):
        assert np.all(g["y"][n:, b] == 0.0)
        assert np.all(g["dx"][n:, b] == 0.0)


@pytest.mark.parametrize("mode", MODES)
def test_packed_wavefront_stack(mode):
    """Unidirectional 3-layer stack (one wavefront launch) with lengths."""
    T, B, I, H = 10, 6, 16, 32
    lengths = [10, 0, 1, 7, 3, 9]
    _announce("packed wavefront", mode, lengths)
    case = _case(mode, 3, 1, T, B, I, H, "f32", seed=4)
    g = run_gpu(mode, 3, 1, case, "f32", lengths=lengths)
    o = run_oracle(mode, 3, 1, case, lengths=lengths)
    check(compare(g, o, mode, 3, 1), *TOL["f32"])


@pytest.mark.parametrize("mode,wtype", list(itertools.product(MODES, ("f32", "bf16"))))
def test_packed_schedules_bitwise_equal_and_full_lengths(mode, wtype):
    """Persistent and stepped schedules agree bitwise with lengths; lengths
    that are all T agree bitwise with no lengths."""
    T, B, I, H = 7, 12, 24, 40
    lengths = _lengths(T, B, seed=3)
    _announce("packed schedules", mode, wtype, lengths)
    case = _case(mode, 2, 2, T, B, I, H, wtype, seed=8)
    a = run_gpu(mode, 2, 2, case, wtype, sched=R.SCHED_PERSISTENT, lengths=lengths)
    b = run_gpu(mode, 2, 2, case, wtype, sched=R.SCHED_STEPPED, lengths=lengths)
    for k in ("y", "hy", "dx", "dh0"):
        assert np.array_equal(a[k], b[k]), k
    full = run_gpu(mode, 2, 2, case, wtype, lengths=[T] * B)
    plain = run_gpu(mode, 2, 2, case, wtype)
    for k in ("y", "hy", "dx", "dh0"):
        assert np.array_equal(full[k], plain[k]), k


def test_changed_lengths_is_bad_call_order():
    h = R.rnn_create("lstm", 1, 1, 8, 16, "f32")
    W = R.pack_weights(h, synth.make_params("lstm", 1, 1, 8, 16, "f32", 2))
    T, B = 5, 3
    x = torch.randn((T, B, 8), device="cuda")
    y = torch.zeros((T, B, 16), device="cuda")
    dx = torch.zeros_like(x)
    ws = torch.empty(R.rnn_workspace_size(h, T, B, 1), dtype=torch.uint8, device="cuda")
    R.rnn_set_sequence_lengths(h, torch.tensor([5, 2, 0], dtype=torch.int32, device="cuda"))
    R.rnn_forward_training(h, T, B, x, None, None, W, y, None, None, ws)
    R.rnn_set_sequence_lengths(h, None)
    with pytest.raises(R.RNNError) as e:
        R.rnn_backward_data(h, T, B, y, y, None, None, W, None, None, dx, None, None, ws)
    assert e.value.status == -4
    torch.cuda.synchronize()
    R.rnn_destroy(h)
