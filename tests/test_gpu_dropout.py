"""Inter-layer dropout on the GPU against the oracle.

The keep masks are integer decisions (Philox4x32-10 words against an integer
threshold), so the library's mask must equal the oracle's bit for bit; the
training pass and its gradients must match the oracle with the same masks to
the usual floating-point tolerances.
"""

from __future__ import annotations

import itertools
import sys

import numpy as np
import pytest
import torch

import layer_rnn_forward_amd as R
from layer_rnn_forward_amd import synth
from oracle import rnn_oracle as orc
from tests.gpu_harness import check, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-3), "bf16": (2e-2, 2e-2)}


def _case(mode, L, D, T, B, I, H, wtype, seed):
    return synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=seed, state_std=0.5,
                           with_state_grads=True)


def _announce(*a):
    print("CASE", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("T,B,D,H,layer,p,seed", [
    (5, 3, 1, 7, 1, 0.3, 1),                       # 105 elements: a ragged last counter
    (9, 19, 2, 40, 2, 0.5, (0xDEADBEEF << 32) | 17),   # high seed word
    (300, 20, 1, 800, 1, 0.1, 12345),              # a full layer input
    (4, 2, 2, 3, 1, 0.0, 5),
    (4, 2, 2, 3, 1, 1.0, 5),
    (33, 7, 2, 5, 3, 0.77, (1 << 64) - 1),
])
def test_mask_is_bit_exact(T, B, D, H, layer, p, seed):
    _announce("mask", T, B, D, H, layer, p, seed)
    h = R.rnn_create("lstm", layer + 1, D, 8, H)
    R.rnn_set_dropout(h, p, seed)
    n = T * B * D * H
    m = torch.full((n + 5,), 7, dtype=torch.uint8, device="cuda")
    R.rnn_dropout_mask(h, T, B, layer, m[:n])
    torch.cuda.synchronize()
    got = m.cpu().numpy()
    want = orc.dropout_keep(p, seed, layer, (T, B, D * H)).ravel().astype(np.uint8)
    assert np.array_equal(got[:n], want)
    assert np.all(got[n:] == 7)   # nothing past the end
    R.rnn_destroy(h)


@pytest.mark.parametrize("mode,L,D,wtype", list(itertools.product(
    ("rnn_tanh", "lstm", "gru"), (2, 3), (1, 2), ("f32", "bf16"))))
def test_dropout_training_parity(mode, L, D, wtype):
    T, B, I, H = 9, 19, 37, 40
    drop = (0.3, 1000 + 10 * L + D)
    _announce("dropout", mode, L, D, wtype, drop)
    case = _case(mode, L, D, T, B, I, H, wtype, seed=21)
    g = run_gpu(mode, L, D, case, wtype, dropout=drop)
    o = run_oracle(mode, L, D, case, dropout=drop)
    check(compare(g, o, mode, L, D), *TOL[wtype])


@pytest.mark.parametrize("mode", ["gru_tf", "lstm"])
def test_dropout_with_packed_rows_and_flavours(mode):
    T, B, I, H = 8, 11, 24, 32
    lengths = [8, 0, 1, 5, 8, 3, 7, 2, 6, 4, 8]
    drop = (0.45, 99)
    _announce("dropout-packed", mode, drop)
    case = _case(mode, 3, 2, T, B, I, H, "f32", seed=22)
    g = run_gpu(mode, 3, 2, case, "f32", lengths=lengths, dropout=drop)
    o = run_oracle(mode, 3, 2, case, lengths=lengths, dropout=drop)
    check(compare(g, o, mode, 3, 2), *TOL["f32"])


def test_dropout_everything():
    _announce("dropout-p1")
    case = _case("lstm", 2, 2, 6, 5, 10, 16, "f32", seed=23)
    g = run_gpu("lstm", 2, 2, case, "f32", dropout=(1.0, 4))
    o = run_oracle("lstm", 2, 2, case, dropout=(1.0, 4))
    check(compare(g, o, "lstm", 2, 2), *TOL["f32"])


def test_inference_never_drops_and_p0_is_exact():
    _announce("dropout-inference")
    case = _case("gru", 3, 1, 7, 6, 12, 24, "f32", seed=24)
    plain = run_gpu("gru", 3, 1, case, "f32")
    inf = run_gpu("gru", 3, 1, case, "f32", training=False, dropout=(0.6, 8))
    for k in ("y", "hy"):
        assert np.array_equal(inf[k], plain[k])
    zero = run_gpu("gru", 3, 1, case, "f32", dropout=(0.0, 8))
    for k in ("y", "hy", "dx", "dh0"):
        assert np.array_equal(zero[k], plain[k])


def test_backward_uses_the_forward_settings():
    # the setting changes between the training forward and its backward calls
    _announce("dropout-settings")
    mode, L, D, T, B, I, H = "lstm", 2, 1, 6, 4, 10, 16
    case = _case(mode, L, D, T, B, I, H, "f32", seed=25)
    h = R.rnn_create(mode, L, D, I, H, "f32")
    R.rnn_set_dropout(h, 0.3, 31)
    W = R.pack_weights(h, case["params"])
    ws = torch.empty(R.rnn_workspace_size(h, T, B, 1), dtype=torch.uint8, device="cuda")
    dev = lambda a: torch.as_tensor(np.ascontiguousarray(a), dtype=torch.float32, device="cuda")
    x, h0, c0, dy = dev(case["x"]), dev(case["h0"]), dev(case["c0"]), dev(case["dy"])
    y = torch.empty(T, B, D * H, device="cuda")
    R.rnn_forward_training(h, T, B, x, h0, c0, W, y, None, None, ws)
    R.rnn_set_dropout(h, 0.8, 32)
    dx = torch.empty(T, B, I, device="cuda")
    R.rnn_backward_data(h, T, B, y, dy, None, None, W, h0, c0, dx, None, None, ws)
    dW = torch.empty(R.rnn_weights_size(h, 1) // 4, device="cuda")
    R.rnn_backward_weights(h, T, B, x, h0, y, ws, dW)
    torch.cuda.synchronize()
    _, _, _, cache = orc.forward(mode, case["x"], case["params"], h0=case["h0"], c0=case["c0"],
                                 num_dirs=D, keep=True, dropout=0.3, dropout_seed=31)
    odx, _, _, odp = orc.backward(mode, case["params"], cache, case["dy"], num_dirs=D)
    gdp = R.unpack_weights(h, dW, grad=1)
    err = np.max(np.abs(dx.double().cpu().numpy() - odx)) / np.max(np.abs(odx))
    assert err < 1e-3
    e2 = np.max(np.abs(gdp[1][0]["w_ih"] - odp[1][0]["w_ih"])) / np.max(np.abs(odp[1][0]["w_ih"]))
    assert e2 < 1e-3
    R.rnn_destroy(h)


@pytest.mark.parametrize("mode", ["lstm", "rnn_tanh", "gru"])
def test_dropout_in_the_layer_wavefront(mode):
    # unidirectional stacks run all layers in one launch: each layer rings a
    # dropped copy of its h for the layer above; the stepped schedule (one
    # launch per step) must give the same bits
    T, B, I, H = 12, 7, 20, 64
    drop = (0.35, 4242)
    _announce("dropout-wavefront", mode, drop)
    case = _case(mode, 4, 1, T, B, I, H, "f32", seed=26)
    gp = run_gpu(mode, 4, 1, case, "f32", sched=R.SCHED_PERSISTENT, dropout=drop)
    gs = run_gpu(mode, 4, 1, case, "f32", sched=R.SCHED_STEPPED, dropout=drop)
    for k in gp:
        if k != "dW":
            assert np.array_equal(gp[k], gs[k]), k
    o = run_oracle(mode, 4, 1, case, dropout=drop)
    check(compare(gp, o, mode, 4, 1), *TOL["f32"])
