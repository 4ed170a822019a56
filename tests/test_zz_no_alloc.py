"""The inference entry point that allocates nothing (rnn_forward_inference_static:
the library's fixed device array in place of the caller's workspace), for
callers that cannot allocate device memory.  Checked through the C ABI
against rnn_forward_inference on the same inputs -- bitwise, since both run
the same plan and kernels -- on two calls in a row, the second with a
smaller input, and for the size limit."""

import sys

import numpy as np
import pytest
import torch

import layer_rnn_forward_amd as R
from layer_rnn_forward_amd import synth

pytestmark = pytest.mark.gpu


def _dev(a):
    if a is None:
        return None
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.float64).float().cuda()


def _both(h, mode, T, B, seed):
    L, D, I, H = h.L, h.D, h.I, h.H
    case = synth.make_case(mode, L, D, T, B, I, H, wtype=h.wtype, seed=seed, state_std=0.3)
    W = R.pack_weights(h, case["params"])
    x, h0 = _dev(case["x"]), _dev(case["h0"])
    c0 = _dev(case["c0"]) if mode == "lstm" else None
    outs = []
    for static in (True, False):
        y = torch.full((T, B, D * H), float("nan"), device="cuda")
        hy = torch.full((L * D, B, H), float("nan"), device="cuda")
        cy = torch.full((L * D, B, H), float("nan"), device="cuda") if mode == "lstm" else None
        if static:
            R.rnn_forward_inference_static(h, T, B, x, h0, c0, W, y, hy, cy)
        else:
            ws = torch.empty(R.rnn_workspace_size(h, T, B, 0), dtype=torch.uint8, device="cuda")
            R.rnn_forward_inference(h, T, B, x, h0, c0, W, y, hy, cy, ws)
        torch.cuda.synchronize()
        outs.append({"y": y, "hy": hy, "cy": cy})
    return outs


@pytest.mark.parametrize("mode,L,D,wtype", [("lstm", 1, 1, "bf16"), ("gru", 2, 2, "f32"), ("rnn_tanh", 3, 1, "bf16")])
def test_static_inference_matches_workspace_call(mode, L, D, wtype):
    print("CASE static inference", mode, L, D, wtype, flush=True)
    sys.stdout.flush()
    I, H = 800, 800
    h = R.rnn_create(mode, L, D, I, H, wtype)
    # a full-size call, then a smaller one: nothing of the first may leak
    for T, B, seed in ((300, 20, 61), (37, 5, 62)):
        if R.rnn_workspace_size(h, T, B, 0) > R.rnn_static_workspace_bytes():
            T = 60   # the deeper stacks at T = 300 exceed the array; keep B and the grid
        a, b = _both(h, mode, T, B, seed)
        for k in ("y", "hy", "cy"):
            if a[k] is not None:
                assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), (T, B, k)
    R.rnn_destroy(h)


def test_static_inference_rejects_oversize():
    h = R.rnn_create("lstm", 1, 1, 800, 800, "bf16")
    T = 2000   # GX alone is T * B * 4H * 4 bytes = 512 MB
    assert R.rnn_workspace_size(h, T, 20, 0) > R.rnn_static_workspace_bytes()
    x = torch.zeros((T, 20, 800), device="cuda")
    y = torch.zeros((T, 20, 800), device="cuda")
    W = torch.zeros(R.rnn_weights_size(h, 0), dtype=torch.uint8, device="cuda")
    with pytest.raises(R.RNNError) as e:
        R.rnn_forward_inference_static(h, T, 20, x, None, None, W, y, None, None)
    assert e.value.status == -3
    R.rnn_destroy(h)
