"""One workspace reused across training steps whose inputs and weights change.

The MXNet "fused RNN operator" page (Operator Registration) keeps the
forward intermediates in a reserved workspace that is reused from one
iteration to the next.  Every step here gets different seeded x, h0, c0, W
and upstream gradients, runs forward_training + backward_data +
backward_weights on the SAME workspace, and is compared bitwise with the
same step on a second workspace that is held at the same time (so the
caching allocator cannot hand back the same block) and was filled with a
0xFF byte pattern before use.  A stale ring line, flag or reserve entry
left by the previous step would show as a mismatch.  One step per case is
also checked against the fp64 oracle.  The shapes keep the DS2 grid
(B = 20, hidden 800: the sweeps span every XCD); both workgroup placements
(linear, and XCD-local recurrence groups) are exercised.
"""

import sys

import numpy as np
import pytest
import torch

import layer_rnn_forward_amd as R
from layer_rnn_forward_amd import synth
from tests.gpu_harness import check, compare, run_oracle

pytestmark = pytest.mark.gpu

KEYS = ("y", "hy", "cy", "dx", "dh0", "dc0", "dW")


def _announce(*a):
    print("CASE", *a, flush=True)
    sys.stdout.flush()


def _dev(a):
    if a is None:
        return None
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.float64).float().cuda()


class TrainStep:
    """Device copies of one case's inputs on a handle; run() does a full
    training step on a given workspace and returns device copies of every
    output and gradient."""

    def __init__(self, h, mode, case):
        self.h, self.mode = h, mode
        x = case["x"]
        self.T, self.B, _ = x.shape
        self.x = _dev(x)
        self.h0 = _dev(case["h0"])
        self.c0 = _dev(case["c0"]) if mode == "lstm" else None
        self.W = R.pack_weights(h, case["params"])
        self.dy = _dev(case["dy"])
        self.dhy = _dev(case["dhy"])
        self.dcy = _dev(case["dcy"]) if mode == "lstm" else None
        L, D, H, I = h.L, h.D, h.H, h.I
        self.shapes = {"y": (self.T, self.B, D * H), "hy": (L * D, self.B, H), "dx": (self.T, self.B, I),
                       "dh0": (L * D, self.B, H)}
        if mode == "lstm":
            self.shapes.update(cy=(L * D, self.B, H), dc0=(L * D, self.B, H))

    def run(self, ws):
        h, T, B = self.h, self.T, self.B
        o = {k: torch.full(s, float("nan"), device="cuda") for k, s in self.shapes.items()}
        o["dW"] = torch.full((R.rnn_weights_size(h, 1) // 4,), float("nan"), device="cuda")
        R.rnn_forward_training(h, T, B, self.x, self.h0, self.c0, self.W, o["y"], o["hy"], o.get("cy"), ws)
        R.rnn_backward_data(h, T, B, o["y"], self.dy, self.dhy, self.dcy, self.W, self.h0, self.c0,
                            o["dx"], o["dh0"], o.get("dc0"), ws)
        R.rnn_backward_weights(h, T, B, self.x, self.h0, o["y"], ws, o["dW"])
        return o


def _fresh(nbytes):
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    return ws


def _to_numpy(h, o):
    out = {k: v.double().cpu().numpy() for k, v in o.items() if k != "dW"}
    out["dW"] = R.unpack_weights(h, o["dW"], grad=1)
    return out


def _bitwise(a, b, where):
    # compared as bit patterns: the NaN fill of never-written bytes (the
    # alignment gaps of the packed gradient buffer) must match too
    for k in KEYS:
        if k in a:
            assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), \
                f"{where}: {k} differs between the reused and a fresh workspace"


CASES = [("lstm", 1, 1, 300, 20, 800, 800, "bf16"), ("gru", 2, 2, 40, 20, 800, 800, "bf16"),
         ("gru_tf", 1, 1, 40, 20, 800, 800, "bf16")]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("place", [0, 1])
@pytest.mark.parametrize("mode,L,D,T,B,I,H,wtype", CASES)
def test_workspace_reuse_changing_inputs(monkeypatch, place, mode, L, D, T, B, I, H, wtype):
    monkeypatch.setenv("RNN_PLACE", str(place))
    _announce("workspace_reuse", mode, L, D, T, B, I, H, wtype, "place", place)
    h = R.rnn_create(mode, L, D, I, H, wtype)
    need = R.rnn_workspace_size(h, T, B, 1)
    ws = _fresh(need)   # reused by every step
    for i, seed in enumerate((101, 202, 303)):
        case = synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=seed, state_std=0.3,
                               with_state_grads=True)
        st = TrainStep(h, mode, case)
        a = st.run(ws)
        other = _fresh(need)   # held together with ws: a different block
        b = st.run(other)
        torch.cuda.synchronize()
        assert R.rnn_device_status(h, ws) == 0 and R.rnn_device_status(h, other) == 0
        _bitwise(a, b, f"step {i} (seed {seed})")
        del other
        if i == 1:
            g = _to_numpy(h, a)
            o = run_oracle(mode, L, D, case)
            check(compare(g, o, mode, L, D), 2e-2, 2e-2)
    R.rnn_destroy(h)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("place", [0, 1])
def test_workspace_reuse_soak(monkeypatch, place):
    """50 training steps on one workspace alternating between two input sets
    (different x, states, weights and gradients) at the DS2 LSTM shape; each
    step bitwise equal to its input set's result on a fresh workspace.  Stops
    at the first mismatch."""
    monkeypatch.setenv("RNN_PLACE", str(place))
    mode, L, D, T, B, I, H, wtype = "lstm", 1, 1, 300, 20, 800, 800, "bf16"
    _announce("workspace_soak", "place", place)
    h = R.rnn_create(mode, L, D, I, H, wtype)
    need = R.rnn_workspace_size(h, T, B, 1)
    steps = [TrainStep(h, mode, synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=s,
                                                state_std=0.3, with_state_grads=True))
             for s in (404, 505)]
    ref = []
    for st in steps:
        w = _fresh(need)
        ref.append(st.run(w))
        torch.cuda.synchronize()
        assert R.rnn_device_status(h, w) == 0
        del w
    ws = _fresh(need)
    for i in range(50):
        o = steps[i % 2].run(ws)
        torch.cuda.synchronize()
        assert R.rnn_device_status(h, ws) == 0, f"device timeout at step {i}"
        _bitwise(o, ref[i % 2], f"soak step {i}")
    R.rnn_destroy(h)
