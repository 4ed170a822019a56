"""GPU (HIP path, through the C ABI) vs the fp64 oracle, element by element.

Tolerances (normwise max relative error per output tensor, ||g - o||_inf /
||o||_inf): fp32 path 1e-4 on y/hy/cy and 1e-3 on every gradient; bf16-weight
path (bf16 matrices and bf16-rounded MFMA operands, fp32 accumulation and
state) 2e-2.
"""

import itertools
import sys

import numpy as np
import pytest
import torch

import layer_rnn_forward_amd as R
from layer_rnn_forward_amd import synth
from tests.gpu_harness import check, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-3), "bf16": (2e-2, 2e-2)}
MODES = ("rnn_tanh", "lstm", "gru")


def _case(mode, L, D, T, B, I, H, wtype, seed=11, scale=None):
    return synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=seed, state_std=0.5,
                           with_state_grads=True, scale=scale)


def _announce(*a):
    print("CASE", *a, flush=True)
    sys.stdout.flush()


def test_small_lstm_workload():
    """The T=16 B=4 I=H=32 fp32 LSTM workload, full training sequence."""
    w = synth.WORKLOADS["lstm_small_f32"]
    _announce(w)
    case = synth.make_workload(w, with_state_grads=True)
    g = run_gpu("lstm", 1, 1, case, "f32")
    o = run_oracle("lstm", 1, 1, case)
    errs = compare(g, o, "lstm", 1, 1)
    print(errs)
    check(errs, *TOL["f32"])


@pytest.mark.parametrize("mode,L,D,wtype", list(itertools.product(MODES, (1, 2), (1, 2), ("f32", "bf16"))))
def test_ragged_parity(mode, L, D, wtype):
    """Ragged sizes: H not a multiple of the MFMA chunk, odd input width,
    batch not a multiple of 16, several tiles of the time-parallel GEMMs."""
    T, B, I, H = 9, 19, 37, 40
    _announce(mode, L, D, wtype, T, B, I, H)
    case = _case(mode, L, D, T, B, I, H, wtype)
    g = run_gpu(mode, L, D, case, wtype)
    o = run_oracle(mode, L, D, case)
    errs = compare(g, o, mode, L, D)
    check(errs, *TOL[wtype])


@pytest.mark.parametrize("mode,wtype", list(itertools.product(MODES, ("f32", "bf16"))))
def test_multi_chunk_batch(mode, wtype):
    """B > 32 splits the batch into independent recurrence groups."""
    T, B, I, H = 6, 45, 24, 48
    _announce(mode, wtype, T, B, I, H)
    case = _case(mode, 2, 2, T, B, I, H, wtype, seed=5)
    g = run_gpu(mode, 2, 2, case, wtype)
    o = run_oracle(mode, 2, 2, case)
    check(compare(g, o, mode, 2, 2), *TOL[wtype])


@pytest.mark.parametrize("mode", MODES)
def test_wavefront_stack(mode):
    """Unidirectional 3-layer stack (layer wavefront in one launch)."""
    T, B, I, H = 12, 7, 20, 64
    _announce(mode, T, B, I, H)
    case = _case(mode, 3, 1, T, B, I, H, "f32", seed=9)
    g = run_gpu(mode, 3, 1, case, "f32")
    o = run_oracle(mode, 3, 1, case)
    check(compare(g, o, mode, 3, 1), *TOL["f32"])


@pytest.mark.parametrize("mode,wtype", list(itertools.product(MODES, ("f32", "bf16"))))
def test_schedules_bitwise_equal(mode, wtype):
    """Persistent and stepped schedules give bitwise identical results, and
    inference equals the training forward bitwise."""
    T, B, I, H = 8, 10, 16, 48
    _announce(mode, wtype)
    case = _case(mode, 2, 2, T, B, I, H, wtype, seed=3)
    a = run_gpu(mode, 2, 2, case, wtype, sched=R.SCHED_PERSISTENT)
    b = run_gpu(mode, 2, 2, case, wtype, sched=R.SCHED_STEPPED)
    c = run_gpu(mode, 2, 2, case, wtype, sched=R.SCHED_PERSISTENT, training=False)
    for k in ("y", "hy", "dx", "dh0"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("y", "hy"):
        assert np.array_equal(a[k], c[k]), k
    for l in range(2):
        for d in range(2):
            for n in a["dW"][l][d]:
                assert np.array_equal(a["dW"][l][d][n], b["dW"][l][d][n]), (l, d, n)


@pytest.mark.parametrize("mode", MODES)
def test_run_to_run_deterministic(mode):
    T, B, I, H = 10, 20, 32, 64
    case = _case(mode, 1, 2, T, B, I, H, "bf16", seed=4)
    a = run_gpu(mode, 1, 2, case, "bf16")
    b = run_gpu(mode, 1, 2, case, "bf16")
    for k in a:
        if k != "dW":
            assert np.array_equal(a[k], b[k]), k
    for d in range(2):
        for n in a["dW"][0][d]:
            assert np.array_equal(a["dW"][0][d][n], b["dW"][0][d][n]), (d, n)


@pytest.mark.parametrize("mode", MODES)
def test_null_states_and_grads(mode):
    """h0/c0 = NULL means zeros, dhy/dcy = NULL means zeros."""
    T, B, I, H = 5, 3, 8, 16
    case = _case(mode, 2, 2, T, B, I, H, "f32", seed=12)
    g = run_gpu(mode, 2, 2, case, "f32", pass_state=False, pass_grads=False)
    o = run_oracle(mode, 2, 2, case, pass_state=False, pass_grads=False)
    check(compare(g, o, mode, 2, 2), *TOL["f32"])


@pytest.mark.parametrize("mode", MODES)
def test_single_step_single_row(mode):
    T, B, I, H = 1, 1, 3, 5
    case = _case(mode, 2, 2, T, B, I, H, "f32", seed=13)
    g = run_gpu(mode, 2, 2, case, "f32")
    o = run_oracle(mode, 2, 2, case)
    check(compare(g, o, mode, 2, 2), *TOL["f32"])


@pytest.mark.parametrize("mode", MODES)
def test_empty_sequence_and_batch(mode):
    """T = 0: hy = h0, y empty; backward: dh0 = dhy, dW = 0.  B = 0: nothing."""
    H, I, L, D = 8, 4, 2, 2
    h = R.rnn_create(mode, L, D, I, H, "f32")
    W = R.pack_weights(h, synth.make_params(mode, L, D, I, H, "f32", 1))
    for T, B in ((0, 3), (4, 0), (0, 0)):
        ws = torch.empty(max(R.rnn_workspace_size(h, T, B, 1), 256), dtype=torch.uint8, device="cuda")
        x = torch.zeros((T, B, I), device="cuda")
        h0 = torch.randn((L * D, B, H), device="cuda")
        c0 = torch.randn((L * D, B, H), device="cuda") if mode == "lstm" else None
        y = torch.zeros((T, B, D * H), device="cuda")
        hy = torch.full((L * D, B, H), float("nan"), device="cuda")
        cy = torch.full((L * D, B, H), float("nan"), device="cuda") if mode == "lstm" else None
        R.rnn_forward_training(h, T, B, x, h0, c0, W, y, hy, cy, ws)
        torch.cuda.synchronize()
        if T == 0:
            assert torch.equal(hy, h0)
            if mode == "lstm":
                assert torch.equal(cy, c0)
        dhy = torch.randn((L * D, B, H), device="cuda")
        dh0 = torch.full((L * D, B, H), float("nan"), device="cuda")
        dx = torch.zeros((T, B, I), device="cuda")
        R.rnn_backward_data(h, T, B, y, torch.zeros_like(y), dhy, None, W, h0, c0, dx, dh0, None, ws)
        dW = torch.full((R.rnn_weights_size(h, 1) // 4,), float("nan"), device="cuda")
        R.rnn_backward_weights(h, T, B, x, h0, y, ws, dW)
        torch.cuda.synchronize()
        if T == 0:
            assert torch.equal(dh0, dhy)
        assert torch.count_nonzero(dW) == 0
    R.rnn_destroy(h)


def test_call_order_and_workspace_errors():
    h = R.rnn_create("lstm", 1, 1, 8, 16, "f32")
    W = R.pack_weights(h, synth.make_params("lstm", 1, 1, 8, 16, "f32", 2))
    T, B = 4, 2
    x = torch.randn((T, B, 8), device="cuda")
    y = torch.zeros((T, B, 16), device="cuda")
    need = R.rnn_workspace_size(h, T, B, 1)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(R.RNNError) as e:
        R.rnn_forward_training(h, T, B, x, None, None, W, y, None, None, small)
    assert e.value.status == -3
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dx = torch.zeros_like(x)
    with pytest.raises(R.RNNError) as e:
        R.rnn_backward_data(h, T, B, y, y, None, None, W, None, None, dx, None, None, ws)
    assert e.value.status == -4
    R.rnn_forward_training(h, T, B, x, None, None, W, y, None, None, ws)
    dW = torch.zeros((R.rnn_weights_size(h, 1) // 4,), device="cuda")
    with pytest.raises(R.RNNError) as e:
        R.rnn_backward_weights(h, T, B, x, None, y, ws, dW)
    assert e.value.status == -4
    with pytest.raises(R.RNNError) as e:   # different T than the forward
        R.rnn_backward_data(h, T - 1, B, y, y, None, None, W, None, None, dx, None, None, ws)
    assert e.value.status == -4
    R.rnn_backward_data(h, T, B, y, y, None, None, W, None, None, dx, None, None, ws)
    R.rnn_backward_weights(h, T, B, x, None, y, ws, dW)
    torch.cuda.synchronize()
    R.rnn_destroy(h)


def test_forced_wait_timeout_is_reported():
    """A spin limit of 0 forced from the host makes every bounded wait of the
    persistent kernel expire at once; every workgroup exits and the status
    call reports the timeout (no hang, no fault)."""
    import os
    import subprocess
    code = (
        "import torch, layer_rnn_forward_amd as R\n"
        "from layer_rnn_forward_amd import synth\n"
        "h = R.rnn_create('lstm', 1, 1, 16, 64, 'f32')\n"
        "R.rnn_set_schedule(h, R.SCHED_PERSISTENT)\n"
        "W = R.pack_weights(h, synth.make_params('lstm', 1, 1, 16, 64, 'f32', 1))\n"
        "T, B = 50, 4\n"
        "ws = torch.empty(R.rnn_workspace_size(h, T, B, 0), dtype=torch.uint8, device='cuda')\n"
        "x = torch.randn((T, B, 16), device='cuda'); y = torch.zeros((T, B, 64), device='cuda')\n"
        "R.rnn_forward_inference(h, T, B, x, None, None, W, y, None, None, ws)\n"
        "print('STATUS', R.rnn_device_status(h, ws))\n"
    )
    env = dict(os.environ, RNN_SPIN_LIMIT="0")   # every wait expires at its first poll
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=120, cwd=str(__import__("pathlib").Path(__file__).parents[1]))
    assert r.returncode == 0, r.stderr
    assert "STATUS -7" in r.stdout, r.stdout


@pytest.mark.parametrize("mode,L,D,wtype", [("lstm", 1, 1, "bf16"), ("gru", 1, 2, "f32"),
                                            ("rnn_tanh", 3, 1, "bf16"), ("lstm", 2, 2, "f32")])
def test_exchange_floor_probe(mode, L, D, wtype):
    """rnn_exchange_floor runs the forward sweep's launch with its exchange
    only: it completes without a device timeout, touches nothing but the
    workspace, and a forward pass on the same workspace afterwards gives
    bitwise the same outputs as before it."""
    T, B, I, H = 12, 6, 24, 40
    _announce("exchange_floor", mode, L, D, wtype)
    case = _case(mode, L, D, T, B, I, H, wtype, seed=21)
    h = R.rnn_create(mode, L, D, I, H, wtype)
    W = R.pack_weights(h, case["params"])
    need = R.rnn_workspace_size(h, T, B, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    x = torch.as_tensor(case["x"], dtype=torch.float64).float().cuda()
    y1 = torch.zeros((T, B, D * H), device="cuda")
    y2 = torch.full((T, B, D * H), 7.0, device="cuda")
    R.rnn_forward_inference(h, T, B, x, None, None, W, y1, None, None, ws)
    R.rnn_exchange_floor(h, T, B, ws)
    assert R.rnn_device_status(h, ws) == 0
    R.rnn_forward_inference(h, T, B, x, None, None, W, y2, None, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(R.RNNError) as e:
        R.rnn_exchange_floor(h, T, B, small)
    assert e.value.status == -3
    # the training pass's plan, on a training workspace
    wst = torch.empty(R.rnn_workspace_size(h, T, B, 1), dtype=torch.uint8, device="cuda")
    R.rnn_exchange_floor(h, T, B, wst, training=True)
    assert R.rnn_device_status(h, wst) == 0
    R.rnn_destroy(h)


@pytest.mark.parametrize("mode,B", list(itertools.product(MODES, (1, 2, 4))))
def test_serving_batches(mode, B):
    """Serving-size batches (1, 2, 4 rows) at the full hidden width of the
    DS2 shape, bf16 weights, both directions."""
    T, I, H = 24, 64, 800
    _announce("serving", mode, B)
    case = _case(mode, 1, 2, T, B, I, H, "bf16", seed=31)
    g = run_gpu(mode, 1, 2, case, "bf16")
    o = run_oracle(mode, 1, 2, case)
    check(compare(g, o, mode, 1, 2), *TOL["bf16"])


@pytest.mark.parametrize("mode,L,D,wtype,split", [("lstm", 1, 1, "f32", 3), ("gru", 1, 2, "bf16", 3),
                                                  ("lstm", 2, 1, "bf16", 2), ("rnn_tanh", 1, 2, "f32", 8)])
def test_forced_split_k(monkeypatch, mode, L, D, wtype, split):
    """Split-K of the data- and weight-gradient products (fp32 partials
    summed in split order by a second kernel), forced at a ragged shape:
    T*B = 820 gives three K splits whose last is short, D*G*H = 544..1632
    gives two or three for the data gradient, and no dimension is a whole
    number of 128-wide tiles.  The factor is clamped to 256 k per split."""
    monkeypatch.setenv("RNN_DW_SPLIT", str(split))
    T, B, I, H = 41, 20, 72, 136
    _announce("forced_split_k", mode, L, D, wtype, split)
    case = _case(mode, L, D, T, B, I, H, wtype, seed=43)
    g = run_gpu(mode, L, D, case, wtype)
    o = run_oracle(mode, L, D, case)
    check(compare(g, o, mode, L, D), *TOL[wtype])


@pytest.mark.parametrize("kind,A,K", [("bf16_16x16x32", 32, 32), ("f32_16x16x4", 32, 16),
                                      ("bf16_32x32x16", 128, 16)])
def test_mfma_peak_probe_is_exact(kind, A, K):
    """The throughput probe behind the measured MFMA peak does all its work:
    every thread's sum of its A accumulators is exactly A * iters * K / 512
    (power-of-two operands, K products per round and chain)."""
    _announce("mfma_peak_probe", kind)
    blocks, iters = 64, 1000
    out = torch.full((blocks * 256,), float("nan"), device="cuda")
    R.rnn_mfma_peak_probe(kind, blocks, iters, out)
    torch.cuda.synchronize()
    assert torch.all(out == A * iters * K / 512.0)
    with pytest.raises(R.RNNError):
        R.rnn_mfma_peak_probe(kind, 0, iters, out)


@pytest.mark.parametrize("mode,D,wtype", list(itertools.product(MODES, (1, 2), ("bf16",))))
def test_xcd_local_groups(monkeypatch, mode, D, wtype):
    """XCD-local recurrence groups (every group's workgroups on one XCD,
    wider per-workgroup unit slices) at the DS2 hidden width and batch:
    the plan takes that placement for both sweeps, and the results match
    the oracle."""
    monkeypatch.setenv("RNN_PLACE", "1")
    T, B, I, H = 24, 20, 96, 800
    _announce("xcd_local", mode, D, wtype, T, B, I, H)
    h = R.rnn_create(mode, 1, D, I, H, wtype)
    info = R.rnn_plan_info(h, T, B, True)
    R.rnn_destroy(h)
    print(info, flush=True)
    assert info["fwd"]["place"] == 1 and info["bwd"]["place"] == 1, info
    assert info["fwd"]["persistent"] == 1 and info["bwd"]["persistent"] == 1, info
    case = _case(mode, 1, D, T, B, I, H, wtype, seed=51)
    g = run_gpu(mode, 1, D, case, wtype)
    o = run_oracle(mode, 1, D, case)
    check(compare(g, o, mode, 1, D), *TOL[wtype])


def _runs(units):
    # run placement: consecutive slices whose units fill one 128-byte line of fp32
    return 32 // units if units < 32 and 32 % units == 0 else 0


def test_default_placement(monkeypatch):
    """With no placement asked for, the bf16 tanh RNN takes XCD-local groups
    (persistent sweeps); the gated cells and fp32 weights take runs of
    line-sharing slices per XCD in the forward (not the two-exchange GRU
    flavours) and, for the LSTM, in the backward, the linear placement in
    the other backward sweeps; a stepped schedule keeps the plan's units on
    a linear grid."""
    monkeypatch.delenv("RNN_PLACE", raising=False)
    T, B, H = 300, 20, 800
    for mode, wtype, want in (("rnn_tanh", "bf16", 1), ("rnn_tanh", "f32", 0), ("lstm", "bf16", 0),
                              ("gru", "bf16", 0), ("gru_tf", "bf16", 0)):
        h = R.rnn_create(mode, 1, 1, H, H, wtype)
        info = R.rnn_plan_info(h, T, B, True)
        want_fwd = want or (0 if mode == "gru_tf" else _runs(info["fwd"]["units"]))
        want_bwd = want or (_runs(info["bwd"]["units"]) if mode == "lstm" else 0)
        assert info["fwd"]["place"] == want_fwd and info["bwd"]["place"] == want_bwd, (mode, wtype, info)
        if want_fwd >= 2:
            assert info["fwd"]["grid"] % (8 * want_fwd) == 0, info
            assert info["fwd"]["grid"] >= info["fwd"]["nwg"] * info["fwd"]["groups"], info
        if want:
            R.rnn_set_schedule(h, R.SCHED_STEPPED)
            st = R.rnn_plan_info(h, T, B, True)
            for k in ("fwd", "bwd"):
                assert st[k]["place"] == 0 and st[k]["persistent"] == 0, st
                assert (st[k]["units"], st[k]["nchunk"]) == (info[k]["units"], info[k]["nchunk"]), (st, info)
                assert st[k]["grid"] == st[k]["nwg"] * st[k]["groups"], st
        R.rnn_destroy(h)


@pytest.mark.parametrize("mode,D,wtype", list(itertools.product(MODES, (1, 2), ("bf16", "f32"))))
def test_line_run_placement(monkeypatch, mode, D, wtype):
    """Runs of line-sharing slices per XCD in both sweeps (RNN_PLACE=2; the
    forward's default) at the DS2 hidden width: the plan takes them, the
    padded grid's idle slots exit, and the results match the oracle."""
    monkeypatch.setenv("RNN_PLACE", "2")
    T, B, I, H = 24, 20, 96, 800
    _announce("line_runs", mode, D, wtype, T, B, I, H)
    h = R.rnn_create(mode, 1, D, I, H, wtype)
    info = R.rnn_plan_info(h, T, B, True)
    R.rnn_destroy(h)
    print(info, flush=True)
    for k in ("fwd", "bwd"):
        assert info[k]["place"] == _runs(info[k]["units"]), info
    assert info["fwd"]["place"] >= 2 or info["bwd"]["place"] >= 2, info
    case = _case(mode, 1, D, T, B, I, H, wtype, seed=53)
    g = run_gpu(mode, 1, D, case, wtype)
    o = run_oracle(mode, 1, D, case)
    check(compare(g, o, mode, 1, D), *TOL[wtype])


@pytest.mark.parametrize("mode,L,D,wtype,H", [
    ("lstm", 1, 1, "bf16", 2048), ("gru", 1, 2, "f32", 1024), ("rnn_tanh", 2, 2, "bf16", 2048),
    ("gru_tf", 1, 1, "bf16", 2048), ("lstm", 3, 1, "bf16", 2048), ("gru", 3, 1, "f32", 1024)])
def test_maximum_hidden_size(mode, L, D, wtype, H):
    """The largest hidden size supported for every shape (1024 with fp32
    weights, 2048 with bf16), training end to end against the oracle; the
    unidirectional stacks at that size are too wide for the layer wavefront
    (each layer would hold W_ih and W_hh) and run one launch per layer."""
    T, B, I = 5, 3, 64
    _announce("max_hidden", mode, L, D, wtype, T, B, I, H)
    h = R.rnn_create(mode, L, D, I, H, wtype)
    info = R.rnn_plan_info(h, T, B, True)
    R.rnn_destroy(h)
    print(info, flush=True)
    if D == 1 and L > 1:
        assert info["fwd"]["groups"] == info["fwd"]["nchunk"], info   # no wavefront
    case = _case(mode, L, D, T, B, I, H, wtype, seed=57)
    g = run_gpu(mode, L, D, case, wtype)
    o = run_oracle(mode, L, D, case)
    check(compare(g, o, mode, L, D), *TOL[wtype])


def test_wavefront_at_moderate_width():
    """Below that width the unidirectional stack keeps the layer wavefront
    (every layer's groups in one launch)."""
    h = R.rnn_create("lstm", 3, 1, 64, 512, "bf16")
    info = R.rnn_plan_info(h, 5, 3, True)
    R.rnn_destroy(h)
    assert info["fwd"]["groups"] == 3 * info["fwd"]["nchunk"], info


def test_bf16_rounding_is_round_to_nearest_even():
    """Every fp32 bit pattern (all 2^32): the library's fp32 -> bf16 rounding
    (the hardware conversion) equals round-to-nearest-even written out on
    the bits, and NaNs stay NaNs; a sub-range adds up the same way."""
    import torch

    m = torch.zeros(1, dtype=torch.int64, device="cuda")
    R.rnn_bf16_rounding_check(0, 1 << 32, m)
    torch.cuda.synchronize()
    assert int(m.item()) == 0
    R.rnn_bf16_rounding_check((1 << 32) - 1000, 1000, m)
    torch.cuda.synchronize()
    assert int(m.item()) == 0
    with pytest.raises(R.RNNError):
        R.rnn_bf16_rounding_check((1 << 32) - 10, 11, m)


@pytest.mark.parametrize("wtype", ["f32", "bf16"])
def test_weights_at_unaligned_offset(wtype):
    """W may sit at any 4-byte offset of a caller's parameter arena: with the
    packed buffer 4 bytes past a 16-byte boundary the products must not take
    their 16-byte vector loads of W_ih, and the results match the oracle."""
    mode, L, D, T, B, I, H = "lstm", 2, 1, 9, 5, 64, 48
    _announce("unaligned W", wtype)
    case = _case(mode, L, D, T, B, I, H, wtype, seed=71)
    h = R.rnn_create(mode, L, D, I, H, wtype)
    packed = R.pack_weights(h, case["params"])
    arena = torch.zeros(packed.numel() + 64, dtype=torch.uint8, device="cuda")
    W = arena[4:4 + packed.numel()]
    W.copy_(packed)
    assert W.data_ptr() % 16 == 4
    xd = torch.as_tensor(case["x"]).float().cuda()
    h0 = torch.as_tensor(case["h0"]).float().cuda()
    c0 = torch.as_tensor(case["c0"]).float().cuda()
    y = torch.full((T, B, D * H), float("nan"), device="cuda")
    hy = torch.full((L * D, B, H), float("nan"), device="cuda")
    cy = torch.full((L * D, B, H), float("nan"), device="cuda")
    ws = torch.empty(R.rnn_workspace_size(h, T, B, 1), dtype=torch.uint8, device="cuda")
    R.rnn_forward_training(h, T, B, xd, h0, c0, W, y, hy, cy, ws)
    dy = torch.as_tensor(case["dy"]).float().cuda()
    dx = torch.full((T, B, I), float("nan"), device="cuda")
    dh0 = torch.full((L * D, B, H), float("nan"), device="cuda")
    dc0 = torch.full((L * D, B, H), float("nan"), device="cuda")
    R.rnn_backward_data(h, T, B, y, dy, None, None, W, h0, c0, dx, dh0, dc0, ws)
    dW = torch.full((R.rnn_weights_size(h, 1) // 4,), float("nan"), device="cuda")
    R.rnn_backward_weights(h, T, B, xd, h0, y, ws, dW)
    torch.cuda.synchronize()
    assert R.rnn_device_status(h, ws) == 0
    g = {"y": y.double().cpu().numpy(), "hy": hy.double().cpu().numpy(), "cy": cy.double().cpu().numpy(),
         "dx": dx.double().cpu().numpy(), "dh0": dh0.double().cpu().numpy(), "dc0": dc0.double().cpu().numpy(),
         "dW": R.unpack_weights(h, dW, grad=1)}
    R.rnn_destroy(h)
    o = run_oracle(mode, L, D, dict(case, dhy=None, dcy=None), pass_grads=False)
    check(compare(g, o, mode, L, D), *TOL[wtype])
