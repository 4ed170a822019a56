"""Cases of the ordering-perturbation check (not collected by pytest).

Each case runs a full training step (forward filling the reserve, backward
through time, weight gradients) or an inference pass through the C ABI and
returns every output as a flat dict of float64 arrays.  The GPU test runs
the cases in its own process with the normal library and in a child process
(``python tests/perturb_cases.py OUT.npz`` with ``RNN_LIB`` set to the
perturbed build) and requires bitwise-equal results: the perturbed build
only inserts pauses at the exchange's waits and flag publications, so any
difference is an ordering fault.  The shapes span every XCD (the DS2 hidden
width of 800 gives 50-100 workgroups per group) and each placement and
exchange kind: linear and line-sharing runs, XCD-local groups (tanh), the
two-exchange GRU flavours, the layer wavefront with dropout, packed rows,
several batch chunks, a one-row serving batch and the stepped schedule.
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from layer_rnn_forward_amd import synth  # noqa: E402

# (name, mode, L, D, T, B, I, H, wtype, extra options of run_gpu)
CASES = [
    ("lstm_bi_bf16", "lstm", 2, 2, 16, 20, 96, 800, "bf16", {}),
    ("gru_packed_f32", "gru", 1, 1, 12, 7, 64, 256, "f32", {"lengths": [12, 0, 5, 12, 1, 9, 3]}),
    ("tanh_xcd_local_bf16", "rnn_tanh", 2, 2, 12, 20, 64, 800, "bf16", {}),
    ("gru_tf_bi_bf16", "gru_tf", 1, 2, 12, 20, 64, 800, "bf16", {}),
    ("lstm_wavefront_dropout_bf16", "lstm", 3, 1, 12, 20, 64, 800, "bf16", {"dropout": (0.3, 5)}),
    ("lstm_serving_b1_bf16", "lstm", 1, 1, 24, 1, 64, 800, "bf16", {"training": False}),
    ("gru_multichunk_f32", "gru", 2, 2, 8, 70, 37, 256, "f32", {}),
    ("gru_paper_packed_bf16", "gru_paper", 2, 1, 10, 13, 64, 384, "bf16", {"lengths": [10, 3, 0, 7, 10, 1, 9, 10, 2, 5, 8, 10, 4]}),
    ("tanh_wavefront_f32", "rnn_tanh", 3, 1, 12, 5, 16, 512, "f32", {}),
    ("lstm_stepped_bf16", "lstm", 1, 2, 10, 20, 64, 800, "bf16", {"sched": 2}),
]


def _flatten(prefix, v, out):
    if isinstance(v, dict):
        for k, x in v.items():
            _flatten(f"{prefix}.{k}", x, out)
    elif isinstance(v, (list, tuple)):
        for i, x in enumerate(v):
            _flatten(f"{prefix}.{i}", x, out)
    else:
        out[prefix] = np.asarray(v, dtype=np.float64)


def run_all():
    from tests.gpu_harness import run_gpu

    out = {}
    for k, (name, mode, L, D, T, B, I, H, wtype, opts) in enumerate(CASES):
        print("perturb case", name, flush=True)
        case = synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=300 + 10 * k)
        _flatten(name, run_gpu(mode, L, D, case, wtype, **opts), out)
    return out


def forward_sweep_us_per_step(T=64):
    """Per-step time of the recurrent forward sweep (DS2 LSTM width, bf16,
    inference, median of 5 launches): evidence that the pauses of the
    perturbed build actually happen (not compared bitwise)."""
    import torch

    import layer_rnn_forward_amd as R
    from tests.gpu_harness import to_dev

    B, I, H = 20, 64, 800
    case = synth.make_case("lstm", 1, 1, T, B, I, H, wtype="bf16", seed=399)
    h = R.rnn_create("lstm", 1, 1, I, H, "bf16")
    W = R.pack_weights(h, case["params"])
    ws = torch.empty(R.rnn_workspace_size(h, T, B, 0), dtype=torch.uint8, device="cuda")
    x, h0, c0 = to_dev(case["x"]), to_dev(case["h0"]), to_dev(case["c0"])
    y = torch.empty((T, B, H), device="cuda")
    hy, cy = torch.empty((1, B, H), device="cuda"), torch.empty((1, B, H), device="cuda")
    times = []
    for _ in range(6):
        R.rnn_set_profiling(h, True)
        R.rnn_forward_inference(h, T, B, x, h0, c0, W, y, hy, cy, ws)
        n, ms = R.rnn_profile_read(h, 1)
        times.append(1000.0 * ms / max(n, 1) / T)
    R.rnn_set_profiling(h, False)
    R.rnn_destroy(h)
    return float(np.median(times[1:]))


if __name__ == "__main__":
    import layer_rnn_forward_amd as R

    print("library", R.lib_path(), flush=True)
    res = run_all()
    np.savez(sys.argv[1], **res)
    print("forward sweep us/step", forward_sweep_us_per_step(), flush=True)
