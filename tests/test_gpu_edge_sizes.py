"""Edge sizes against the oracle: sequences of thousands of steps (the
exchange rings and flag values grow with T) and batches of hundreds of rows
(many recurrence groups; grids too large to be co-resident take the stepped
schedule automatically).  Full training passes, every output and gradient
compared element by element."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import layer_rnn_forward_amd as R  # noqa: E402
from layer_rnn_forward_amd import synth  # noqa: E402
from tests.gpu_harness import check, compare, run_gpu, run_oracle  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-3), "bf16": (2e-2, 2e-2)}

# (mode, weights, L, D, T, B, I, H, persistent sweeps expected)
CASES = [
    ("lstm", "bf16", 1, 1, 4096, 2, 16, 64, True),
    ("gru", "f32", 2, 2, 2000, 3, 8, 32, True),
    ("rnn_tanh", "bf16", 1, 2, 3000, 1, 4, 128, True),
    ("gru_tf", "bf16", 1, 1, 1500, 4, 16, 96, True),
    ("lstm", "bf16", 1, 1, 20, 512, 64, 256, True),
    ("gru", "bf16", 1, 2, 12, 1024, 32, 128, False),
    ("lstm", "f32", 2, 1, 10, 300, 100, 512, False),
]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_edge_size(k):
    mode, wtype, L, D, T, B, I, H, persistent = CASES[k]
    print("edge case", k, mode, wtype, L, D, T, B, I, H, flush=True)
    h = R.rnn_create(mode, L, D, I, H, wtype)
    plan = R.rnn_plan_info(h, T, B, True)
    R.rnn_destroy(h)
    print("plan", plan, flush=True)
    # the automatic schedule: persistent when the grid fits, stepped otherwise
    assert bool(plan["fwd"]["persistent"]) == persistent
    case = synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=9100 + k)
    g = run_gpu(mode, L, D, case, wtype)
    o = run_oracle(mode, L, D, case)
    check(compare(g, o, mode, L, D), *TOL[wtype])
