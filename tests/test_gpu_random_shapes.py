"""Randomised shapes against the oracle: every mode in turn, 1-3 layers, one or two
directions, batches 1-70, input widths 1-2048, hidden widths 8-1536, with
packed rows and inter-layer dropout mixed in, drawn from a fixed seed.  A
second set mixes in what the first keeps fixed: inference passes, the
stepped schedule, calls without initial state, up to four layers and
sequences of up to 64 steps.

Shapes whose input fan-in dwarfs the hidden width (I > 16 H) are drawn again:
with weights ~ U(+-1/sqrt(H)) their pre-activations reach a standard
deviation of ~9 and the bf16 rounding of x alone moves the oracle past the
2e-2 bound (a property of bf16 inputs, not of the kernels); fp32 weights are
drawn with H <= 1024, the largest hidden width every fp32 shape supports."""

import os
import random
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from layer_rnn_forward_amd import synth  # noqa: E402
from tests.gpu_harness import check, compare, run_gpu, run_oracle  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-3), "bf16": (2e-2, 2e-2)}


MODES = ["rnn_tanh", "lstm", "gru", "gru_tf", "gru_paper"]


def _draw(rng, mode):
    while True:
        wtype = rng.choice(["f32", "bf16"])
        L, D = rng.choice([1, 1, 2, 3]), rng.choice([1, 2])
        T = rng.randint(1, 16)
        B = rng.choice([1, 2, 3, 5, 8, 13, 20, 33, 64, 70])
        H = rng.choice([8, 24, 40, 64, 100, 128, 200, 256, 384, 512, 800, 1024, 1536])
        I = rng.choice([1, 3, 16, 37, 64, 200, 512, 800, 2048])
        if I > 16 * H or (wtype == "f32" and H > 1024):
            continue
        lengths = [rng.randint(0, T) for _ in range(B)] if rng.random() < 0.25 else None
        drop = (0.25, rng.randint(1, 99)) if L > 1 and rng.random() < 0.25 else None
        return mode, wtype, L, D, T, B, I, H, lengths, drop


_rng = random.Random(20261203)
CASES = [_draw(_rng, MODES[k % len(MODES)]) for k in range(20)]


def _draw_mixed(rng, mode):
    while True:
        wtype = rng.choice(["f32", "bf16"])
        L, D = rng.choice([1, 1, 2, 3, 4]), rng.choice([1, 2])
        T = rng.choice([1, 2, 5, 17, 33, 64])
        B = rng.choice([1, 2, 4, 6, 7, 16, 20, 31, 40, 96])
        H = rng.choice([16, 32, 48, 96, 160, 320, 640, 768, 1000, 1024, 1280])
        I = rng.choice([2, 8, 50, 128, 300, 640, 1024])
        if I > 16 * H or (wtype == "f32" and H > 1024):
            continue
        training = rng.random() < 0.75
        # the two-exchange GRU flavours run only persistently
        sched = 2 if (rng.random() < 0.25 and mode not in ("gru_tf", "gru_paper")) else 0
        pass_state = rng.random() < 0.75
        lengths = [rng.randint(0, T) for _ in range(B)] if rng.random() < 0.2 else None
        drop = (0.3, rng.randint(1, 99)) if training and L > 1 and rng.random() < 0.25 else None
        return mode, wtype, L, D, T, B, I, H, training, sched, pass_state, lengths, drop


_rng_mixed = random.Random(20261204)
MIXED_CASES = [_draw_mixed(_rng_mixed, MODES[k % len(MODES)]) for k in range(20)]


@pytest.mark.parametrize("k", range(len(CASES)))
def test_random_shape(k):
    mode, wtype, L, D, T, B, I, H, lengths, drop = CASES[k]
    print("random case", k, mode, wtype, L, D, T, B, I, H, "lengths" if lengths else "", drop, flush=True)
    case = synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=5000 + k)
    g = run_gpu(mode, L, D, case, wtype, lengths=lengths, dropout=drop)
    o = run_oracle(mode, L, D, case, lengths=lengths, dropout=drop)
    check(compare(g, o, mode, L, D), *TOL[wtype])


@pytest.mark.parametrize("k", range(len(MIXED_CASES)))
def test_random_mixed(k):
    mode, wtype, L, D, T, B, I, H, training, sched, pass_state, lengths, drop = MIXED_CASES[k]
    print("mixed case", k, mode, wtype, L, D, T, B, I, H, "train" if training else "inference",
          "sched", sched, "state" if pass_state else "no state", "lengths" if lengths else "", drop, flush=True)
    case = synth.make_case(mode, L, D, T, B, I, H, wtype=wtype, seed=7000 + k)
    g = run_gpu(mode, L, D, case, wtype, sched=sched, training=training, backward=training,
                pass_state=pass_state, lengths=lengths, dropout=drop)
    o = run_oracle(mode, L, D, case, backward=training, pass_state=pass_state, lengths=lengths, dropout=drop)
    check(compare(g, o, mode, L, D), *TOL[wtype])
