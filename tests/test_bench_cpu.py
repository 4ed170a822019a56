"""The benchmark's arithmetic, checked on the CPU: the flop count it divides
by (the GEMM flops of the pages' formulation, 2*M*N*K), its split into the
kernel kinds, the per-kernel roofline entries, and the refusal of a
multi-GPU run (this build measures one GPU)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from layer_rnn_forward_amd import synth  # noqa: E402


def test_forward_flops_closed_form():
    # one LSTM layer at the DS2 shape: GX = X W_ih^T (T*B x 4H x I) and the
    # recurrence h W_hh^T (T*B x 4H x H), 2 flops per multiply-add
    assert bench.flops("lstm", 300, 20, 800, 800, 1, 1) == 2 * 300 * 20 * 4 * 800 * (800 + 800)
    # the training step is three times the forward: 184.32 GFLOP
    assert 3 * bench.flops("lstm", 300, 20, 800, 800, 1, 1) == 184_320_000_000
    # five bidirectional layers: layer 0 reads I, the others the 2H-wide
    # concatenation of the layer below
    per_dir_l0 = 2 * 300 * 20 * 3 * 800 * (800 + 800)
    per_dir_up = 2 * 300 * 20 * 3 * 800 * (1600 + 800)
    assert bench.flops("gru", 300, 20, 800, 800, 5, 2) == 2 * per_dir_l0 + 4 * 2 * per_dir_up
    assert bench.flops("rnn_tanh", 10, 3, 7, 5, 1, 1) == 2 * 10 * 3 * 1 * 5 * (7 + 5)


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_kernel_flops_add_up_to_the_training_step(name):
    w = synth.WORKLOADS[name]
    parts = bench.kernel_flops(w)
    total = 3 * bench.flops(w.mode, w.T, w.B, w.input_size, w.hidden, w.layers, w.dirs)
    assert sum(parts.values()) == pytest.approx(total, rel=1e-12)
    # the backward's products: dX equals the input projection, dW is both
    assert parts["gemm_dx"] == parts["gemm_input"]
    assert parts["gemm_dw"] == pytest.approx(parts["gemm_input"] + parts["recurrent_fwd"], rel=1e-12)
    assert parts["recurrent_bwd"] == parts["recurrent_fwd"]


def test_kernel_roofline_entries():
    w = synth.WORKLOADS["lstm_ds2_bf16"]
    steps = 20
    kern = {"gemm_input": {"launches": 20, "avg_us": 64.0, "total_ms": 1.28},
            "recurrent_bwd": {"launches": 20, "avg_us": 800.0, "total_ms": 16.0}}
    r = bench.kernel_rooflines(w, kern, steps, floor_us=1.6)
    assert set(r) == {"gemm_input", "recurrent_bwd"}
    g = r["gemm_input"]
    # 30.72 GFLOP in 64 us
    assert g["achieved"] == pytest.approx(30.72e9 / 64e-6 / 1e12, rel=1e-3)
    assert g["bound"] == "mfma" and g["peak"] == 2500.0
    assert g["frac_mfma_peak"] == pytest.approx(g["achieved"] / 2500.0, rel=1e-3)
    b = r["recurrent_bwd"]
    assert b["bound"] == "latency"
    assert b["us_per_recurrent_step"] == pytest.approx(800.0 / 300, rel=1e-3)
    assert b["frac_of_latency_floor"] == pytest.approx(1.6 / (800.0 / 300), rel=1e-3)
    assert b["achieved"] == pytest.approx(30.72e9 / 800e-6 / 1e12, rel=1e-3)


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
