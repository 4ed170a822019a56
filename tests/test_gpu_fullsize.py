"""Full-size parity at the Deep Speech 2 shapes (T=300, B=20, input/hidden
800), in the launch configuration the benchmark times (automatic schedule:
persistent sweeps).  Every output and gradient element is compared with the
fp64 oracle; tolerances as in test_gpu_parity.
"""

import pytest

from layer_rnn_forward_amd import synth
from tests.gpu_harness import check, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-3), "bf16": (2e-2, 2e-2)}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["lstm_ds2_f32", "lstm_ds2_bf16", "gru_ds2_f32"])
def test_ds2_single_layer(name):
    w = synth.WORKLOADS[name]
    print("CASE", w, flush=True)
    case = synth.make_workload(w)
    g = run_gpu(w.mode, w.layers, w.dirs, case, w.wtype)
    o = run_oracle(w.mode, w.layers, w.dirs, case)
    errs = compare(g, o, w.mode, w.layers, w.dirs)
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    check(errs, *TOL[w.wtype])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["lstm_ds2_l5_bi_bf16", "gru_ds2_l5_bi_bf16",
                                  "tanh_ds2_l5_bi_bf16", "lstm_ds2_l5_uni_bf16"])
def test_ds2_five_layer(name):
    w = synth.WORKLOADS[name]
    print("CASE", w, flush=True)
    case = synth.make_workload(w)
    g = run_gpu(w.mode, w.layers, w.dirs, case, w.wtype)
    o = run_oracle(w.mode, w.layers, w.dirs, case)
    errs = compare(g, o, w.mode, w.layers, w.dirs)
    worst = max(errs, key=errs.get)
    print("worst", worst, f"{errs[worst]:.2e}", flush=True)
    check(errs, *TOL[w.wtype])
