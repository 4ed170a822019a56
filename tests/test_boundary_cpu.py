"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/rnn.h declares, and its host-only calls (descriptor, weight
layout, workspace size, status strings, argument checks) behave as declared.
No compute call is made here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rnn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rnn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def R():
    import layer_rnn_forward_amd as R
    R.load_library()
    return R


def test_header_declares_the_operator_calls():
    names = declared_functions()
    for n in ("rnn_create", "rnn_workspace_size", "rnn_forward_inference", "rnn_forward_training",
              "rnn_backward_data", "rnn_backward_weights", "rnn_destroy", "rnn_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(R):
    lib = ctypes.CDLL(R.lib_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(R):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert R.rnn_status_string(code) and R.rnn_status_string(code) != "unknown status"
    assert R.rnn_status_string(-99) == "unknown status"


@pytest.mark.parametrize("args", [
    ("lstm", 0, 1, 8, 8), ("lstm", 1, 3, 8, 8), ("lstm", 1, 1, 0, 8), ("gru", 1, 1, 8, -1)])
def test_create_rejects_bad_descriptors(R, args):
    with pytest.raises(R.RNNError) as e:
        R.rnn_create(*args)
    assert e.value.status == -1


@pytest.mark.parametrize("mode,G", [("rnn_tanh", 1), ("lstm", 4), ("gru", 3), ("gru_tf", 3),
                                    ("gru_paper", 3)])
@pytest.mark.parametrize("wtype,es", [("f32", 4), ("bf16", 2)])
def test_weight_layout(R, mode, G, wtype, es):
    L, D, I, H = 3, 2, 13, 7
    h = R.rnn_create(mode, L, D, I, H, wtype)
    spans = []
    for grad in (0, 1):
        total = R.rnn_weights_size(h, grad)
        for l in range(L):
            I_l = I if l == 0 else D * H
            for d in range(D):
                for which, (cnt, bytes_per) in enumerate(
                        [(G * H * I_l, es if not grad else 4), (G * H * H, es if not grad else 4),
                         (G * H, 4), (G * H, 4)]):
                    off, n = R.rnn_weight_offset(h, grad, l, d, which)
                    assert n == cnt
                    assert off + n * bytes_per <= total
                    if d == 0:
                        assert off % 256 == 0
                    spans.append((grad, off, off + n * bytes_per))
        # no two tensors overlap
        s = sorted(x[1:] for x in spans if x[0] == grad)
        for (a0, a1), (b0, b1) in zip(s, s[1:]):
            assert a1 <= b0
    with pytest.raises(R.RNNError):
        R.rnn_weight_offset(h, 0, L, 0, 0)
    with pytest.raises(R.RNNError):
        R.rnn_weight_offset(h, 0, 0, D, 0)


def test_workspace_size_properties(R):
    for mode in ("rnn_tanh", "lstm", "gru", "gru_tf", "gru_paper"):
        for wtype in ("f32", "bf16"):
            h = R.rnn_create(mode, 2, 2, 800, 800, wtype)
            inf = R.rnn_workspace_size(h, 300, 20, 0)
            tr = R.rnn_workspace_size(h, 300, 20, 1)
            assert tr > inf > 0
            assert R.rnn_workspace_size(h, 600, 20, 1) > tr
            assert R.rnn_workspace_size(h, 0, 20, 1) > 0
            assert R.rnn_workspace_size(h, 300, 20, 1) == tr  # deterministic
    h = R.rnn_create("lstm", 1, 1, 800, 800, "bf16")
    # the reserve (5 fp32 values per step, row and unit) dominates training
    tr = R.rnn_workspace_size(h, 300, 20, 1)
    assert tr >= 300 * 20 * 800 * 5 * 4
    with pytest.raises(R.RNNError):
        R.rnn_workspace_size(h, -1, 20, 1)


@pytest.mark.parametrize("mode", ["rnn_tanh", "lstm", "gru", "gru_tf", "gru_paper"])
def test_hidden_size_limit(R, mode):
    """The register-resident W_hh slices bound the hidden size: 1024 (fp32
    weights) and 2048 (bf16 weights) are supported for every mode, stack and
    batch, inference and training (a unidirectional stack whose wavefront
    would not fit runs its layers one launch each); one unit more with one
    row and one layer is UNSUPPORTED, cleanly."""
    for wtype, hmax in (("f32", 1024), ("bf16", 2048)):
        for L, D, B in ((1, 1, 1), (3, 1, 1), (3, 1, 20), (2, 2, 5), (1, 2, 128)):
            h = R.rnn_create(mode, L, D, 64, hmax, wtype)
            for training in (0, 1):
                assert R.rnn_workspace_size(h, 16, B, training) > 0, (wtype, L, D, B, training)
            R.rnn_destroy(h)
        h = R.rnn_create(mode, 1, 1, 64, hmax + 1, wtype)
        for training in (0, 1):
            with pytest.raises(R.RNNError, match="unsupported"):
                R.rnn_workspace_size(h, 16, 1, training)
        R.rnn_destroy(h)


def test_dropout_setter_and_workspace(R):
    h = R.rnn_create("lstm", 3, 2, 64, 48)
    base_tr = R.rnn_workspace_size(h, 20, 8, 1)
    base_inf = R.rnn_workspace_size(h, 20, 8, 0)
    R.rnn_set_dropout(h, 0.25, (1 << 63) + 5)
    # one fp32 [T][B][D*H] slot per dropped layer (layers 1 and 2), inference unchanged
    assert R.rnn_workspace_size(h, 20, 8, 1) >= base_tr + 2 * 20 * 8 * 2 * 48 * 4
    assert R.rnn_workspace_size(h, 20, 8, 0) == base_inf
    R.rnn_set_dropout(h, 0.0, 1)
    assert R.rnn_workspace_size(h, 20, 8, 1) == base_tr
    R.rnn_set_dropout(h, 1.0, 1)
    for bad in (-0.01, 1.01, float("nan")):
        with pytest.raises(R.RNNError) as e:
            R.rnn_set_dropout(h, bad, 1)
        assert e.value.status == -1
    # mask query: layer 0 and layer L have no dropout
    for layer in (0, 3):
        assert R.load_library().rnn_dropout_mask(h.ptr, None, 2, 2, layer, None) == -1
    R.rnn_destroy(h)
    # a single layer has nothing to drop
    h1 = R.rnn_create("gru", 1, 1, 16, 16)
    w = R.rnn_workspace_size(h1, 10, 4, 1)
    R.rnn_set_dropout(h1, 0.5, 3)
    assert R.rnn_workspace_size(h1, 10, 4, 1) == w
    R.rnn_destroy(h1)


def test_schedule_setter(R):
    h = R.rnn_create("lstm", 1, 1, 8, 8)
    for s in (0, 1, 2):
        R.rnn_set_schedule(h, s)
    with pytest.raises(R.RNNError):
        R.rnn_set_schedule(h, 7)


def test_product_path_has_no_oracle_dependency():
    """The package and its native sources never import, include or load the
    oracle."""
    pkg = os.path.join(ROOT, "layer_rnn_forward_amd")
    pat = re.compile(r"^\s*(from\s+oracle|import\s+oracle|#include\s+.*oracle)", re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), f
                assert "rnn_oracle" not in text, f


def test_workspace_covers_split_k_partials(R, monkeypatch):
    """The workspace holds the fp32 partials of split-K products: forcing
    eight splits (clamped to K/256 per product) must make room for eight
    partial copies of the fused weight gradients (dW_ih and dW_hh, 3200 x 801
    each at this shape) and for the data gradient's (6000 x 800)."""
    h = R.rnn_create("lstm", 1, 1, 800, 800, "f32")
    T, B = 300, 20
    monkeypatch.setenv("RNN_DW_SPLIT", "1")
    w1 = R.rnn_workspace_size(h, T, B, 1)
    monkeypatch.setenv("RNN_DW_SPLIT", "8")
    w8 = R.rnn_workspace_size(h, T, B, 1)
    assert w8 > w1
    assert w8 >= 8 * 2 * 3200 * 801 * 4          # weight-gradient partials (K = 6000)
    assert w8 >= 8 * T * B * 800 * 4              # data-gradient partials (K = 3200)
    monkeypatch.delenv("RNN_DW_SPLIT")
    assert R.rnn_workspace_size(h, T, B, 1) <= w8
    R.rnn_destroy(h)


def test_plan_info_is_consistent(R, monkeypatch):
    """The plan diagnostic reports a plan whose batch chunks cover the batch,
    whose workgroups cover the hidden width and whose grid holds every group
    (host only; without a GPU nothing is co-resident, so the sweeps are
    stepped and the placement linear)."""
    for mode, L, D, wtype in (("lstm", 1, 1, "bf16"), ("gru", 2, 2, "f32"), ("rnn_tanh", 5, 1, "bf16")):
        h = R.rnn_create(mode, L, D, 800, 800, wtype)
        for place in ("0", "1"):
            monkeypatch.setenv("RNN_PLACE", place)
            info = R.rnn_plan_info(h, 300, 20, True)
            for kind in ("fwd", "bwd"):
                p = info[kind]
                assert p["nchunk"] * p["rows"] >= 20 > (p["nchunk"] - 1) * p["rows"]
                assert p["nwg"] * p["units"] >= 800 > (p["nwg"] - 1) * p["units"]
                assert p["grid"] >= p["nwg"] * p["groups"]
                if p["place"] == 0:
                    assert p["grid"] == p["nwg"] * p["groups"]
        assert R.rnn_plan_info(h, 300, 20, False).keys() == {"fwd"}
        R.rnn_destroy(h)
    monkeypatch.delenv("RNN_PLACE")
