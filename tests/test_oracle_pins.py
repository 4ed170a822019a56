"""Pins of the fp64 oracle (CPU only).

The oracle is checked against what the pages and mathematics fix: the
hand-worked GRU flavour values, zero-weight closed forms (forward and BPTT),
central finite differences for every gradient, ``torch.nn`` in float64 as a
library special case, and structural invariants.
"""

import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import rnn_oracle as orc
from tests import oracle_checks as oc

MODES = ("rnn_tanh", "lstm", "gru")


def test_gru_flavours_worked_values():
    assert oc.check_gru_worked_values(orc) < 1e-11


def test_gru_flavours_are_distinguished():
    # the worked case (ii) separates all three flavours by more than 0.05
    import json
    import os
    spec = json.load(open(os.path.join(oc.GOLDEN, "gru_variants_worked.json")))
    c = spec["cases"][1]
    vals = sorted([c["pytorch"], c["tf"], c["paper"]])
    assert min(b - a for a, b in zip(vals, vals[1:])) > 0.05


def test_forward_closed_forms():
    assert oc.check_closed_forms(orc) < 1e-11


def test_bptt_closed_forms():
    assert oc.check_bptt_closed_forms(orc) < 1e-12


@pytest.mark.parametrize("mode,L,D", list(itertools.product(MODES, (1, 2), (1, 2))))
def test_matches_torch_nn_float64(mode, L, D):
    assert oc.check_against_torch(orc, mode, L, D) < 1e-11


@pytest.mark.parametrize("mode,L,D", list(itertools.product(MODES, (1, 2), (1, 2))))
def test_finite_differences(mode, L, D):
    assert oc.check_finite_differences(orc, mode, L, D) < 1e-6


@pytest.mark.parametrize("variant,L,D", list(itertools.product(("tf", "paper"), (1, 2), (1, 2))))
def test_gru_flavour_finite_differences(variant, L, D):
    """Backward of the TensorFlow and original-paper GRU flavours (n reads
    (r*h) W_hn^T) against central differences, with and without lengths."""
    assert oc.check_finite_differences(orc, "gru", L, D, gru_variant=variant) < 1e-6
    assert oc.check_finite_differences(orc, "gru", L, D, gru_variant=variant, lengths=[1, 3]) < 1e-6


# ------------------------------------------------------- variable lengths
@pytest.mark.parametrize("mode,L,D", list(itertools.product(MODES, (1, 2), (1, 2))))
def test_packed_matches_torch_nn_float64(mode, L, D):
    """torch.nn on pack_padded_sequence input (rows of lengths 4, 1, 3)."""
    assert oc.check_against_torch(orc, mode, L, D, lengths=[4, 1, 3]) < 1e-11


@pytest.mark.parametrize("mode,L,D", list(itertools.product(MODES, (1, 2), (1, 2))))
def test_packed_rows_equal_truncated_sequences(mode, L, D):
    assert oc.check_packed_truncation(orc, mode, L, D, lengths=[5, 0, 2, 3]) < 1e-13


@pytest.mark.parametrize("mode,D", list(itertools.product(MODES, (1, 2))))
def test_packed_finite_differences(mode, D):
    assert oc.check_finite_differences(orc, mode, 2, D, lengths=[1, 3]) < 1e-6


@pytest.mark.parametrize("mode", MODES)
def test_full_lengths_equal_unpacked(mode):
    case = oc.rand_case(mode, 2, 2, 4, 3, 3, 5, seed=3)
    a = orc.forward(mode, case["x"], case["params"], h0=case["h0"], c0=case["c0"], num_dirs=2)
    b = orc.forward(mode, case["x"], case["params"], h0=case["h0"], c0=case["c0"], num_dirs=2,
                    lengths=[4, 4, 4])
    for u, v in zip(a[:3], b[:3]):
        if u is not None:
            assert np.array_equal(u, v)


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("mode", MODES)
def test_reverse_direction_is_time_reversed_forward(mode):
    # I1: direction 1 on x == direction 0 (with direction-1 weights) on x reversed
    c = oc.rand_case(mode, 1, 2, 5, 3, 4, 3, seed=21)
    y, hy, cy, _ = orc.forward(mode, c["x"], c["params"], h0=c["h0"], c0=c["c0"], num_dirs=2)
    p1 = [[c["params"][0][1]]]
    c0 = c["c0"][1:2] if mode == "lstm" else None
    yr, hyr, cyr, _ = orc.forward(mode, c["x"][::-1].copy(), p1, h0=c["h0"][1:2], c0=c0)
    np.testing.assert_allclose(y[:, :, 3:], yr[::-1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hy[1], hyr[0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", MODES)
def test_batch_rows_independent(mode):
    # I2: permuting batch rows permutes every output and gradient the same way
    c = oc.rand_case(mode, 2, 2, 4, 5, 3, 4, seed=22)
    perm = np.array([3, 0, 4, 1, 2])
    y, hy, cy, cache = orc.forward(mode, c["x"], c["params"], h0=c["h0"], c0=c["c0"],
                                   num_dirs=2, keep=True)
    dx, dh0, dc0, dp = orc.backward(mode, c["params"], cache, c["dy"], dhy=c["dhy"],
                                    dcy=c["dcy"], num_dirs=2)
    c0p = c["c0"][:, perm] if mode == "lstm" else None
    dcyp = c["dcy"][:, perm] if mode == "lstm" else None
    y2, hy2, cy2, cache2 = orc.forward(mode, c["x"][:, perm], c["params"], h0=c["h0"][:, perm],
                                       c0=c0p, num_dirs=2, keep=True)
    dx2, dh02, dc02, dp2 = orc.backward(mode, c["params"], cache2, c["dy"][:, perm],
                                        dhy=c["dhy"][:, perm], dcy=dcyp, num_dirs=2)
    np.testing.assert_allclose(y2, y[:, perm], atol=1e-13)
    np.testing.assert_allclose(dx2, dx[:, perm], atol=1e-13)
    np.testing.assert_allclose(dh02, dh0[:, perm], atol=1e-13)
    for l in range(2):
        for d in range(2):
            for k in dp[l][d]:
                np.testing.assert_allclose(dp2[l][d][k], dp[l][d][k], atol=1e-12)


@pytest.mark.parametrize("mode", MODES)
def test_final_state_is_last_output(mode):
    # I3: hy[d=0] = y[T-1, :, :H]; hy[d=1] = y[0, :, H:] (top layer)
    c = oc.rand_case(mode, 2, 2, 6, 2, 3, 4, seed=23)
    y, hy, _, _ = orc.forward(mode, c["x"], c["params"], h0=c["h0"], c0=c["c0"], num_dirs=2)
    assert np.array_equal(hy[2], y[-1, :, :4])
    assert np.array_equal(hy[3], y[0, :, 4:])


@pytest.mark.parametrize("mode,D", list(itertools.product(MODES, (1, 2))))
def test_stack_equals_chained_layers(mode, D):
    # I4: an L-layer call == L chained single-layer calls, forward and backward
    c = oc.rand_case(mode, 3, D, 4, 2, 3, 4, seed=24)
    y, hy, cy, cache = orc.forward(mode, c["x"], c["params"], h0=c["h0"], c0=c["c0"],
                                   num_dirs=D, keep=True)
    dx, dh0, dc0, dp = orc.backward(mode, c["params"], cache, c["dy"], dhy=c["dhy"],
                                    dcy=c["dcy"], num_dirs=D)
    inp = c["x"]
    caches = []
    for l in range(3):
        sl = slice(l * D, (l + 1) * D)
        c0 = c["c0"][sl] if mode == "lstm" else None
        inp, hyl, cyl, cl = orc.forward(mode, inp, [c["params"][l]], h0=c["h0"][sl], c0=c0,
                                        num_dirs=D, keep=True)
        caches.append(cl)
        np.testing.assert_allclose(hyl, hy[sl], atol=1e-14)
    np.testing.assert_allclose(inp, y, atol=1e-14)
    g = c["dy"]
    for l in (2, 1, 0):
        sl = slice(l * D, (l + 1) * D)
        dcy = c["dcy"][sl] if mode == "lstm" else None
        g, dh0l, dc0l, dpl = orc.backward(mode, [c["params"][l]], caches[l], g,
                                          dhy=c["dhy"][sl], dcy=dcy, num_dirs=D)
        np.testing.assert_allclose(dh0l, dh0[sl], atol=1e-13)
        for d in range(D):
            for k in dpl[0][d]:
                np.testing.assert_allclose(dpl[0][d][k], dp[l][d][k], atol=1e-12)
    np.testing.assert_allclose(g, dx, atol=1e-13)


@pytest.mark.parametrize("mode", MODES)
def test_gradients_linear_in_upstream(mode):
    # I6: gradients are linear in (dy, dhy, dcy); zero in -> zero out
    c = oc.rand_case(mode, 2, 2, 4, 2, 3, 4, seed=25)
    _, _, _, cache = orc.forward(mode, c["x"], c["params"], h0=c["h0"], c0=c["c0"],
                                 num_dirs=2, keep=True)
    rng = np.random.default_rng(3)
    dy2 = rng.normal(size=c["dy"].shape)
    dhy2 = rng.normal(size=c["dhy"].shape)
    dcy2 = rng.normal(size=c["dhy"].shape) if mode == "lstm" else None

    def run(dy, dhy, dcy):
        return orc.backward(mode, c["params"], cache, dy, dhy=dhy, dcy=dcy, num_dirs=2)

    a = run(c["dy"], c["dhy"], c["dcy"])
    b = run(dy2, dhy2, dcy2)
    comb = run(c["dy"] + 2 * dy2, c["dhy"] + 2 * dhy2,
               (c["dcy"] + 2 * dcy2) if mode == "lstm" else None)
    np.testing.assert_allclose(comb[0], a[0] + 2 * b[0], atol=1e-12)
    np.testing.assert_allclose(comb[1], a[1] + 2 * b[1], atol=1e-12)
    z = run(np.zeros_like(c["dy"]), np.zeros_like(c["dhy"]),
            np.zeros_like(c["dhy"]) if mode == "lstm" else None)
    assert not np.any(z[0]) and not np.any(z[1])
    for l in range(2):
        for d in range(2):
            for k in z[3][l][d]:
                assert not np.any(z[3][l][d][k])


@pytest.mark.parametrize("mode", MODES)
def test_bias_gradient_relations(mode):
    # I7: lstm/vanilla db_ih == db_hh; GRU equal on r and z, n-slice of db_hh
    # is sum(da_n * r) and differs in general
    c = oc.rand_case(mode, 1, 2, 5, 3, 4, 3, seed=26)
    _, _, _, cache = orc.forward(mode, c["x"], c["params"], h0=c["h0"], c0=c["c0"],
                                 num_dirs=2, keep=True)
    _, _, _, dp = orc.backward(mode, c["params"], cache, c["dy"], dhy=c["dhy"], dcy=c["dcy"],
                               num_dirs=2)
    H = 3
    for d in range(2):
        if mode == "gru":
            np.testing.assert_allclose(dp[0][d]["b_ih"][:2 * H], dp[0][d]["b_hh"][:2 * H],
                                       atol=1e-14)
            assert np.max(np.abs(dp[0][d]["b_ih"][2 * H:] - dp[0][d]["b_hh"][2 * H:])) > 1e-6
        else:
            np.testing.assert_allclose(dp[0][d]["b_ih"], dp[0][d]["b_hh"], atol=1e-14)


def test_single_step_by_hand():
    # I8: T = 1, H = I = 1, scalar cells evaluated with the math module
    s = lambda a: 1.0 / (1.0 + math.exp(-a))
    x, h, c = 0.7, -0.3, 0.45
    wi = [0.2, -0.5, 0.9, 0.4]
    wh = [-0.6, 0.1, 0.3, -0.8]
    bi = [0.05, 0.2, -0.1, 0.3]
    bh = [-0.15, 0.1, 0.25, -0.05]
    p = {"w_ih": np.array(wi).reshape(4, 1), "w_hh": np.array(wh).reshape(4, 1),
         "b_ih": np.array(bi), "b_hh": np.array(bh)}
    a = [wi[k] * x + bi[k] + wh[k] * h + bh[k] for k in range(4)]
    i, f, g, o = s(a[0]), s(a[1]), math.tanh(a[2]), s(a[3])
    c1 = f * c + i * g
    h1 = o * math.tanh(c1)
    y, hy, cy, _ = orc.forward("lstm", np.full((1, 1, 1), x), [[p]], h0=np.full((1, 1, 1), h),
                               c0=np.full((1, 1, 1), c))
    assert abs(float(hy[0, 0, 0]) - h1) < 1e-15 and abs(float(cy[0, 0, 0]) - c1) < 1e-15
    # GRU (PyTorch flavour) with the first three rows
    pg = {"w_ih": np.array(wi[:3]).reshape(3, 1), "w_hh": np.array(wh[:3]).reshape(3, 1),
          "b_ih": np.array(bi[:3]), "b_hh": np.array(bh[:3])}
    r = s(wi[0] * x + bi[0] + wh[0] * h + bh[0])
    z = s(wi[1] * x + bi[1] + wh[1] * h + bh[1])
    n = math.tanh(wi[2] * x + bi[2] + r * (wh[2] * h + bh[2]))
    hg = (1 - z) * n + z * h
    y, hy, _, _ = orc.forward("gru", np.full((1, 1, 1), x), [[pg]], h0=np.full((1, 1, 1), h))
    assert abs(float(hy[0, 0, 0]) - hg) < 1e-15
    # the PyTorch snippet's form hy = n + z*(h - n) is the same number
    assert abs(hg - (n + z * (h - n))) < 1e-15
    pv = {"w_ih": np.array([[wi[0]]]), "w_hh": np.array([[wh[0]]]),
          "b_ih": np.array([bi[0]]), "b_hh": np.array([bh[0]])}
    y, hy, _, _ = orc.forward("rnn_tanh", np.full((1, 1, 1), x), [[pv]],
                              h0=np.full((1, 1, 1), h))
    assert abs(float(hy[0, 0, 0]) - math.tanh(a[0])) < 1e-15


def test_flop_counts():
    # GEMM flops of the Deep Speech 2 single-layer LSTM: 2*T*B*4H*(I+H)
    assert oracle.forward_flops("lstm", 300, 20, 800, 800, 1, 1) == 61_440_000_000
    assert oracle.train_step_flops("lstm", 300, 20, 800, 800, 1, 1) == 184_320_000_000
    assert oracle.forward_flops("gru", 300, 20, 800, 800, 1, 1) == 46_080_000_000
    assert oracle.forward_flops("lstm", 300, 20, 800, 800, 5, 2) == 860_160_000_000
    assert oracle.forward_flops("rnn_tanh", 300, 20, 800, 800, 5, 2) == 215_040_000_000
