"""Pins of the oracle's Philox generator and of its inter-layer dropout.

Philox: the known-answer vectors published with the Random123 library of
Salmon et al. ("Parallel random numbers: as easy as 1, 2, 3", SC'11), and the
4x64 instance against numpy's ``Philox`` bit generator (a library routine of
the same family; numpy increments its 256-bit counter before each block).

Dropout: the keep mask's statistics and its dependence on layer and seed,
the mask gather against the scalar generator, the training pass against a
composition of one-layer ``torch.nn`` modules with the mask applied between
them, and central finite differences with dropout active.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import philox as px
from oracle import rnn_oracle as orc
from tests import oracle_checks as oc


def test_philox_known_answers():
    assert oc.philox_kat_failures(px) == []


def _split64(v, n):
    return [(v >> (64 * i)) & ((1 << 64) - 1) for i in range(n)]


@pytest.mark.parametrize("counter,key", [(0, 0), (7, 12345), ((1 << 64) - 1, 3),
                                         (0x0123456789ABCDEF_FEDCBA9876543210, (5 << 64) | 9)])
def test_philox4x64_matches_numpy(counter, key):
    bg = np.random.Philox(counter=counter, key=key)
    raw = [int(v) for v in bg.random_raw(8)]
    k = _split64(key, 2)
    mine = []
    for i in (1, 2):   # numpy increments before generating
        mine += px.philox4(_split64((counter + i) % (1 << 256), 4), k, 64)
    assert raw == mine


def test_philox_array_matches_scalar():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 1 << 32, size=(4, 50), dtype=np.uint64)
    for k0, k1 in ((0, 0), (0xDEADBEEF, 0x12345678)):
        arr = px.philox4x32_array(c[0], c[1], c[2], c[3], k0, k1)
        for j in range(50):
            assert [int(a[j]) for a in arr] == px.philox4([int(v) for v in c[:, j]], (k0, k1), 32)


def test_dropout_threshold():
    assert orc.dropout_threshold(0.0) == 0
    assert orc.dropout_threshold(1.0) == 1 << 32
    assert orc.dropout_threshold(0.5) == 1 << 31
    assert orc.dropout_threshold(0.25) == 1 << 30
    for bad in (-0.1, 1.5):
        with pytest.raises(ValueError):
            orc.dropout_threshold(bad)


def test_dropout_mask_properties():
    assert oc.dropout_mask_failures(orc, px) == []


@pytest.mark.parametrize("mode", ["rnn_tanh", "lstm", "gru"])
@pytest.mark.parametrize("L,D", [(2, 1), (3, 2)])
@pytest.mark.parametrize("p", [0.3, 1.0])
def test_dropout_against_torch_composition(mode, L, D, p):
    assert oc.check_dropout_against_torch(orc, mode, L, D, p, seed=77) < 1e-11


@pytest.mark.parametrize("mode,variant", [("lstm", "pytorch"), ("gru", "tf")])
def test_dropout_finite_differences(mode, variant):
    err = oc.check_finite_differences(orc, mode, 2, 2, T=3, B=2, I=3, H=3, gru_variant=variant,
                                      dropout=0.4, dropout_seed=5)
    assert err < 1e-6


def test_dropout_zero_is_no_dropout():
    case = oc.rand_case("lstm", 3, 2, 4, 3, 5, 6, seed=1)
    a = orc.forward("lstm", case["x"], case["params"], h0=case["h0"], c0=case["c0"], num_dirs=2)
    b = orc.forward("lstm", case["x"], case["params"], h0=case["h0"], c0=case["c0"], num_dirs=2,
                    dropout=0.0, dropout_seed=123)
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u, v)
    # a single layer has nothing to drop
    c = oc.rand_case("gru", 1, 1, 4, 3, 5, 6, seed=2)
    y0 = orc.forward("gru", c["x"], c["params"], h0=c["h0"])[0]
    y1 = orc.forward("gru", c["x"], c["params"], h0=c["h0"], dropout=0.7, dropout_seed=9)[0]
    assert np.array_equal(y0, y1)
