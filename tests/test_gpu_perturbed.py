"""Race detection by ordering perturbation: the perturbed build
(``librnn_mi355x_perturb.so``, -DRNN_PERTURB) pauses pseudo-randomly at every
flag wait and flag publication of the recurrent sweeps, so producers,
consumers and the waves of a workgroup meet with skews the normal build never
has.  The arithmetic is unchanged, so every output and gradient must be
bitwise equal to the normal build's: a missing wait, a wrong producer range,
a flag published before its stores or a workgroup-internal race would show
as a difference.  The perturbed library runs in a child process (one library
per process); this process runs the normal one."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import layer_rnn_forward_amd as R  # noqa: E402
from layer_rnn_forward_amd.build import PERTURB_LIB  # noqa: E402
from tests import perturb_cases  # noqa: E402

pytestmark = pytest.mark.gpu


def test_perturbed_build_is_bitwise_equal(tmp_path):
    assert os.path.exists(PERTURB_LIB), "the perturbed test build is missing (run build())"
    assert os.path.realpath(R.lib_path()) != os.path.realpath(PERTURB_LIB)
    ref = perturb_cases.run_all()
    out = tmp_path / "perturbed.npz"
    env = dict(os.environ, RNN_LIB=PERTURB_LIB)
    print("running the perturbed build in a child process", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "perturb_cases.py"), str(out)],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.returncode
    assert "perturb" in r.stdout.split("library", 1)[1].splitlines()[0]
    got = np.load(out)
    assert sorted(got.files) == sorted(ref), (sorted(got.files), sorted(ref))
    bad = []
    for k, v in ref.items():
        g = got[k]
        assert g.shape == v.shape, k
        # NaN-aware bitwise comparison (a NaN would itself be a failure elsewhere)
        if not np.array_equal(g.view(np.uint64), v.view(np.uint64)):
            bad.append((k, float(np.nanmax(np.abs(g - v)))))
    assert not bad, bad
    # every case produced finite outputs
    for k, v in ref.items():
        assert np.isfinite(v).all(), k
    # the pauses happened: the perturbed forward sweep's step is much slower
    # (about three pauses of ~1.7 us on average per step, against a
    # ~2.5 us step)
    base = perturb_cases.forward_sweep_us_per_step()
    pert = float(r.stdout.split("forward sweep us/step", 1)[1].split()[0])
    print("forward sweep us/step: normal", base, "perturbed", pert, flush=True)
    assert pert > 1.5 * base, (base, pert)
