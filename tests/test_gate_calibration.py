"""The calibrated gate biases of the 1.5B workloads reproduce the stated exit masses on
the calibration samples that tests/golden/make_gate_bias.py stored (the oracle's linear
terms z_k = g_k . h^(l_k) at the positions each workload's decode steps consume: 511..1022
after A's 512-token prompt, 8191..8446 after D's 8192-token prompt): the mean over positions of the
stick-breaking p_k (gist.science summary, section 2 "Methodik", part "Architektur":
equation for p_k) with w_k = sigmoid(z_k + b_k) equals the stated mass.  The biases the
workloads carry are the stored ones."""
import json
import os

import numpy as np

from synth import workload
from synth.configs import BIAS_CAL_1P5B_40_25_20_15, BIAS_CAL_1P5B_60_20_10_10

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gate_bias_1p5b.json")


def _masses(z, b):
    w = 1.0 / (1.0 + np.exp(-(z + np.asarray(b)[None, :])))
    p = np.zeros((z.shape[0], 4))
    rest = np.ones(z.shape[0])
    for k in range(3):
        p[:, k] = rest * w[:, k]
        rest = rest * (1.0 - w[:, k])
    p[:, 3] = rest
    return p.mean(axis=0)


def test_calibrated_biases_give_stated_masses():
    g = json.load(open(GOLDEN))
    for name, b_cfg, n in (("A", BIAS_CAL_1P5B_40_25_20_15, 512), ("D", BIAS_CAL_1P5B_60_20_10_10, 256)):
        z = np.asarray(g[name]["z"])
        assert z.shape == (n, 3)
        assert np.allclose(g[name]["bias"], b_cfg, rtol=0, atol=1e-12)
        m = _masses(z, b_cfg)
        assert np.allclose(m, g[name]["mass"], rtol=0, atol=1e-6), (name, m)
        # the header stores the biases as float32: the masses move by far less than 1e-3
        m32 = _masses(z, np.asarray(b_cfg, np.float32).astype(np.float64))
        assert np.allclose(m32, g[name]["mass"], rtol=0, atol=1e-5)
    # without calibration (sigmoid(b) alone) the same sample misses the stated masses
    from synth.configs import BIAS_MASS_40_25_20_15
    zA = np.asarray(g["A"]["z"])
    assert np.max(np.abs(_masses(zA, BIAS_MASS_40_25_20_15) - np.asarray(g["A"]["mass"]))) > 0.05
    # and the A biases do not carry over to the 8K positions (the linear term drifts)
    zD = np.asarray(g["D"]["z"])
    assert np.max(np.abs(_masses(zD, BIAS_CAL_1P5B_40_25_20_15) - np.asarray(g["A"]["mass"]))) > 0.05


def test_workloads_carry_the_calibrated_biases():
    assert workload("A").model.gate_bias == BIAS_CAL_1P5B_40_25_20_15
    assert workload("C").model.gate_bias == BIAS_CAL_1P5B_40_25_20_15
    assert workload("D").model.gate_bias == BIAS_CAL_1P5B_60_20_10_10


def test_bench_window_mass():
    """bench.py's expected exit mass of a timed window: over the whole calibrated range it is
    the stated mass; over A's first 20 positions it is the drifted mass of those positions;
    outside the sample, and for workloads without one, it is None."""
    import bench
    m = bench.expected_window_mass(workload("A"), 511, 512)
    assert np.allclose(m["value"], [0.4, 0.25, 0.2, 0.15], atol=1e-4), m
    assert m["positions"] == [511, 1022]
    m = bench.expected_window_mass(workload("D"), 8191, 256)
    assert np.allclose(m["value"], [0.6, 0.2, 0.1, 0.1], atol=1e-4), m
    g = json.load(open(GOLDEN))
    w20 = _masses(np.asarray(g["A"]["z"])[:20], BIAS_CAL_1P5B_40_25_20_15)
    assert np.allclose(bench.expected_window_mass(workload("A"), 511, 20)["value"], w20, atol=1e-4)
    assert bench.expected_window_mass(workload("A"), 1010, 20) is None      # past position 1022
    assert bench.expected_window_mass(workload("B"), 511, 20) is None       # no calibration sample
