"""Pins of the oracle's exit probabilities, mixture and sampler: closed forms of the
stick-breaking product, brute force on small distributions, and chi-square tests
of sampled tokens and exits against pi_mix and p_k."""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import model as om
from synth import cached_weights, tiny_variant
from synth.configs import BIAS_MASS_40_25_20_15, BIAS_MASS_60_20_10_10


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_exit_probs_sum_to_one():
    rng = np.random.default_rng(0)
    for _ in range(200):
        w = list(rng.random(3)) + [1.0]
        p = om.exit_probs(w)
        assert abs(sum(p) - 1.0) < 1e-12
        assert all(x >= 0 for x in p)
        # first exit: w_1; last exit: prod of (1 - w_j)
        assert p[0] == w[0]
        assert abs(p[3] - (1 - w[0]) * (1 - w[1]) * (1 - w[2])) < 1e-15


@pytest.mark.parametrize("biases,mass", [
    (BIAS_MASS_40_25_20_15, (0.4, 0.25, 0.2, 0.15)),
    (BIAS_MASS_60_20_10_10, (0.6, 0.2, 0.1, 0.1)),
])
def test_stated_exit_masses_at_zero_linear_term(biases, mass):
    p = om.exit_probs([sig(b) for b in biases] + [1.0])
    assert np.allclose(p, mass, rtol=0, atol=1e-12)


def test_closed_gates_put_all_mass_on_last_exit():
    p = om.exit_probs([0.0, 0.0, 0.0, 1.0])
    assert p == [0.0, 0.0, 0.0, 1.0]


def test_walk_gates_brute_force():
    w = [0.3, 0.5, 0.25, 1.0]
    # exits from the strict '<' rule at and around each boundary
    assert om.walk_gates(w, [0.0, 0.9, 0.9, 0.5]) == 0
    assert om.walk_gates(w, [0.3, 0.0, 0.9, 0.5]) == 1
    assert om.walk_gates(w, [0.3, 0.5, 0.2, 0.5]) == 2
    assert om.walk_gates(w, [0.3, 0.5, 0.25, 0.5]) == 3
    # exit frequencies over a product grid of u_1..u_3 equal p_k exactly
    g = (np.arange(40) + 0.5) / 40
    counts = np.zeros(4)
    for a in g:
        for b in g:
            for c in g:
                counts[om.walk_gates(w, [a, b, c, 0.0])] += 1
    assert np.allclose(counts / counts.sum(), om.exit_probs(w), atol=1e-12)


def test_inverse_cdf_boundaries():
    pi = np.array([0.25, 0.25, 0.5])
    assert om.inverse_cdf(pi, 0.0) == 0
    assert om.inverse_cdf(pi, np.nextafter(0.25, 0)) == 0
    assert om.inverse_cdf(pi, 0.25) == 1
    assert om.inverse_cdf(pi, 0.5) == 2
    assert om.inverse_cdf(pi, np.nextafter(1.0, 0)) == 2
    # zero-probability ids are never drawn
    pi0 = np.array([0.0, 0.5, 0.0, 0.5, 0.0])
    assert om.inverse_cdf(pi0, 0.0) == 1
    assert om.inverse_cdf(pi0, 0.5) == 3
    # rounding leaves the running sum short of u: the last id with nonzero mass
    pis = np.array([0.3, 0.3, 0.3999999, 0.0])
    assert om.inverse_cdf(pis, 0.99999995) == 2


def test_inverse_cdf_grid_frequencies():
    rng = np.random.default_rng(1)
    pi = rng.random(7)
    pi /= pi.sum()
    n = 200000
    u = (np.arange(n) + 0.5) / n
    counts = np.bincount([om.inverse_cdf(pi, x) for x in u], minlength=7)
    assert np.allclose(counts / n, pi, atol=2.0 / n)


def test_mixture_is_weighted_sum():
    rng = np.random.default_rng(2)
    pis = [rng.dirichlet(np.ones(11)) for _ in range(4)]
    p = om.exit_probs([0.2, 0.7, 0.4, 1.0])
    mix = om.mixture(pis, p)
    assert abs(mix.sum() - 1.0) < 1e-12
    for i in range(11):
        assert abs(mix[i] - sum(p[k] * pis[k][i] for k in range(4))) < 1e-15


def test_sampled_tokens_follow_pi_mix(weights_dir):
    """Tiny vocabulary (V = 16), one fixed context: tokens drawn by walking the gates
    and inverting the chosen exit's CDF follow pi_mix; exits follow p_k."""
    m = tiny_variant(vocab=16, init_std=0.05, gate_bias=BIAS_MASS_40_25_20_15)
    M = om.OracleModel(cached_weights(m, weights_dir))
    prompt = [3, 9, 1, 14, 7]
    outs, _ = om.generate(M, prompt, np.full((1, 4), 0.5, np.float32))
    o = outs[0]
    mix = om.mixture(o.pis, o.p)
    # the exit distributions differ, so using a single exit would be detected
    assert max(np.abs(o.pis[0] - o.pis[3])) > 0.02
    rng = np.random.default_rng(123)
    n = 200000
    U = rng.random((n, 4))
    toks = np.empty(n, dtype=np.int64)
    exits = np.empty(n, dtype=np.int64)
    for i in range(n):
        e = om.walk_gates(o.w, U[i])
        exits[i] = e
        toks[i] = om.inverse_cdf(o.pis[e], U[i, 3])
    tc = np.bincount(toks, minlength=16)
    ec = np.bincount(exits, minlength=4)
    assert stats.chisquare(tc, mix * n).pvalue > 1e-3
    assert stats.chisquare(ec, np.asarray(o.p) * n).pvalue > 1e-3
    # and it rejects the last exit's distribution alone
    assert stats.chisquare(tc, o.pis[3] * n).pvalue < 1e-6
