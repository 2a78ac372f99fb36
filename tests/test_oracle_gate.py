"""Pins of the oracle's linear router at finite logits.

The router output of exit k is w_k = sigmoid(g_k . h^(l_k) + b_k) on the residual
stream after the exit's last layer, and the last exit's w is 1 (gist.science summary,
section 2 "Methodik", part "Architektur": router output w_k, equation for p_k).  The
values below come from torch's sigmoid and dot product on hand-built vectors, and, for
a decode step of the tiny model, from the textbook forward's hidden states and the
weight generator's own gate vectors, never from the oracle's arithmetic.
"""
import math
from types import SimpleNamespace

import numpy as np
import torch

from oracle import model as om
from synth import TINY, cached_weights, tensor_specs
from synth.weights import _tensor_values
from tests import textbook


def _linear_router(gate_w, bias):
    return SimpleNamespace(router_mlp=False, n_exits=len(gate_w), gate_w=gate_w, gate_bias=bias)


def test_linear_gate_against_torch_on_hand_built_vectors():
    d = 24
    # distinct gate vectors: one is a unit vector, one a ramp, one alternating; the dot
    # products with h differ in sign and size, so a dropped dot term, a wrong sign or a
    # neighbouring exit's vector changes the result
    h = np.array([(-1.0) ** i * (0.25 + 0.125 * i) for i in range(d)])
    g = [np.zeros(d), np.linspace(-0.3, 0.5, d), np.array([0.2 if i % 2 else -0.1 for i in range(d)]),
         np.zeros(d)]
    g[0][5] = 1.3
    b = [0.7, -1.1, 0.4, math.inf]
    M = _linear_router(g, b)
    want = [float(torch.sigmoid(torch.dot(torch.as_tensor(g[k]), torch.as_tensor(h)) + b[k])) for k in range(3)]
    # the three logits are far apart, so each gate's value identifies its vector
    assert min(abs(want[i] - want[j]) for i in range(3) for j in range(i)) > 0.05
    for k in range(3):
        got = om.gate(M, k, h)
        assert abs(got - want[k]) < 1e-15, (k, got, want[k])
        # the dot term matters: the gate differs from sigmoid(b_k) alone
        assert abs(got - 1.0 / (1.0 + math.exp(-b[k]))) > 1e-2
    assert om.gate(M, 3, h) == 1.0


def test_linear_gate_large_logits_saturate_without_overflow():
    d = 4
    h = np.array([300.0, -200.0, 100.0, 50.0])
    g = [np.array([1.0, 0.0, 0.0, 0.0]), np.array([0.0, 1.0, 0.0, 0.0]), np.array([0.0, 0.0, 0.01, 0.0]),
         np.zeros(d)]
    M = _linear_router(g, [0.0, 0.0, -0.5, math.inf])
    assert om.gate(M, 0, h) == 1.0                   # sigmoid(300) rounds to 1
    assert 0.0 < om.gate(M, 1, h) < 1e-80            # sigmoid(-200) = e^-200 / (1 + e^-200)
    assert abs(om.gate(M, 1, h) - math.exp(-200.0)) < 1e-95
    assert abs(om.gate(M, 2, h) - float(torch.sigmoid(torch.tensor(0.5, dtype=torch.float64)))) < 1e-15


def test_decode_step_gates_equal_sigmoid_of_textbook_hidden_states(tiny_path):
    """One decode step of the tiny model: w_k of the oracle equals sigmoid(g_k . h_k + b_k)
    with h_k the textbook forward's hidden state after layer l_k at the decoded position
    and g_k drawn again from the weight generator."""
    M = om.OracleModel(tiny_path)
    specs = tensor_specs(TINY)
    gvec = {}
    for i, (name, shape, kind) in enumerate(specs):
        if name.endswith(".gate_w"):
            gvec[int(name[1])] = _tensor_values(TINY, i, shape, kind).astype(np.float64)
    rng = np.random.default_rng(11)
    prompt = rng.integers(0, TINY.vocab, size=9)
    U = np.full((3, 4), 0.999, np.float32)           # walk to the last exit, all heads
    outs, _ = om.generate(M, prompt, U)
    seq = list(prompt) + [o.token for o in outs[:-1]]
    hs, _, _, _ = textbook.forward(M, seq)
    P = len(prompt) - 1
    for t, o in enumerate(outs):
        for k in range(3):
            h = torch.as_tensor(hs[k][P + t])
            # the weights header stores each bias as float32
            b = float(np.float32(TINY.gate_bias[k]))
            z = torch.dot(torch.as_tensor(gvec[k]), h) + b
            want = float(torch.sigmoid(z))
            assert abs(o.w[k] - want) < 1e-12, (t, k, o.w[k], want)
            # the linear term moves the gate by far more than the tolerance above, so a
            # dropped dot term or another exit's vector would fail the comparison
            assert abs(float(z) - b) > 1e-5
        assert o.w[3] == 1.0
