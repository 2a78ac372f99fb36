"""Pins of the oracle's forward-only mixture objective (L_mix, L_compute): with every
intermediate gate closed it is the standard cross-entropy of the final head and depth
1; with gate 1 always open it is exit 1's cross-entropy and depth l_1 / L (both against
the textbook torch forward and torch's cross_entropy); Jensen's bounds hold per
position; and exp(-nll) equals the mixture the sampler draws from."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import model as om
from synth import cached_weights, tiny_variant
from tests import textbook

TOKENS = [5, 17, 300, 2, 99, 41, 7, 7, 250, 1, 64, 3]


def _ce(logits, tokens):
    z = torch.as_tensor(np.asarray(logits[:-1]))
    y = torch.as_tensor(np.asarray(tokens[1:], dtype=np.int64))
    return float(F.cross_entropy(z, y))


def test_closed_gates_give_final_head_cross_entropy(weights_dir):
    M = om.OracleModel(cached_weights(tiny_variant(gate_bias=(-math.inf,) * 3), weights_dir))
    out = om.mixture_loss(M, TOKENS, beta=0.5)
    _, logits, _, _ = textbook.forward(M, TOKENS)
    assert abs(out.L_mix - _ce(logits[3], TOKENS)) < 1e-10
    assert out.L_compute == 1.0
    assert abs(out.L_total - (out.L_mix + 0.5)) < 1e-12


def test_open_first_gate_gives_exit1_cross_entropy(weights_dir):
    M = om.OracleModel(cached_weights(tiny_variant(gate_bias=(math.inf, 0.0, 0.0)), weights_dir))
    out = om.mixture_loss(M, TOKENS)
    _, logits, _, _ = textbook.forward(M, TOKENS)
    assert abs(out.L_mix - _ce(logits[0], TOKENS)) < 1e-10
    assert abs(out.L_compute - M.exit_layers[0] / M.L) < 1e-15


def test_jensen_bounds_and_sampler_mixture(weights_dir):
    for m in (tiny_variant(), tiny_variant(head="shared", adapter_dim=16, router="mlp", router_dim=8)):
        M = om.OracleModel(cached_weights(m, weights_dir))
        out = om.mixture_loss(M, TOKENS)
        for i in range(len(TOKENS) - 1):
            p = np.asarray(om.exit_probs(list(out.w[i])))
            # -log sum p pi <= sum p (-log pi), and >= -log max pi
            assert out.nll_mix[i] <= float(np.sum(p * -out.logp[i])) + 1e-12
            assert out.nll_mix[i] >= -float(np.max(out.logp[i])) - 1e-12
        # the same mixture the decode step forms for sampling
        st = om.new_state(M, len(TOKENS))
        om.prefill(M, st, TOKENS[:5])
        o = om.decode_step(M, st, TOKENS[5], [0.5] * 4)
        mix = om.mixture(o.pis, o.p)
        assert abs(math.exp(-out.nll_mix[5]) - mix[TOKENS[6]]) < 1e-12
        assert np.allclose(out.w[5], o.w, rtol=0, atol=1e-14)
