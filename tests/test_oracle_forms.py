"""Pins of the oracle's second parametrisation (the pages' own exit and router forms):
every exit reads the one final norm + LM head through a residual adapter MLP, and the
halting gate is a router MLP.

Pinned by: the weights-file round trip; closed forms of special cases (a router whose
output layer is zero is its bias; a router whose first layer is zero has a constant
hidden layer; an adapter with one nonzero weight in each matrix adds one scaled SiLU
term); the textbook LLaMA forward where the adapters are the identity (all exits then
read the final head); sampling frequencies against pi_mix and p_k; and deferral
exactness (tokens, exits and KV bit-identical to sequential decoding)."""
import math

import numpy as np
from scipy import stats

from oracle import deferred as od
from oracle import model as om
from synth import cached_weights, tensor_specs, tiny_variant
from synth.configs import BIAS_MASS_40_25_20_15
from synth.weights import _tensor_values
from tests import textbook

FORMS = tiny_variant(head="shared", adapter_dim=16, router="mlp", router_dim=8)


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_reader_reproduces_written_values_forms(weights_dir):
    M = om.OracleModel(cached_weights(FORMS, weights_dir))
    assert M.shared_head and M.router_mlp and M.adapter_dim == 16 and M.router_dim == 8
    specs = tensor_specs(FORMS)
    got = {"x0.router_w1": M.router_w1[0], "x1.router_b1": M.router_b1[1], "x2.router_w2": M.router_w2[2],
           "x3.router_w1": M.router_w1[3], "x1.adapter_down": M.adapter_down[1], "x2.adapter_up": M.adapter_up[2],
           "final_norm": M.final_norm, "head": M.head[0]}
    for i, (name, shape, kind) in enumerate(specs):
        if name in got:
            want = _tensor_values(FORMS, i, shape, kind).reshape(shape)
            assert np.array_equal(np.asarray(got[name], np.float32), want), name
    assert not np.any(M.router_w1[3]) and not np.any(M.router_w2[3]) and not np.any(M.router_b1[0])
    # one shared head and one final norm for every exit
    assert all(h is M.head[0] for h in M.head) and len(M.adapter_down) == 3


def test_router_mlp_closed_forms(weights_dir):
    M = om.OracleModel(cached_weights(FORMS, weights_dir))
    rng = np.random.default_rng(11)
    h = rng.standard_normal(M.d) * 3.0
    # output layer zero: the router is its bias
    M.router_w2[0][:] = 0.0
    assert abs(om.gate(M, 0, h) - sig(M.gate_bias[0])) < 1e-15
    # first layer zero, hidden bias c: every hidden unit is silu(c)
    c = 0.7
    M.router_w1[1][:] = 0.0
    M.router_b1[1][:] = c
    v = M.router_w2[1]
    z = (c / (1.0 + math.exp(-c))) * float(np.sum(v)) + M.gate_bias[1]
    assert abs(om.gate(M, 1, h) - sig(z)) < 1e-13
    # one weight in each layer: hidden unit j sees a * h[i]
    M.router_w1[2][:] = 0.0
    M.router_b1[2][:] = 0.0
    M.router_w2[2][:] = 0.0
    a, wj = 0.13, -2.5
    M.router_w1[2][5, 17] = a
    M.router_w2[2][5] = wj
    t = a * h[17]
    z = wj * t / (1.0 + math.exp(-t)) + M.gate_bias[2]
    assert abs(om.gate(M, 2, h) - sig(z)) < 1e-13
    # the last exit always stops
    assert om.gate(M, 3, h) == 1.0


def test_adapter_closed_form(weights_dir):
    M = om.OracleModel(cached_weights(FORMS, weights_dir))
    rng = np.random.default_rng(12)
    h = rng.standard_normal(M.d) * 2.0
    Dn, Up = M.adapter_down[1], M.adapter_up[1]
    Dn[:] = 0.0
    Up[:] = 0.0
    Dn[3, 5] = 0.9
    Up[7, 3] = -1.3
    t = 0.9 * h[5]
    want = h.copy()
    want[7] += -1.3 * t / (1.0 + math.exp(-t))
    assert np.allclose(om.adapter(M, 1, h), want, rtol=0, atol=1e-14)
    assert np.array_equal(om.adapter(M, 3, h), h)
    # exit logits: the final norm and head applied to the adapter output
    z = om.head_logits(M, 1, h)
    x = want / math.sqrt(float(np.mean(want * want)) + M.eps) * M.final_norm
    assert np.allclose(z, M.head[1] @ x, rtol=1e-12, atol=1e-12)


def test_identity_adapters_give_textbook_logits(weights_dir):
    """With the adapters' output layers at zero every exit applies the final norm and
    head to its hidden state: the textbook forward's exit logits."""
    M = om.OracleModel(cached_weights(FORMS, weights_dir))
    for k in range(3):
        M.adapter_up[k][:] = 0.0
    tokens = [5, 17, 300, 2, 99, 41, 7]
    hs, logits, _, _ = textbook.forward(M, tokens)
    kv = om.KVCache(M, len(tokens))
    X = np.asarray(M.embed[np.asarray(tokens)], dtype=np.float64)
    pos = np.arange(len(tokens))
    k = 0
    for l in range(M.L):
        X = om.layer_rows(M, l, X, pos, kv)
        if l + 1 == M.exit_layers[k]:
            for i in range(len(tokens)):
                z = om.head_logits(M, k, X[i])
                assert np.allclose(z, logits[k][i], rtol=1e-10, atol=1e-10)
            k += 1


def test_sampled_tokens_follow_pi_mix_forms(weights_dir):
    m = tiny_variant(vocab=16, init_std=0.05, gate_bias=BIAS_MASS_40_25_20_15, head="shared", adapter_dim=16,
                     router="mlp", router_dim=8)
    M = om.OracleModel(cached_weights(m, weights_dir))
    outs, _ = om.generate(M, [3, 9, 1, 14, 7], np.full((1, 4), 0.5, np.float32))
    o = outs[0]
    mix = om.mixture(o.pis, o.p)
    assert max(np.abs(o.pis[0] - o.pis[3])) > 0.02
    rng = np.random.default_rng(321)
    n = 200000
    U = rng.random((n, 4))
    toks = np.empty(n, dtype=np.int64)
    exits = np.empty(n, dtype=np.int64)
    for i in range(n):
        e = om.walk_gates(o.w, U[i])
        exits[i] = e
        toks[i] = om.inverse_cdf(o.pis[e], U[i, 3])
    assert stats.chisquare(np.bincount(toks, minlength=16), mix * n).pvalue > 1e-3
    assert stats.chisquare(np.bincount(exits, minlength=4), np.asarray(o.p) * n).pvalue > 1e-3
    assert stats.chisquare(np.bincount(toks, minlength=16), o.pis[3] * n).pvalue < 1e-6


def test_deferred_equals_sequential_forms(weights_dir):
    M = om.OracleModel(cached_weights(FORMS, weights_dir))
    rng = np.random.default_rng(13)
    prompt = list(rng.integers(0, M.V, size=20))
    U = rng.random((40, 4)).astype(np.float32)
    seq, st = om.generate(M, prompt, U, all_heads=False)
    run = od.generate_deferred(M, prompt, U, order="row")
    assert run.tokens == [o.token for o in seq]
    assert run.exits == [o.exit for o in seq]
    n = len(prompt) - 1 + len(U)
    assert np.array_equal(run.state.kv.K[:, :n], st.kv.K[:, :n])
    assert np.array_equal(run.state.kv.V[:, :n], st.kv.V[:, :n])
    assert max(max(r) for r in run.chunk_rows) > 1
