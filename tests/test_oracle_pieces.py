"""Pins of the oracle's layer arithmetic against library routines and the
strict-generalisation property (zero routing mass on intermediate exits gives a
standard transformer exactly)."""
import math
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model as om
from synth import TINY, cached_weights, tensor_specs, tiny_variant
from synth.weights import _tensor_values, f32_to_bf16_bits
from tests import textbook


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 96))
    g = rng.standard_normal(96)
    ref = F.rms_norm(torch.as_tensor(x), (96,), weight=torch.as_tensor(g), eps=1e-5).numpy()
    assert rel(om.rmsnorm(x, g, 1e-5), ref) < 1e-14


def test_silu_softmax_match_torch():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 33)) * 4
    assert rel(om.silu(x), F.silu(torch.as_tensor(x)).numpy()) < 1e-14
    assert rel(om.softmax(x), torch.softmax(torch.as_tensor(x), -1).numpy()) < 1e-14


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 3, 32))
    pos = rng.integers(0, 5000, size=9)
    ref = textbook.rope_complex(torch.as_tensor(x).transpose(0, 1), pos, 1e4).transpose(0, 1).numpy()
    assert rel(om.rope(x, pos, 1e4), ref) < 1e-13


def test_rope_relative_position_invariance():
    # <rope(q, m), rope(k, n)> depends only on m - n
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    dots = []
    for m, n in [(10, 3), (107, 100), (5007, 5000)]:
        a = om.rope(q, np.array([m]), 1e4)
        b = om.rope(k, np.array([n]), 1e4)
        dots.append(float(np.sum(a * b)))
    assert max(dots) - min(dots) < 1e-10 * max(1.0, abs(dots[0]))
    # position 0 is the identity
    assert np.array_equal(om.rope(q, np.array([0]), 1e4), q)


def test_causal_attention_matches_sdpa():
    rng = np.random.default_rng(9)
    n, H, hd = 23, 3, 16
    q = rng.standard_normal((n, H, hd))
    K = rng.standard_normal((n, H, hd))
    V = rng.standard_normal((n, H, hd))
    out = om.causal_attention(q, K, V, np.arange(n))
    t = lambda a: torch.as_tensor(a).transpose(0, 1)[None]
    ref = F.scaled_dot_product_attention(t(q), t(K), t(V), is_causal=True)[0].transpose(0, 1).numpy()
    assert rel(out, ref) < 1e-13
    # a chunk of rows at positions 15..22 over the full cache gives the same rows
    out2 = om.causal_attention(q[15:], K, V, np.arange(15, n))
    assert rel(out2, ref[15:]) < 1e-13


def test_reader_reproduces_written_values(tiny_path):
    M = om.OracleModel(tiny_path)
    specs = tensor_specs(TINY)
    got = {"embed": M.embed, "l3.wk": M.wk[3], "l7.wd": M.wd[7], "l0.attn_norm": M.attn_norm[0],
           "x2.gate_w": M.gate_w[2], "x3.gate_w": M.gate_w[3], "x1.head": M.head[1]}
    for i, (name, shape, kind) in enumerate(specs):
        if name in got:
            want = _tensor_values(TINY, i, shape, kind).reshape(shape)
            assert np.array_equal(np.asarray(got[name], np.float32), want), name
    assert M.exit_layers == [2, 4, 6, 8]
    assert M.gate_bias[3] == math.inf


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5e-3, 3.0e38], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    ref = torch.as_tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(back, ref)


def test_exit4_is_standard_transformer(weights_dir):
    """Strict generalisation: with every intermediate bias at -inf, p = (0,0,0,1)
    exactly and the decode logits equal a textbook LLaMA forward."""
    m = tiny_variant(gate_bias=(-math.inf,) * 3)
    M = om.OracleModel(cached_weights(m, weights_dir))
    rng = np.random.default_rng(3)
    prompt = rng.integers(0, m.vocab, size=12)
    U = rng.random((6, 4)).astype(np.float32)
    U[:, :3] = 0.0                      # u = 0 stops at any gate with w > 0
    outs, st = om.generate(M, prompt, U)
    for o in outs:
        assert o.exit == 4
        assert o.p == [0.0, 0.0, 0.0, 1.0]
    seq = list(prompt) + [o.token for o in outs[:-1]]
    hs, logits, Ks, Vs = textbook.forward(M, seq)
    P = len(prompt) - 1
    for t, o in enumerate(outs):
        for k in range(4):
            assert rel(o.logits[k], logits[k][P + t]) < 1e-11
            assert rel(o.h[k], hs[k][P + t]) < 1e-11
    n = len(seq)
    for l in range(M.L):
        assert rel(st.kv.K[l, :n], Ks[l]) < 1e-11
        assert rel(st.kv.V[l, :n], Vs[l]) < 1e-11


def test_prefill_chunk_equals_token_by_token(tiny_path):
    """A causal chunk through prefill gives the same KV as one token at a time."""
    M = om.OracleModel(tiny_path)
    rng = np.random.default_rng(4)
    toks = rng.integers(0, M.V, size=10)
    a = om.new_state(M, 16)
    om.prefill(M, a, toks)
    b = om.new_state(M, 16)
    for t in toks:
        om.prefill(M, b, [t])
    assert rel(a.kv.K[:, :10], b.kv.K[:, :10]) < 1e-12
    assert rel(a.kv.V[:, :10], b.kv.V[:, :10]) < 1e-12
