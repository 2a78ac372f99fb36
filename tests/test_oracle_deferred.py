"""Pins of the deferred schedule: deferring the layers above the exit and running
them later batched with following tokens gives the same tokens, exits and
per-layer KV as sequential full-depth decoding."""
import itertools

import numpy as np
import pytest

from oracle import deferred as od
from oracle import model as om
from synth import TINY, cached_weights, tiny_variant, uniforms, workload
from synth.configs import BIAS_MASS_40_25_20_15

STOP = 0.0                           # u = 0 stops at any gate with w > 0
GO = np.float32(1.0 - 2.0 ** -24)    # u just below 1 passes any gate with w < 1 - 2^-24


def forced_uniforms(pattern, u4):
    U = np.empty((len(pattern), 4), np.float32)
    for t, e in enumerate(pattern):
        U[t, :3] = GO
        if e < 4:
            U[t, e - 1] = STOP
        U[t, 3] = u4[t]
    return U


def test_deferred_equals_sequential_config_T(tiny_path):
    M = om.OracleModel(tiny_path)
    w = workload("T")
    from synth import prompts
    prompt = prompts(w)[0]
    U = uniforms(w)[:40, 0, :]
    seq, st = om.generate(M, prompt, U, all_heads=False)
    run = od.generate_deferred(M, prompt, U, order="row")
    assert run.tokens == [o.token for o in seq]
    assert run.exits == [o.exit for o in seq]
    n = len(prompt) - 1 + len(U)
    assert np.array_equal(run.state.kv.K[:, :n], st.kv.K[:, :n])
    assert np.array_equal(run.state.kv.V[:, :n], st.kv.V[:, :n])
    assert run.state.kv.written[:, :n].all()
    # some tokens really were deferred
    assert max(max(r) for r in run.chunk_rows) > 1
    # the batched (layer-at-a-time) chunk order agrees to rounding
    run2 = od.generate_deferred(M, prompt, U, order="layer")
    assert run2.tokens == run.tokens and run2.exits == run.exits
    assert np.max(np.abs(run2.state.kv.K[:, :n] - st.kv.K[:, :n])) < 1e-12


def test_deferred_layers_really_pending_before_flush(tiny_path):
    M = om.OracleModel(tiny_path)
    prompt = [5, 6, 7]
    pattern = [1, 1, 2, 1]
    U = forced_uniforms(pattern, [0.5] * 4)
    run = od.generate_deferred(M, prompt, U, flush=False)
    assert run.exits == pattern
    P = len(prompt) - 1
    # positions P..P+3 exited at 1,1,2,1: segment-2 frontier stops at P+3 (the exit-2 step),
    # segment 3/4 frontiers never move
    assert run.frontiers[-1] == [P + 4, P + 3, P, P]
    written = run.state.kv.written
    seg = lambda s: list(M.segment_layers(s))
    assert written[seg(0), P:P + 4].all()
    assert written[seg(1), P:P + 3].all() and not written[seg(1), P + 3].any()
    assert not written[seg(2) + seg(3), P:P + 4].any()


def _micro():
    return tiny_variant(n_layers=4, d_model=32, n_heads=2, head_dim=16, ffn=48, vocab=32,
                        gate_bias=BIAS_MASS_40_25_20_15)


def test_brute_force_forced_exit_patterns(weights_dir):
    """Every exit pattern over 5 steps (4^5 = 1024): tokens, exits, chunk sizes and
    every layer's KV after flush equal sequential decoding bit for bit."""
    M = om.OracleModel(cached_weights(_micro(), weights_dir))
    prompt = [4, 17]
    P = len(prompt) - 1
    u4 = [0.11, 0.52, 0.93, 0.37, 0.68]
    for pattern in itertools.product([1, 2, 3, 4], repeat=5):
        U = forced_uniforms(pattern, u4)
        seq, st = om.generate(M, prompt, U, all_heads=False)
        run = od.generate_deferred(M, prompt, U)
        assert [o.exit for o in seq] == list(pattern)
        assert run.exits == list(pattern)
        assert run.tokens == [o.token for o in seq]
        n = P + 5
        assert np.array_equal(run.state.kv.K[:, :n], st.kv.K[:, :n])
        assert np.array_equal(run.state.kv.V[:, :n], st.kv.V[:, :n])
        # chunk rows at segment s = 1 + steps since the last token that reached s
        for t, e in enumerate(pattern):
            for s in range(e):
                last = max([j for j in range(t) if pattern[j] > s], default=-1)
                assert run.chunk_rows[t][s] == t - last
