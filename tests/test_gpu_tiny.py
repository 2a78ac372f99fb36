"""Parity of the HIP path with the oracle on the tiny fp32 model (64-token prompt,
64 decode steps): tokens and exits bit-exact (near-boundary draws counted), logits
and every layer's KV within 1e-4 relative."""
import math

import numpy as np
import pytest

from oracle import model as om
from synth import TINY, cached_weights, prompts, tiny_variant, uniforms, workload
from tests.parity import StepCheck, check_step, rel, run_forced

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_exits_transformer_amd.lib as L
    L.library()
    return L


def _kv_check(h, lib, st, n, tol=TOL):
    worst = 0.0
    for l in range(st.kv.K.shape[0]):
        k, v = lib.nv_debug_kv(h, 0, l, 0, n)
        worst = max(worst, rel(k, st.kv.K[l, :n]), rel(v, st.kv.V[l, :n]))
    assert worst < tol, f"KV relative error {worst}"
    return worst


def test_tiny_workload_forced_parity(lib, weights_dir):
    w = workload("T")
    path = cached_weights(TINY, weights_dir)
    M = om.OracleModel(path)
    prompt = prompts(w)[0]
    U = uniforms(w)[:, 0, :]
    outs, st = om.generate(M, prompt, U, max_ctx=w.max_ctx)
    h = lib.nv_load(path, 1, w.max_ctx)
    try:
        lib.nv_prefill(h, 0, prompt)
        recs = run_forced(h, lib, outs)
        res = StepCheck()
        for t, (o, (tok, ex, lg, gw)) in enumerate(zip(outs, recs)):
            check_step(t, o, tok, ex, lg, gw, res)
        print(f"\nT: steps {res.steps} exits equal {res.exit_equal} tokens equal {res.token_equal} "
              f"near-boundary {res.near_boundary} max logit rel {res.max_logit_rel:.2e} "
              f"max gate abs {res.max_gate_abs:.2e}")
        assert not res.unexplained, res.unexplained
        assert res.max_logit_rel < TOL
        assert res.max_gate_abs < 1e-6
        # some steps exited early, so deferral really ran
        exits = [r[1] for r in recs]
        assert min(exits) == 1 and max(exits) == 4
        lib.nv_flush(h, -1)
        n, f = lib.nv_debug_frontiers(h, 0)
        assert n == len(prompt) - 1 + len(U) and list(f) == [n] * 4
        _kv_check(h, lib, st, n)
    finally:
        lib.nv_free(h)


def test_tiny_free_run_matches_oracle(lib, weights_dir):
    """Without teacher forcing the device's own samples reproduce the oracle's sequence."""
    w = workload("T")
    path = cached_weights(TINY, weights_dir)
    M = om.OracleModel(path)
    prompt = prompts(w)[0]
    U = uniforms(w)[:32, 0, :]
    outs, _ = om.generate(M, prompt, U, max_ctx=w.max_ctx, all_heads=False)
    h = lib.nv_load(path, 1, w.max_ctx)
    try:
        lib.nv_prefill(h, 0, prompt)
        for t, o in enumerate(outs):
            tok, ex = lib.nv_step(h, U[t:t + 1])
            d = om.boundary_distances(o, int(tok[0]), int(ex[0]))
            if int(tok[0]) != o.token or int(ex[0]) != o.exit:
                assert min(d["gates"] + [d["token"] or 1.0]) < 1e-5, f"step {t} diverged"
                break
    finally:
        lib.nv_free(h)


STOP, GO = 0.0, np.float32(1.0 - 2.0 ** -24)


def _forced_u(pattern, rng):
    U = rng.random((len(pattern), 4)).astype(np.float32)
    for t, e in enumerate(pattern):
        U[t, :3] = GO
        if e < 4:
            U[t, e - 1] = STOP
    return U


@pytest.mark.parametrize("pattern", [
    [1] * 20 + [4] + [2] * 5 + [4],          # long chunks: 21 rows at segments 2..4
    [1, 2, 3, 4] * 6,
    [3] * 9 + [1] * 40 + [2, 4],             # a 41-row chunk at segment 2 (several row blocks)
])
def test_tiny_forced_exit_patterns(lib, weights_dir, pattern):
    path = cached_weights(TINY, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(len(pattern))
    prompt = rng.integers(0, M.V, size=17)
    U = _forced_u(pattern, rng)
    outs, st = om.generate(M, prompt, U, max_ctx=128)
    h = lib.nv_load(path, 1, 128)
    try:
        lib.nv_prefill(h, 0, prompt)
        recs = run_forced(h, lib, outs)
        res = StepCheck()
        for t, (o, (tok, ex, lg, gw)) in enumerate(zip(outs, recs)):
            assert ex == pattern[t]
            check_step(t, o, tok, ex, lg, gw, res)
        assert not res.unexplained, res.unexplained
        assert res.max_logit_rel < TOL
        lib.nv_flush(h, 0)
        lib.nv_flush(h, 0)                     # second flush is a no-op
        _kv_check(h, lib, st, len(prompt) - 1 + len(U))
    finally:
        lib.nv_free(h)


def test_tiny_closed_gates_is_standard_decode(lib, weights_dir):
    """All intermediate biases at -inf: every token exits at 4 and the device matches the
    oracle (itself pinned to a textbook transformer)."""
    m = tiny_variant(gate_bias=(-math.inf,) * 3)
    path = cached_weights(m, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(11)
    prompt = rng.integers(0, M.V, size=9)
    U = rng.random((12, 4)).astype(np.float32)
    U[:, :3] = 0.0
    outs, st = om.generate(M, prompt, U, max_ctx=32)
    h = lib.nv_load(path, 1, 32)
    try:
        lib.nv_prefill(h, 0, prompt)
        recs = run_forced(h, lib, outs)
        for (tok, ex, lg, gw), o in zip(recs, outs):
            assert ex == 4
            assert gw[0] == 0.0 and gw[1] == 0.0 and gw[2] == 0.0 and gw[3] == 1.0
            assert rel(lg, o.logits[3]) < TOL
        n, f = lib.nv_debug_frontiers(h, 0)
        assert list(f) == [n] * 4               # nothing deferred
        _kv_check(h, lib, st, n)
    finally:
        lib.nv_free(h)


def test_tiny_prompt_of_one_token(lib, weights_dir):
    path = cached_weights(TINY, weights_dir)
    M = om.OracleModel(path)
    U = np.array([[0.3, 0.9, 0.2, 0.61], [0.95, 0.1, 0.5, 0.05]], np.float32)
    outs, st = om.generate(M, [42], U, max_ctx=8)
    h = lib.nv_load(path, 1, 8)
    try:
        lib.nv_prefill(h, 0, [42])
        recs = run_forced(h, lib, outs)
        res = StepCheck()
        for t, (o, (tok, ex, lg, gw)) in enumerate(zip(outs, recs)):
            check_step(t, o, tok, ex, lg, gw, res)
        assert not res.unexplained
        lib.nv_flush(h)
        _kv_check(h, lib, st, 2)
    finally:
        lib.nv_free(h)


def test_tiny_error_paths(lib, weights_dir):
    path = cached_weights(TINY, weights_dir)
    h = lib.nv_load(path, 2, 8)
    try:
        with pytest.raises(lib.NvError) as e:
            lib.nv_step(h, np.zeros((1, 4), np.float32))
        assert e.value.status == lib.NV_ESTATE
        with pytest.raises(lib.NvError) as e:
            lib.nv_prefill(h, 0, [1, 2, 512])
        assert e.value.status == lib.NV_EINVAL
        with pytest.raises(lib.NvError) as e:
            lib.nv_prefill(h, 2, [1])
        assert e.value.status == lib.NV_EINVAL
        with pytest.raises(lib.NvError) as e:
            lib.nv_prefill(h, 0, list(range(9)))
        assert e.value.status == lib.NV_ECAPACITY
        lib.nv_prefill(h, 1, [3, 4])
        with pytest.raises(lib.NvError) as e:      # sequence 0 missing: not contiguous from 0
            lib.nv_step(h, np.zeros((2, 4), np.float32))
        assert e.value.status == lib.NV_ESTATE
        lib.nv_prefill(h, 0, [5, 6, 7, 8, 9, 10, 11])
        for bad in (1.0, -0.1, np.nan):
            u = np.full((2, 4), 0.5, np.float32)
            u[1, 2] = bad
            with pytest.raises(lib.NvError) as e:
                lib.nv_step(h, u)
            assert e.value.status == lib.NV_EINVAL
        lib.nv_step(h, np.full((2, 4), 0.5, np.float32))   # sequence 0: position 6 consumed
        lib.nv_step(h, np.full((2, 4), 0.5, np.float32))   # position 7 = max_ctx - 1 consumed
        with pytest.raises(lib.NvError) as e:
            lib.nv_step(h, np.full((2, 4), 0.5, np.float32))
        assert e.value.status == lib.NV_ECAPACITY
    finally:
        lib.nv_free(h)
