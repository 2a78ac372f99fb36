"""Parity of the HIP path with the oracle in the pages' own exit and router forms: every
exit reads the one final RMSNorm + LM head through a residual adapter MLP, and the
halting gate is a router MLP.

- Tiny fp32 model (adapter bottleneck 16, router hidden 8): a 64-token prompt and 48
  decode steps with free draws, and forced exit patterns with deferred chunks; tokens
  and exits exact (near-boundary draws counted), logits and every layer's KV within
  1e-4 relative, gates within 1e-6.
- Four sequences decoding together, stopping at different exits in the same step (one
  shared head pass over all of them, grouped by exit for the adapters); each sequence
  against its own oracle run.
- The 1.5B model in this form (workload E, bf16, bottleneck 192, router hidden 64) on
  sampled steps: logits and sampled layers' KV within 2e-2."""
import numpy as np
import pytest

from oracle import model as om
from synth import cached_weights, prompts, tiny_variant, uniforms, workload
from tests.parity import StepCheck, check_step, decoded_kv_report, hidden_rows_worst, rel, run_forced

pytestmark = pytest.mark.gpu

FORMS = tiny_variant(head="shared", adapter_dim=16, router="mlp", router_dim=8)
STOP, GO = 0.0, np.float32(1.0 - 2.0 ** -24)


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_exits_transformer_amd.lib as L
    L.library()
    return L


def _forced_u(pattern, rng):
    U = rng.random((len(pattern), 4)).astype(np.float32)
    for t, e in enumerate(pattern):
        if e == 0:
            continue
        U[t, :3] = GO
        if e < 4:
            U[t, e - 1] = STOP
    return U


@pytest.mark.parametrize("pattern", [
    [0] * 48,
    [1, 1, 2, 4, 1, 3, 3, 4, 2, 1, 1, 1, 4, 2, 2, 3, 4],
])
def test_forms_tiny_parity(lib, weights_dir, pattern):
    path = cached_weights(FORMS, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(len(pattern))
    prompt = rng.integers(0, M.V, size=64)
    U = _forced_u(pattern, rng)
    max_ctx = len(prompt) + len(pattern)
    outs, st = om.generate(M, prompt, U, max_ctx=max_ctx)
    h = lib.nv_load(path, 1, max_ctx)
    try:
        assert h.cfg.head_form == 1 and h.cfg.router_form == 1
        assert h.cfg.adapter_dim == 16 and h.cfg.router_dim == 8
        lib.nv_prefill(h, 0, prompt)
        recs = run_forced(h, lib, outs)
        res = StepCheck()
        for t, (o, (tok, ex, lg, gw)) in enumerate(zip(outs, recs)):
            if pattern[t]:
                assert ex == pattern[t]
            check_step(t, o, tok, ex, lg, gw, res)
        print("\nforms tiny:", res.summary())
        assert not res.unexplained, res.unexplained
        assert res.max_logit_rel < 1e-4
        assert res.max_gate_abs < 1e-6
        exits = [r[1] for r in recs]
        assert min(exits) == 1 and max(exits) == 4
        lib.nv_flush(h)
        n = len(prompt) - 1 + len(pattern)
        worst = 0.0
        for l in range(M.L):
            k, v = lib.nv_debug_kv(h, 0, l, 0, n)
            worst = max(worst, rel(k, st.kv.K[l, :n]), rel(v, st.kv.V[l, :n]))
        assert worst < 1e-4, worst
    finally:
        lib.nv_free(h)


def test_forms_tiny_batch_mixed_exits(lib, weights_dir):
    """Four sequences; at each step they stop at different exits (forced), so one shared
    head pass covers several exits' adapters."""
    path = cached_weights(FORMS, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(44)
    B, steps = 4, 12
    pats = [[(t + i) % 4 + 1 for t in range(steps)] for i in range(B)]
    ps = [rng.integers(0, M.V, size=20 + 7 * i) for i in range(B)]
    Us = [_forced_u(p, rng) for p in pats]
    runs = [om.generate(M, ps[i], Us[i], max_ctx=len(ps[i]) + steps) for i in range(B)]
    h = lib.nv_load(path, B, max(len(p) for p in ps) + steps)
    try:
        for i in range(B):
            lib.nv_prefill(h, i, ps[i])
        res = [StepCheck() for _ in range(B)]
        for t in range(steps):
            U = np.stack([Us[i][t] for i in range(B)])
            nxt = np.array([runs[i][0][t].token for i in range(B)], np.int32)
            tok, ex = lib.nv_step_forced(h, U, nxt)
            assert sorted(int(e) for e in ex) == [1, 2, 3, 4]
            for i in range(B):
                o = runs[i][0][t]
                check_step(t, o, int(tok[i]), int(ex[i]), lib.nv_debug_logits(h, i), lib.nv_debug_gates(h, i),
                           res[i])
        for i in range(B):
            print(f"\nforms batch seq {i}:", res[i].summary())
            assert not res[i].unexplained, res[i].unexplained
            assert res[i].max_logit_rel < 1e-4
        lib.nv_flush(h)
        for i in range(B):
            n = len(ps[i]) - 1 + steps
            st = runs[i][1]
            for l in (0, 3, 7):
                k, v = lib.nv_debug_kv(h, i, l, 0, n)
                assert rel(k, st.kv.K[l, :n]) < 1e-4 and rel(v, st.kv.V[l, :n]) < 1e-4
    finally:
        lib.nv_free(h)


def test_workload_E_sampled(lib, weights_dir):
    w = workload("E")
    path = cached_weights(w.model, weights_dir)
    M = om.OracleModel(path)
    prompt = prompts(w)[0]
    U = uniforms(w)[:8, 0, :].copy()
    for t, e in zip(range(4, 8), [1, 2, 1, 4]):
        U[t, :3] = GO
        if e < 4:
            U[t, e - 1] = STOP
    max_ctx = len(prompt) + len(U)
    outs, st = om.generate(M, prompt, U, max_ctx=max_ctx)
    h = lib.nv_load(path, 1, max_ctx)
    try:
        lib.nv_prefill(h, 0, prompt)
        recs = run_forced(h, lib, outs)
        res = StepCheck()
        for t, (o, (tok, ex, lg, gw)) in enumerate(zip(outs, recs)):
            check_step(t, o, tok, ex, lg, gw, res, logit_band=True)
        print("\nE:", end=" ")
        exits = [r[1] for r in recs]
        assert exits[4:] == [1, 2, 1, 4]
        res.finish(2e-2, max_logit_explained=None)   # V = 32000: token intervals ~3e-5
        lib.nv_flush(h)
        P = len(prompt) - 1
        rep = decoded_kv_report(lib, h, 0, st, (0, 11, 12, 23, 24, 47), P, exits, w.model.seg_layers)
        hid = hidden_rows_worst(lib, h, 0, outs, P)
        print("E per-row KV worst", {k: f"{v:.2e}" for k, v in rep.items()}, f"hidden rows {hid:.2e}")
        assert max(rep.values()) < 2e-2 and hid < 2e-2
    finally:
        lib.nv_free(h)
