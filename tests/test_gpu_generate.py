"""Batched decoding with sequences advancing through the segments independently
(nv_generate), against the oracle and against lock-step decoding.

- Lock-step policy vs nv_step (tiny fp32, own heads): the same launches, so tokens,
  exits, logits and KV are bit-identical.
- Greedy policy, both exit forms, five sequences in non-contiguous slots with prompts of
  3..60 tokens: every sequence's tokens and exits equal its own oracle run (free draws)
  until a draw within 1e-5 of an oracle decision boundary, if any; KV of every layer
  within 1e-4 after a flush.
- Continuous batching: sequences join (prefill into a free slot) and generate in
  changing subsets; each sequence's concatenated output equals its oracle run.
- Argument errors.
- The 1.5B batch-16 workload (prompts 256..1024), 8 tokens per sequence under the greedy
  policy: frontiers follow each sequence's exits; after a flush, the shortest-prompt
  sequence's KV at layer 0 and at seven deep layers equals the oracle's full-depth pass
  over the same tokens row by row (prompt rows, and decoded rows computed directly or in
  a later chunk), and equals a fresh device prefill of the same tokens (deferral is
  exact), within 2e-2."""
import numpy as np
import pytest

from oracle import model as om
from synth import cached_weights, prompts, tiny_variant, uniforms, workload
from tests.parity import decoded_kv_report, rel

pytestmark = pytest.mark.gpu

OWN = tiny_variant()
FORMS = tiny_variant(head="shared", adapter_dim=16, router="mlp", router_dim=8)
TOL = 2e-2


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_exits_transformer_amd.lib as L
    L.library()
    return L


def _check_free_run(M, prompt, U, tokens, exits, tag):
    """Tokens and exits equal the oracle's free run until a draw within 1e-5 of one of
    the oracle's decision boundaries; returns the oracle state and the equal prefix."""
    outs, st = om.generate(M, prompt, U, max_ctx=len(prompt) + len(U), all_heads=False)
    for t, o in enumerate(outs):
        if int(tokens[t]) != o.token or int(exits[t]) != o.exit:
            d = om.boundary_distances(o, int(tokens[t]), int(exits[t]))
            assert min(d["gates"] + [d["token"] if d["token"] is not None else 1.0]) < 1e-5, \
                f"{tag}: token {t} diverged (device {tokens[t]}/{exits[t]}, oracle {o.token}/{o.exit})"
            print(f"{tag}: near-boundary divergence at token {t}")
            return st, t
    return st, len(outs)


def test_lockstep_policy_equals_nv_step(lib, weights_dir):
    path = cached_weights(OWN, weights_dir)
    rng = np.random.default_rng(21)
    ps = [rng.integers(0, OWN.vocab, size=n) for n in (10, 33, 5, 48)]
    T = 20
    U = rng.random((len(ps), T, 4)).astype(np.float32)
    res = []
    for mode in ("step", "generate"):
        h = lib.nv_load(path, len(ps), 80)
        try:
            for i, p in enumerate(ps):
                lib.nv_prefill(h, i, p)
            if mode == "step":
                toks, exs = [], []
                for t in range(T):
                    tok, ex = lib.nv_step(h, U[:, t, :])
                    toks.append(tok)
                    exs.append(ex)
                toks, exs = np.stack(toks, 1), np.stack(exs, 1)
            else:
                toks, exs = lib.nv_generate(h, list(range(len(ps))), U, lib.SCHED_LOCKSTEP)
            logits = [lib.nv_debug_logits(h, i) for i in range(len(ps))]
            lib.nv_flush(h)
            kv = [lib.nv_debug_kv(h, i, l, 0, len(ps[i]) - 1 + T) for i in range(len(ps)) for l in (0, 5, 7)]
            res.append((toks, exs, logits, kv))
        finally:
            lib.nv_free(h)
    (t1, e1, l1, k1), (t2, e2, l2, k2) = res
    assert np.array_equal(t1, t2) and np.array_equal(e1, e2)
    assert len(set(e1.ravel().tolist())) == 4
    for a, b in zip(l1, l2):
        assert np.array_equal(a, b)
    for (ka, va), (kb, vb) in zip(k1, k2):
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)


@pytest.mark.parametrize("shape", [OWN, FORMS], ids=["own-heads", "shared-head"])
def test_greedy_policy_matches_oracle(lib, weights_dir, shape):
    path = cached_weights(shape, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(22)
    slots = [4, 0, 2, 5, 1]                       # slot 3 stays empty
    ps = [rng.integers(0, M.V, size=n) for n in (3, 60, 17, 41, 8)]
    T = 24
    U = rng.random((len(slots), T, 4)).astype(np.float32)
    h = lib.nv_load(path, 6, 90)
    try:
        for s, p in zip(slots, ps):
            lib.nv_prefill(h, s, p)
        toks, exs = lib.nv_generate(h, slots, U, lib.SCHED_GREEDY)
        assert toks.shape == (len(slots), T)
        lib.nv_flush(h)
        for i, (s, p) in enumerate(zip(slots, ps)):
            st, ok = _check_free_run(M, p, U[i], toks[i], exs[i], f"{shape.head} slot {s}")
            n_cons, f = lib.nv_debug_frontiers(h, s)
            assert n_cons == len(p) - 1 + T and list(f) == [n_cons] * 4
            if ok < T:
                continue
            worst = 0.0
            for l in range(M.L):
                k, v = lib.nv_debug_kv(h, s, l, 0, n_cons)
                worst = max(worst, rel(k, st.kv.K[l, :n_cons]), rel(v, st.kv.V[l, :n_cons]))
            assert worst < 1e-4, (s, worst)
        print(f"\n{shape.head}: exits per sequence", [np.bincount(e, minlength=5)[1:].tolist() for e in exs])
    finally:
        lib.nv_free(h)


def test_continuous_batching(lib, weights_dir):
    path = cached_weights(OWN, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(23)
    ps = [rng.integers(0, M.V, size=n) for n in (12, 30, 7)]
    Us = [rng.random((24, 4)).astype(np.float32) for _ in ps]
    got = [[] for _ in ps]
    used = [0, 0, 0]
    h = lib.nv_load(path, 3, 64)
    try:
        def gen(slots, n, policy):
            U = np.stack([Us[s][used[s]:used[s] + n] for s in slots])
            toks, exs = lib.nv_generate(h, slots, U, policy)
            for i, s in enumerate(slots):
                got[s] += list(zip(toks[i].tolist(), exs[i].tolist()))
                used[s] += n
        lib.nv_prefill(h, 0, ps[0])
        lib.nv_prefill(h, 1, ps[1])
        gen([0, 1], 8, lib.SCHED_GREEDY)
        lib.nv_prefill(h, 2, ps[2])                # joins while the others are mid-generation
        gen([2, 0], 6, lib.SCHED_GREEDY)
        gen([1], 4, lib.SCHED_LOCKSTEP)
        gen([1, 2, 0], 5, lib.SCHED_GREEDY)
        tok, ex = lib.nv_step(h, np.stack([Us[s][used[s]] for s in range(3)]))   # nv_step continues from there
        for s in range(3):
            got[s].append((int(tok[s]), int(ex[s])))
            used[s] += 1
        assert used == [20, 18, 12]
        for s in range(3):
            t = np.array([a for a, _ in got[s]])
            e = np.array([b for _, b in got[s]])
            _, ok = _check_free_run(M, ps[s], Us[s][:used[s]], t, e, f"slot {s}")
            print(f"slot {s}: {used[s]} tokens, equal prefix {ok}")
    finally:
        lib.nv_free(h)


def test_generate_errors(lib, weights_dir):
    path = cached_weights(OWN, weights_dir)
    h = lib.nv_load(path, 3, 16)
    try:
        lib.nv_prefill(h, 0, [1, 2, 3])
        lib.nv_prefill(h, 2, [4, 5])
        U = np.full((2, 3, 4), 0.5, np.float32)
        cases = [([0, 0], U, lib.SCHED_GREEDY, lib.NV_EINVAL),          # listed twice
                 ([0, 1], U, lib.SCHED_GREEDY, lib.NV_ESTATE),          # slot 1 not prefilled
                 ([0, 3], U, lib.SCHED_GREEDY, lib.NV_EINVAL),          # out of range
                 ([0, 2], U, 7, lib.NV_EINVAL),                         # unknown policy
                 ([0, 2], np.full((2, 15, 4), 0.5, np.float32), lib.SCHED_GREEDY, lib.NV_ECAPACITY)]
        bad = U.copy()
        bad[1, 2, 3] = np.nan
        cases.append(([0, 2], bad, lib.SCHED_GREEDY, lib.NV_EINVAL))
        for slots, u, pol, status in cases:
            with pytest.raises(lib.NvError) as e:
                lib.nv_generate(h, slots, u, pol)
            assert e.value.status == status, (slots, pol)
        # no tokens: a no-op; then the handle still decodes
        t0, _ = lib.nv_generate(h, [0, 2], np.zeros((2, 0, 4), np.float32))
        assert t0.shape == (2, 0)
        toks, exs = lib.nv_generate(h, [2, 0], U)
        assert toks.shape == (2, 3) and exs.min() >= 1 and exs.max() <= 4
    finally:
        lib.nv_free(h)


def _layer0_kv(M, tokens):
    n = len(tokens)
    X = np.asarray(M.embed[np.asarray(tokens, dtype=np.int64)], dtype=np.float64)
    a = om.rmsnorm(X, M.attn_norm[0], M.eps)
    pos = np.arange(n)
    k = om.rope(om.lin(a, M.wk[0]).reshape(n, M.H, M.hd), pos, M.rope_base)
    v = om.lin(a, M.wv[0]).reshape(n, M.H, M.hd)
    return k, v


def test_workload_C_greedy_properties(lib, weights_dir):
    w = workload("C")
    path = cached_weights(w.model, weights_dir)
    ps = prompts(w)
    T = 8
    U = np.ascontiguousarray(uniforms(w)[:T].transpose(1, 0, 2))    # [16][T][4]
    max_ctx = max(len(p) for p in ps) + T
    deep = [11, 12, 23, 24, 35, 36, 47]
    j = int(np.argmin([len(p) for p in ps]))
    h = lib.nv_load(path, w.batch, max_ctx)
    try:
        for i, p in enumerate(ps):
            lib.nv_prefill(h, i, p)
        toks, exs = lib.nv_generate(h, list(range(w.batch)), U, lib.SCHED_GREEDY)
        print("\nC greedy exits:", np.bincount(exs.ravel(), minlength=5)[1:].tolist())
        for i, p in enumerate(ps):
            n, f = lib.nv_debug_frontiers(h, i)
            assert n == len(p) - 1 + T
            for s in range(4):
                reached = [t for t in range(T) if exs[i, t] > s]
                assert f[s] == (len(p) - 1 + reached[-1] + 1 if reached else len(p) - 1), (i, s)
        lib.nv_flush(h)
        n = len(ps[j]) - 1 + T
        seq = np.concatenate([ps[j], toks[j, :-1]])
        k0, v0 = lib.nv_debug_kv(h, j, 0, 0, n)
        kv_deep = {l: lib.nv_debug_kv(h, j, l, 0, n) for l in deep}
        M = om.OracleModel(path)
        ok, ov = _layer0_kv(M, seq)
        e0 = max(rel(k0, ok), rel(v0, ov))
        print(f"C layer-0 KV rel {e0:.3e}")
        assert e0 < TOL
        # every sampled layer against the oracle's full-depth pass over the same tokens
        # (Summary section 2, Inferenz: Piggybacking: after the flush the cache holds every
        # layer at every position), per row, split into prompt rows and decoded rows that
        # ran directly or in a later chunk
        st = om.new_state(M, n)
        om.prefill(M, st, seq)
        rep = decoded_kv_report(lib, h, j, st, [0] + deep, len(ps[j]) - 1, [int(e) for e in exs[j]],
                                w.model.seg_layers)
        print("C greedy per-row KV worst against the oracle", {k: f"{v:.2e}" for k, v in rep.items()})
        assert max(rep.values()) < TOL
        del M, st
    finally:
        lib.nv_free(h)
    h2 = lib.nv_load(path, 1, max_ctx)
    try:
        lib.nv_prefill(h2, 0, np.concatenate([seq, toks[j, -1:]]))
        worst = 0.0
        for l in deep:
            k2, v2 = lib.nv_debug_kv(h2, 0, l, 0, n)
            worst = max(worst, rel(kv_deep[l][0], k2), rel(kv_deep[l][1], v2))
        print(f"C greedy deferred-vs-prefill KV worst rel {worst:.3e}")
        assert worst < TOL
    finally:
        lib.nv_free(h2)
