"""Parity of the split-K matrix-core decode product (row groups of 5-64 rows, K a multiple
of 512: every K slice of 512 is one block's, and a second kernel adds the slices in order
and applies the epilogue) with the oracle, on a bf16 model whose widths are multiples of 512
(d 512, 4 heads of 128, MLP width 1024, so every block product takes the path): logits,
gates, tokens and exits as in the other bf16 tests, every layer's KV at the decoded
positions and their hidden rows within 2e-2 relative (per row).  Forced exits make
catch-up chunks of 6, 9, 13, 19, 21, 32, 40 and 64 rows at the deeper segments (one to
four 16-row tiles).  A second test runs the same chunks through the split-K path and
through the single-block matrix-core path and compares the KV they write."""
import numpy as np
import pytest

from oracle import model as om
from synth import cached_weights, tiny_variant
from tests.parity import StepCheck, check_step, decoded_kv_report, hidden_rows_worst, rel, run_forced

pytestmark = pytest.mark.gpu

TOL = 2e-2
SK_MODEL = tiny_variant(wdtype="bf16", n_layers=4, d_model=512, n_heads=4, head_dim=128, ffn=1024, vocab=512)
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


@pytest.mark.parametrize("prompt_len,pattern", [
    (9, [1] * 8 + [4] + [2] * 3),          # a 9-row chunk at segments 2..4
    (30, [1] * 20 + [4] + [0] * 4),        # a 21-row chunk, then free draws
    (17, [1] * 31 + [4]),                  # a 32-row chunk (two 16-row tiles)
    (12, [2] * 12 + [3] * 6 + [4]),        # chunks of 13 (segment 3) and 19 (segment 4) rows
    (7, [1] * 5 + [4] + [0] * 3),          # a 6-row chunk (one tile, 10 rows of padding)
    (5, [1] * 39 + [4]),                   # a 40-row chunk (three tiles)
    (4, [1] * 63 + [4]),                   # a 64-row chunk (four tiles)
], ids=["chunk9", "chunk21", "chunk32", "chunks13-19", "chunk6", "chunk40", "chunk64"])
def test_splitk_parity(lib, weights_dir, prompt_len, pattern, monkeypatch):
    monkeypatch.delenv("NVIUM_SK_MIN_ROWS", raising=False)
    monkeypatch.delenv("NVIUM_MFMA_MIN_ROWS", raising=False)
    path = cached_weights(SK_MODEL, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(100 + prompt_len)
    prompt = rng.integers(0, M.V, size=prompt_len)
    U = _forced_u(pattern, rng)
    max_ctx = prompt_len + len(pattern)
    outs, st = om.generate(M, prompt, U, max_ctx=max_ctx)
    h = lib.nv_load(path, 1, max_ctx)
    try:
        lib.nv_prefill(h, 0, prompt)
        recs = run_forced(h, lib, outs)
        res = StepCheck()
        for t, (o, (tok, ex, lg, gw)) in enumerate(zip(outs, recs)):
            if pattern[t]:
                assert ex == pattern[t]
            check_step(t, o, tok, ex, lg, gw, res, logit_band=True)
        print("\nsplit-K:", end=" ")
        res.finish(TOL)
        lib.nv_flush(h)
        P = prompt_len - 1
        rep = decoded_kv_report(lib, h, 0, st, range(M.L), P, [r[1] for r in recs], SK_MODEL.seg_layers)
        hid = hidden_rows_worst(lib, h, 0, outs, P)
        print("split-K per-row KV worst", {k: f"{v:.2e}" for k, v in rep.items()}, f"hidden rows {hid:.2e}")
        assert max(rep.values()) < TOL and hid < TOL
    finally:
        lib.nv_free(h)


def test_splitk_and_single_block_paths_agree(lib, weights_dir, monkeypatch):
    """A 19-row prefill and a 25-row catch-up chunk through the split-K product and through
    the single-block matrix-core product write the same KV to bf16 rounding at every layer
    (positions 0-43: the prefill's 19, then 25 decode steps, the last one at exit 4)."""
    monkeypatch.delenv("NVIUM_MFMA_MIN_ROWS", raising=False)
    path = cached_weights(SK_MODEL, weights_dir)
    rng = np.random.default_rng(7)
    prompt = rng.integers(0, SK_MODEL.vocab, size=20)
    pattern = [1] * 24 + [4]
    U = _forced_u(pattern, rng)
    kvs = []
    for sk in ("5", "0"):
        monkeypatch.setenv("NVIUM_SK_MIN_ROWS", sk)
        h = lib.nv_load(path, 1, 64)
        try:
            lib.nv_prefill(h, 0, prompt)
            for t in range(len(pattern)):
                lib.nv_step(h, U[t:t + 1])
            kvs.append([lib.nv_debug_kv(h, 0, l, 0, 44) for l in range(SK_MODEL.n_layers)])
        finally:
            lib.nv_free(h)
    for (k1, v1), (k2, v2) in zip(*kvs):
        assert rel(k1, k2) < 1e-2 and rel(v1, v2) < 1e-2



def test_splitk_multirow_heads(lib, weights_dir, monkeypatch):
    """Eight sequences stopping at one exit in every step: the exit head of 8 rows and the
    block products of 8-64-row groups take the split-K product.  Each sequence's tokens,
    exits, logits and gates against its own oracle run (the exit pattern forced, the same
    for all eight: 1, 2, 3 and 4 in turn, with deferred chunks at every depth)."""
    monkeypatch.delenv("NVIUM_MFMA_MIN_ROWS", raising=False)
    monkeypatch.delenv("NVIUM_SK_MIN_ROWS", raising=False)
    path = cached_weights(SK_MODEL, weights_dir)
    M = om.OracleModel(path)
    B, n_steps = 8, 12
    pattern = [1, 2, 3, 4] * (n_steps // 4)
    rng = np.random.default_rng(21)
    prompts = [rng.integers(0, M.V, size=int(rng.integers(6, 30))) for _ in range(B)]
    Us = [_forced_u(pattern, rng) for _ in range(B)]
    max_ctx = 30 + n_steps
    oracle = [om.generate(M, prompts[b], Us[b], max_ctx=max_ctx)[0] for b in range(B)]
    h = lib.nv_load(path, B, max_ctx)
    try:
        for b in range(B):
            lib.nv_prefill(h, b, prompts[b])
        res = StepCheck()
        for t in range(n_steps):
            U = np.stack([oracle[b][t].u for b in range(B)]).astype(np.float32)
            nxt = np.array([oracle[b][t].token for b in range(B)], np.int32)
            tok, ex = lib.nv_step_forced(h, U, nxt)
            for b in range(B):
                assert ex[b] == pattern[t]
                check_step(t, oracle[b][t], int(tok[b]), int(ex[b]), lib.nv_debug_logits(h, b),
                           lib.nv_debug_gates(h, b), res, logit_band=True)
        print("\nsplit-K heads of 8 rows:", end=" ")
        res.finish(TOL)
    finally:
        lib.nv_free(h)
