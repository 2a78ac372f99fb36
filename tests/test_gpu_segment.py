"""Parity of the persistent segment kernel (one cooperative launch per segment for a
single decode row) with the oracle, on a small bf16 model with 128-wide heads (d 256,
2 heads, SwiGLU 512, 8 layers): logits and KV within 2e-2 relative; exits and tokens
equal unless a draw lies within the decision shift that the checked logits and gates
imply (counted and reported).  Exit patterns force single-row chunks at every segment
(the kernel runs) or deferred chunks (the per-phase kernels run), and long contexts
give key ranges beyond what a block prefetches."""
import numpy as np
import pytest

from oracle import model as om
from synth import cached_weights, tiny_variant
from tests.parity import StepCheck, check_step, decoded_kv_report, hidden_rows_worst, rel, run_forced

pytestmark = pytest.mark.gpu

TOL = 2e-2
SEG_MODEL = tiny_variant(wdtype="bf16", d_model=256, n_heads=2, head_dim=128, ffn=512)
STOP, GO = 0.0, np.float32(1.0 - 2.0 ** -24)


@pytest.fixture(autouse=True)
def segment_on(monkeypatch):
    monkeypatch.setenv("NVIUM_SEGMENT", "1")   # read by nv_load


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
            continue                      # free draw
        U[t, :3] = GO
        if e < 4:
            U[t, e - 1] = STOP
    return U


def _run_case(lib, path, M, prompt, pattern, rng, tag):
    U = _forced_u(pattern, rng)
    max_ctx = len(prompt) + len(pattern)
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
        print(f"\n{tag}:", end=" ")
        res.finish(TOL)
        lib.nv_flush(h)
        P = len(prompt) - 1
        rep = decoded_kv_report(lib, h, 0, st, range(M.L), P, [r[1] for r in recs], M.L // 4)
        hid = hidden_rows_worst(lib, h, 0, outs, P)
        print(f"{tag} per-row KV worst", {k: f"{v:.2e}" for k, v in rep.items()}, f"hidden rows {hid:.2e}")
        assert max(rep.values()) < TOL and hid < TOL
    finally:
        lib.nv_free(h)


@pytest.mark.parametrize("prompt_len,pattern", [
    (64, [4] * 16),                             # single-row chunks at every segment
    (2, [4] * 6),                               # a 1-token prefill, then contexts of 1..6 keys
    (90, [0] * 24),                             # free draws: single rows and deferred chunks
    (40, [1, 4, 2, 4, 3, 4, 4, 1, 1, 4, 4]),    # deferred chunks between single-row launches
])
def test_segment_kernel_parity(lib, weights_dir, prompt_len, pattern):
    path = cached_weights(SEG_MODEL, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(prompt_len + len(pattern))
    prompt = rng.integers(0, M.V, size=prompt_len)
    _run_case(lib, path, M, prompt, pattern, rng, f"segment kernel p{prompt_len}")


def test_segment_kernel_long_context(lib, weights_dir):
    """3300 keys: 32 splits per head of about 104 keys, more than a block's waves
    prefetch (96), so the in-phase key loop runs too."""
    path = cached_weights(SEG_MODEL, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(33)
    prompt = rng.integers(0, M.V, size=3300)
    _run_case(lib, path, M, prompt, [4, 4, 4], rng, "segment kernel ctx 3300")


def test_segment_kernel_matches_per_phase_kernels(lib, weights_dir, monkeypatch):
    """The same single-row steps through the persistent kernel and through the per-phase
    kernels (NVIUM_SEGMENT=0) give the same logits and KV to bf16 rounding."""
    path = cached_weights(SEG_MODEL, weights_dir)
    rng = np.random.default_rng(8)
    prompt = rng.integers(0, SEG_MODEL.vocab, size=50)
    U = _forced_u([4] * 8, rng)
    nxt = rng.integers(0, SEG_MODEL.vocab, size=8).astype(np.int32)
    res = []
    for flag in ("1", "0"):
        monkeypatch.setenv("NVIUM_SEGMENT", flag)
        h = lib.nv_load(path, 1, 64)
        try:
            lib.nv_prefill(h, 0, prompt)
            logits = []
            for t in range(8):
                lib.nv_step_forced(h, U[t:t + 1], nxt[t:t + 1])
                logits.append(lib.nv_debug_logits(h, 0))
            kv = [lib.nv_debug_kv(h, 0, l, 0, 57) for l in range(SEG_MODEL.n_layers)]
            res.append((logits, kv))
        finally:
            lib.nv_free(h)
    (l1, kv1), (l2, kv2) = res
    for a, b in zip(l1, l2):
        assert rel(a, b) < 1e-2
    for (k1, v1), (k2, v2) in zip(kv1, kv2):
        assert rel(k1, k2) < 1e-2 and rel(v1, v2) < 1e-2
