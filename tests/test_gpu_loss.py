"""Parity of the device mixture objective (nv_mixture_loss) with the oracle's
mixture_loss: L_mix, L_compute, L_total and every position's router outputs,
log pi_k of the target, -log pi_mix and expected depth.

- Tiny fp32 model, both exit forms (own heads + linear gate; shared head with adapters +
  router MLP): 299 positions, in one head pass per exit (the default, as many rows as a
  256 MiB logits workspace holds) and in passes of 256 and a ragged 43 rows.  Router
  outputs within 1e-6, log-probabilities within 1e-4 absolute, the means within 1e-6
  relative.
- The shortest sequence (two tokens, one position) and the argument errors.
- After the loss the sequence decodes exactly as after nv_prefill of the same tokens
  (the same segment kernels ran; the exits only read the hidden rows).
- Tiny bf16 model at 4500 tokens (more rows than one prefill piece holds) and the 1.5B
  bf16 model on a 128-token prefix of its synthetic prompt (oracle values stored under
  tests/golden): within 2e-2."""
import json
import os

import numpy as np
import pytest

from oracle import model as om
from synth import cached_weights, prompts, tiny_variant, workload
from tests.parity import rel

pytestmark = pytest.mark.gpu

OWN = tiny_variant()
FORMS = tiny_variant(head="shared", adapter_dim=16, router="mlp", router_dim=8)
BF16_TINY = tiny_variant(wdtype="bf16", ffn=384)


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_exits_transformer_amd.lib as L
    L.library()
    return L


def _compare(got, pp, want, tol_w, tol_lp, tol_mean, tag):
    L_mix, L_comp, L_tot = got
    dw = float(np.max(np.abs(pp[:, :4] - want.w)))
    dlp = float(np.max(np.abs(pp[:, 4:8] - want.logp)))
    dn = rel(pp[:, 8], want.nll_mix)
    dd = rel(pp[:, 9], want.depth)
    print(f"\n{tag}: L_mix {L_mix:.8f} vs {want.L_mix:.8f}, L_compute {L_comp:.8f} vs {want.L_compute:.8f}; "
          f"max |dw| {dw:.2e} max |dlogp| {dlp:.2e} nll rel {dn:.2e} depth rel {dd:.2e}")
    assert np.all(pp[:, 3] == 1.0)
    assert dw < tol_w and dlp < tol_lp
    assert dn < tol_mean and dd < tol_mean
    assert abs(L_mix - want.L_mix) < tol_mean * abs(want.L_mix)
    assert abs(L_comp - want.L_compute) < tol_mean * abs(want.L_compute)
    assert abs(L_tot - want.L_total) < tol_mean * abs(want.L_total)


@pytest.mark.parametrize("rows", [None, "256"], ids=["one-pass", "passes-256-43"])
@pytest.mark.parametrize("shape", [OWN, FORMS], ids=["own-heads", "shared-head"])
def test_loss_tiny_fp32(lib, weights_dir, shape, rows, monkeypatch):
    if rows:
        monkeypatch.setenv("NVIUM_LOSS_ROWS", rows)   # read by nv_load
    path = cached_weights(shape, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(299)
    tokens = rng.integers(0, M.V, size=300)
    beta = 0.37
    want = om.mixture_loss(M, tokens, beta)
    h = lib.nv_load(path, 1, 300)
    try:
        got, pp = lib.nv_mixture_loss(h, 0, tokens, beta, per_pos=True)
    finally:
        lib.nv_free(h)
    _compare(got, pp, want, 1e-6, 1e-4, 1e-6, f"tiny fp32 {shape.head}/{shape.router}")


def test_loss_single_position_and_errors(lib, weights_dir):
    path = cached_weights(OWN, weights_dir)
    M = om.OracleModel(path)
    tokens = [7, 300]
    want = om.mixture_loss(M, tokens, 1.0)
    h = lib.nv_load(path, 2, 16)
    try:
        got, pp = lib.nv_mixture_loss(h, 1, tokens, 1.0, per_pos=True)
        _compare(got, pp, want, 1e-6, 1e-4, 1e-6, "one position")
        for bad, status in (([5], lib.NV_EINVAL), ([1] * 17, lib.NV_ECAPACITY), ([1, M.V], lib.NV_EINVAL)):
            with pytest.raises(lib.NvError) as e:
                lib.nv_mixture_loss(h, 0, bad)
            assert e.value.status == status
        with pytest.raises(lib.NvError) as e:
            lib.nv_mixture_loss(h, 2, tokens)
        assert e.value.status == lib.NV_EINVAL
        with pytest.raises(lib.NvError) as e:
            lib.nv_mixture_loss(h, 0, tokens, float("nan"))
        assert e.value.status == lib.NV_EINVAL
    finally:
        lib.nv_free(h)


@pytest.mark.parametrize("shape", [OWN, FORMS], ids=["own-heads", "shared-head"])
def test_decode_after_loss_equals_decode_after_prefill(lib, weights_dir, shape):
    path = cached_weights(shape, weights_dir)
    rng = np.random.default_rng(5)
    tokens = rng.integers(0, shape.vocab, size=90)
    U = rng.random((6, 4)).astype(np.float32)
    nxt = rng.integers(0, shape.vocab, size=6).astype(np.int32)
    runs = []
    for use_loss in (True, False):
        h = lib.nv_load(path, 1, 128)
        try:
            if use_loss:
                lib.nv_mixture_loss(h, 0, tokens)
            else:
                lib.nv_prefill(h, 0, tokens)
            recs = []
            for t in range(6):
                tok, ex = lib.nv_step_forced(h, U[t:t + 1], nxt[t:t + 1])
                recs.append((int(tok[0]), int(ex[0]), lib.nv_debug_logits(h, 0)))
            lib.nv_flush(h)
            kv = lib.nv_debug_kv(h, 0, shape.n_layers - 1, 0, 95)
            runs.append((recs, kv))
        finally:
            lib.nv_free(h)
    (r1, kv1), (r2, kv2) = runs
    for (t1, e1, l1), (t2, e2, l2) in zip(r1, r2):
        assert t1 == t2 and e1 == e2 and np.array_equal(l1, l2)
    assert np.array_equal(kv1[0], kv2[0]) and np.array_equal(kv1[1], kv2[1])


def test_loss_tiny_bf16_long(lib, weights_dir):
    path = cached_weights(BF16_TINY, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(4500)
    tokens = rng.integers(0, M.V, size=4500)
    want = om.mixture_loss(M, tokens, 0.1)
    h = lib.nv_load(path, 1, 4500)
    try:
        got, pp = lib.nv_mixture_loss(h, 0, tokens, 0.1, per_pos=True)
    finally:
        lib.nv_free(h)
    _compare(got, pp, want, 2e-2, 2e-1, 2e-2, "tiny bf16 4500 tokens")


def test_loss_tiny_bf16_mixed_passes(lib, weights_dir, monkeypatch):
    """Head passes of 280 and 19 rows: the first runs the long-chunk head product with the
    cross-entropy fused into its epilogue, the second (below that product's 33-row
    minimum) stores its logits for k_xent.  Both against the oracle, as the other bf16
    cases."""
    monkeypatch.setenv("NVIUM_LOSS_ROWS", "280")   # read by nv_load
    path = cached_weights(BF16_TINY, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(2800)
    tokens = rng.integers(0, M.V, size=300)
    want = om.mixture_loss(M, tokens, 0.25)
    h = lib.nv_load(path, 1, 300)
    try:
        got, pp = lib.nv_mixture_loss(h, 0, tokens, 0.25, per_pos=True)
    finally:
        lib.nv_free(h)
    _compare(got, pp, want, 2e-2, 2e-1, 2e-2, "tiny bf16 passes 280 + 19")


def test_loss_1p5b_bf16(lib, weights_dir):
    """Expected values from tests/golden/loss_1p5b_a128.json (written by
    tests/golden/make_loss_1p5b.py, which runs the oracle; about a minute on the CPU)."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "loss_1p5b_a128.json")))
    w = workload("A")
    tokens = prompts(w)[0][:g["n_tokens"]]
    assert [int(t) for t in tokens] == g["tokens"], "synthetic prompt changed: rerun the golden script"
    path = cached_weights(w.model, weights_dir)
    h = lib.nv_load(path, 1, 128)
    try:
        got, pp = lib.nv_mixture_loss(h, 0, tokens, g["beta"], per_pos=True)
    finally:
        lib.nv_free(h)
    want = om.LossOut(g["L_mix"], g["L_compute"], g["L_total"], np.array(g["nll_mix"]), np.array(g["depth"]),
                      np.array(g["logp"]), np.array(g["w"]))
    _compare(got, pp, want, 2e-2, 2e-1, 2e-2, "1.5B bf16 128 tokens")
