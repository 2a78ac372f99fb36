"""Matrix-core chunk attention (launch groups of more than 64 rows on a bf16 KV cache)
against the oracle, for head_dim 32, 64 and 128.

A full-depth prefill of 65, 200 and 1100 positions on small 4-layer bf16 models, with
128-row items of eight 16-row waves: one item holding 65 rows (four full waves, one with a
single row, three with none); a full item and a ragged 72-row one; nine items with key
ranges split at 512 and merged by the combine pass.  Every layer's keys and values (each layer's input
went through the previous layer's attention) and the final hidden states (through the
last layer's attention) within 2e-2 relative."""
import numpy as np
import pytest

from oracle import model as om
from synth import cached_weights, tiny_variant
from tests.parity import rel

pytestmark = pytest.mark.gpu

TOL = 2e-2
SHAPES = {
    32: tiny_variant(wdtype="bf16", n_layers=4, d_model=128, n_heads=4, head_dim=32, ffn=256),
    64: tiny_variant(wdtype="bf16", n_layers=4, d_model=128, n_heads=2, head_dim=64, ffn=256),
    128: tiny_variant(wdtype="bf16", n_layers=4, d_model=256, n_heads=2, head_dim=128, ffn=512),
}


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_exits_transformer_amd.lib as L
    L.library()
    return L


@pytest.mark.parametrize("n", [66, 201, 1101])
@pytest.mark.parametrize("hd", [32, 64, 128])
def test_chunk_attention_mfma(lib, weights_dir, hd, n):
    shape = SHAPES[hd]
    path = cached_weights(shape, weights_dir)
    M = om.OracleModel(path)
    rng = np.random.default_rng(hd * 10000 + n)
    prompt = rng.integers(0, M.V, size=n)
    r = n - 1                                     # positions the prefill runs
    kv = om.KVCache(M, r)
    X = np.asarray(M.embed[np.asarray(prompt[:r], dtype=np.int64)], dtype=np.float64)
    pos = np.arange(r)
    for l in range(M.L):
        X = om.layer_rows(M, l, X, pos, kv)
    h = lib.nv_load(path, 1, n)
    try:
        lib.nv_prefill(h, 0, prompt)
        worst = 0.0
        for l in range(M.L):
            k, v = lib.nv_debug_kv(h, 0, l, 0, r)
            worst = max(worst, rel(k, kv.K[l, :r]), rel(v, kv.V[l, :r]))
        hid = lib.nv_debug_hidden(h, 0, 0, r)
    finally:
        lib.nv_free(h)
    eh = rel(hid, X)
    row_worst = max(rel(hid[i], X[i]) for i in (0, 63, 64, r - 1))
    print(f"\nhd {hd} n {n}: KV worst rel {worst:.2e}, hidden rel {eh:.2e}, sampled rows {row_worst:.2e}")
    assert worst < TOL and eh < TOL and row_worst < TOL
