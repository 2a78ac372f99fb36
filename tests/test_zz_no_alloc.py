"""nv_exit_draw_static (the exit draw with the library's own per-GPU scratch, for callers
that cannot allocate) against nv_exit_draw with a caller workspace, through the C ABI: two
rounds in a row, the second with a smaller input (1.5B shape, then the tiny one), several
uniforms each; logits bit-identical and tokens equal."""
import numpy as np
import pytest

from synth.weights import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(rng, d, V, bf16):
    h = (rng.standard_normal(d) * 3.0).astype(np.float32)
    g = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    W = (rng.standard_normal((V, d)) * 0.02).astype(np.float32)
    return h, g, (f32_to_bf16_bits(W).view(np.int16) if bf16 else W)


def test_static_scratch_matches_workspace_entry_point():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_exits_transformer_amd.lib as L
    L.library()
    rng = np.random.default_rng(77)
    for d, V, bf16 in [(1536, 32000, True), (128, 512, False)]:    # the second round is smaller
        h, g, W = _inputs(rng, d, V, bf16)
        th, tg, tW = (torch.as_tensor(x, device="cuda") for x in (h, g, W))
        us = rng.random(8).astype(np.float32)
        la = torch.empty(V, dtype=torch.float32, device="cuda")
        lb = torch.empty(V, dtype=torch.float32, device="cuda")
        ta = torch.full((len(us),), -1, dtype=torch.int32, device="cuda")
        tb = torch.full((len(us),), -2, dtype=torch.int32, device="cuda")
        ws_bytes = L.nv_exit_draw_workspace(V)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        wd = 1 if bf16 else 0
        for i, u in enumerate(us):
            L.nv_exit_draw_static(th, tg, tW, wd, d, V, 1e-5, float(u), lb, tb[i:i + 1].data_ptr())
            torch.cuda.synchronize()
            got_b = lb.cpu().numpy().copy()
            L.nv_exit_draw(th, tg, tW, wd, d, V, 1e-5, float(u), la, ta[i:i + 1].data_ptr(), ws, ws_bytes)
            torch.cuda.synchronize()
            assert np.array_equal(got_b.view(np.uint32), la.cpu().numpy().view(np.uint32)), (d, V, i)
        a, b = ta.cpu().numpy(), tb.cpu().numpy()
        print(f"\nd {d} V {V}: tokens {b.tolist()}")
        assert np.array_equal(a, b), (a, b)
        assert (b >= 0).all() and (b < V).all()
    # sizes beyond the scratch are refused before anything runs
    x = torch.zeros(16, device="cuda")
    assert L.library().nv_exit_draw_static(x.data_ptr(), x.data_ptr(), x.data_ptr(), 0, 128, 65544, 1e-5, 0.5,
                                            x.data_ptr(), x.data_ptr(), None) == L.NV_EINVAL
