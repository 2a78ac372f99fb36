"""nv_exit_draw (one exit's RMSNorm + LM head and the inverse-CDF draw, on caller buffers)
against the oracle: logits against the oracle's head (float64), and for each of many
uniforms the token against the oracle's inverse CDF of softmax(logits) in token-id order;
a difference is accepted only within 1e-5 of a boundary of the oracle's CDF, and the token
must always be the exact draw of the device's own logits (within 1e-6 of a boundary).
Shapes: the tiny model's (d 128, vocab 512, float32) and the 1.5B model's (d 1536,
vocab 32000, bf16 weights)."""
import numpy as np
import pytest

from oracle import model as om
from synth.weights import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_exits_transformer_amd.lib as L
    L.library()
    return L


def _case(rng, d, V, bf16):
    h = (rng.standard_normal(d) * 3.0).astype(np.float32)           # residual-stream scale
    g = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    W = (rng.standard_normal((V, d)) * 0.02).astype(np.float32)
    if bf16:
        bits = f32_to_bf16_bits(W)
        Wv = (bits.astype(np.uint32) << 16).view(np.float32)
        return h, g, bits, Wv
    return h, g, W, W


def _draw(lib, torch, h, g, Wdev, wdtype, d, V, u, eps=1e-5):
    dev = "cuda"
    th = torch.as_tensor(h, device=dev)
    tg = torch.as_tensor(g, device=dev)
    tW = torch.as_tensor(Wdev.view(np.int16) if wdtype == 1 else Wdev, device=dev)
    logits = torch.empty(V, dtype=torch.float32, device=dev)
    tok = torch.full((len(u),), -7, dtype=torch.int32, device=dev)
    ws_bytes = lib.nv_exit_draw_workspace(V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    for i, ui in enumerate(u):
        lib.nv_exit_draw(th, tg, tW, wdtype, d, V, eps, float(ui), logits, tok[i:i + 1].data_ptr(), ws, ws_bytes)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), tok.cpu().numpy()


@pytest.mark.parametrize("d,V,bf16", [(128, 512, False), (1536, 32000, True)], ids=["tiny-f32", "1p5b-bf16"])
def test_exit_draw_against_oracle(lib, d, V, bf16):
    import torch
    rng = np.random.default_rng(d + V)
    h, g, Wdev, Wv = _case(rng, d, V, bf16)
    u = np.concatenate([rng.random(60), [0.0, np.float32(1.0 - 2.0 ** -24), 0.5, 1e-7]]).astype(np.float32)
    lg, tok = _draw(lib, torch, h, g, Wdev, 1 if bf16 else 0, d, V, u)
    # logits: the oracle's exit head (the stored weight values, float64)
    want = om.lin(om.rmsnorm(h.astype(np.float64)[None, :], g.astype(np.float64), 1e-5), Wv.astype(np.float64))[0]
    rel = np.linalg.norm(lg - want) / np.linalg.norm(want)
    print(f"\nd {d} V {V}: logits rel {rel:.2e}")
    assert rel < 1e-5
    pi = om.softmax(want)
    F = np.cumsum(pi)
    z = lg.astype(np.float64)
    e = np.exp(z - z.max())
    Fd = np.cumsum(e / e.sum())
    near = 0
    for ui, t in zip(u, tok):
        assert 0 <= t < V
        own = om.inverse_cdf(e / e.sum(), float(ui))
        if own != t:
            lo = Fd[t - 1] if t > 0 else 0.0
            assert min(abs(float(ui) - lo), abs(Fd[t] - float(ui))) < 1e-6, (ui, t, own)
        ref = om.inverse_cdf(pi, float(ui))
        if ref != t:
            lo = F[t - 1] if t > 0 else 0.0
            dist = min(abs(float(ui) - lo), abs(F[t] - float(ui)))
            assert dist < 1e-5, (ui, t, ref, dist)
            near += 1
    print(f"d {d} V {V}: {len(u)} draws, {near} within 1e-5 of an oracle boundary")
    assert tok[len(u) - 4] == 0 or pi[0] == 0.0        # u = 0 draws the first id with mass


def test_exit_draw_peaked_distribution(lib):
    """One logit far above the rest: every draw is that id (the others underflow to zero
    mass in float32 exponentials), including u next to 1."""
    import torch
    d, V = 128, 512
    rng = np.random.default_rng(3)
    h = np.zeros(d, np.float32)
    h[0] = 1.0
    g = np.ones(d, np.float32)
    W = (rng.standard_normal((V, d)) * 0.01).astype(np.float32)
    W[77, 0] = 1e4 / np.sqrt(d)        # RMSNorm(h)[0] = sqrt(d): logit 77 is 1e4
    u = np.array([0.0, 0.3, np.float32(1.0 - 2.0 ** -24)], np.float32)
    _, tok = _draw(lib, torch, h, g, W, 0, d, V, u)
    assert list(tok) == [77, 77, 77]


def test_exit_draw_errors(lib):
    import torch
    L = lib.library()
    dev = "cuda"
    x = torch.zeros(4096, dtype=torch.float32, device=dev)
    ws = torch.zeros(64, dtype=torch.uint8, device=dev)
    p = x.data_ptr()
    assert lib.nv_exit_draw_workspace(12) == 0
    assert lib.nv_exit_draw_workspace(512) == 512
    assert L.nv_exit_draw(None, p, p, 0, 128, 512, 1e-5, 0.5, p, p, ws.data_ptr(), 512, None) == lib.NV_EINVAL
    assert L.nv_exit_draw(p, p, p, 0, 128, 500, 1e-5, 0.5, p, p, ws.data_ptr(), 512, None) == lib.NV_EINVAL
    assert L.nv_exit_draw(p, p, p, 0, 128, 512, 1e-5, 1.0, p, p, ws.data_ptr(), 512, None) == lib.NV_EINVAL
    assert L.nv_exit_draw(p, p, p, 2, 128, 512, 1e-5, 0.5, p, p, ws.data_ptr(), 512, None) == lib.NV_EINVAL
    assert L.nv_exit_draw(p, p, p, 0, 128, 512, 1e-5, 0.5, p, p, ws.data_ptr(), 64, None) == lib.NV_ECAPACITY
