"""An independent textbook LLaMA-2 forward in torch (float64, CPU), used to pin the oracle.

Written from the standard definition with library routines: torch.nn.functional
rms_norm, scaled_dot_product_attention(is_causal=True) and silu; rotary
embedding as a complex rotation (each pair (x_i, x_{i+hd/2}) is the complex
number x_i + j x_{i+hd/2}, multiplied by exp(j * pos * base^(-2i/hd))).
"""
import numpy as np
import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def rope_complex(x, pos, base):
    """x: [H, n, hd] float64 tensor, pos: [n]."""
    hd = x.shape[-1]
    half = hd // 2
    theta = base ** (-torch.arange(half, dtype=torch.float64) * 2.0 / hd)
    ang = torch.as_tensor(pos, dtype=torch.float64)[:, None] * theta[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def forward(M, tokens):
    """Full-depth causal forward over `tokens` at positions 0..n-1.

    Returns (h_exit [n_exits][n, d], logits [n_exits][n, V], K [L][n, H, hd], V [L][n, H, hd])."""
    n = len(tokens)
    d, H, hd = M.d, M.H, M.hd
    pos = np.arange(n)
    x = _t(M.embed[np.asarray(tokens)])
    hs, Ks, Vs = [], [], []
    for l in range(M.L):
        a = F.rms_norm(x, (d,), weight=_t(M.attn_norm[l]), eps=M.eps)
        q = (a @ _t(M.wq[l]).T).view(n, H, hd).transpose(0, 1)
        k = (a @ _t(M.wk[l]).T).view(n, H, hd).transpose(0, 1)
        v = (a @ _t(M.wv[l]).T).view(n, H, hd).transpose(0, 1)
        q = rope_complex(q, pos, M.rope_base)
        k = rope_complex(k, pos, M.rope_base)
        Ks.append(k.transpose(0, 1).numpy().copy())
        Vs.append(v.transpose(0, 1).numpy().copy())
        o = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)[0]
        x = x + o.transpose(0, 1).reshape(n, d) @ _t(M.wo[l]).T
        m = F.rms_norm(x, (d,), weight=_t(M.mlp_norm[l]), eps=M.eps)
        x = x + (F.silu(m @ _t(M.wg[l]).T) * (m @ _t(M.wu[l]).T)) @ _t(M.wd[l]).T
        if (l + 1) in M.exit_layers:
            hs.append(x.clone())
    logits = [F.rms_norm(h, (d,), weight=_t(M.exit_norm[k]), eps=M.eps) @ _t(M.head[k]).T
              for k, h in enumerate(hs)]
    return [h.numpy() for h in hs], [z.numpy() for z in logits], Ks, Vs
