"""CPU oracle of the N-vium mixture-of-exits decode step.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py import this package.  The product path never calls it.

Plain NumPy in float64, one token at a time, every layer for every token, all
exits evaluated.  It shares no code with the HIP path; both read the same
seeded weights file (this module has its own reader).

Citations are to the pages on "N-vium: Mixture-of-Exits Transformer for
Accelerated Exact Generation" (arXiv 2605.13190):
  [Arch]      gist.science technical summary, section 2 "Methodik", part
              "Architektur": blocks ending in a router, router output w_k, the
              equation for p_k with w_{N_V} = 1, the equation for pi_mix; a
              router MLP produces w_k; all exits share the final LM head, with
              light adapter MLPs mapping intermediate states to its geometry.
  [Piggy]     same summary, section 2, part "Inferenz: Piggybacking": layers
              above the exit are deferred, their hidden states are concatenated
              with later tokens' states at those depths, KV becomes complete.
  [Contrib]   same summary, section 3 "Hauptbeitraege": exact sampling from the
              mixture; complete and exact KV caches.
  [Results]   same summary, section 4: LLaMA-2 architecture, 4 exits.
  [General]   same summary, section 5, and the abstract: zero routing mass on the
              intermediate heads recovers the standard transformer exactly.
  [Abstract]  the English abstract (quoted on the gptget.net and fugumt pages).

Readings where the pages are silent (each is listed with its reason in the
design notes): in the first form every exit has its own RMSNorm and LM head and
the router is the linear gate sigmoid(g_k . h + b_k) on the un-normalised
residual stream after the exit's last layer; in the second form (the pages'
own) the router is a one-hidden-layer MLP, sigmoid(w2_k . silu(W1_k h + b1_k) +
b_k), and exit k < N_V reads the final RMSNorm + LM head through the residual
adapter h + U_k silu(D_k h); LLaMA-2 layer = pre-norm RMSNorm, MHA with rotate-half
RoPE on 0-based positions, scale 1/sqrt(hd), SwiGLU MLP, no linear biases;
the exit is chosen by walking the gates with u_1..u_3 (stop at gate k iff
u_k < w_k) and the token by inverse CDF with u_4 in token-id order (smallest
i with u_4 < F(i)).
"""
from __future__ import annotations

import math
import struct
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------------------------
# weights file reader (format: 256-byte header, then 256-aligned tensors in a fixed order)
# --------------------------------------------------------------------------------------------


class OracleModel:
    """Model parameters as float64 (small models) or float32 (large; cast per use)."""

    def __init__(self, path: str, keep_f32_above: int = 50_000_000):
        with open(path, "rb") as f:
            hdr = f.read(256)
        if hdr[:8] != b"NVIUMW01":
            raise ValueError("not an N-vium weights file")
        (hbytes, L, d, H, hd, F, V, nx, wd) = struct.unpack_from("<9i", hdr, 8)
        eps, rope_base = struct.unpack_from("<2f", hdr, 44)
        self.exit_layers = list(struct.unpack_from("<4i", hdr, 52))
        self.gate_bias = [float(b) for b in struct.unpack_from("<4f", hdr, 68)]
        head_form, self.adapter_dim, router_form, self.router_dim = struct.unpack_from("<4i", hdr, 84)
        self.shared_head = head_form == 1
        self.router_mlp = router_form == 1
        self.L, self.d, self.H, self.hd, self.F, self.V, self.n_exits = L, d, H, hd, F, V, nx
        self.eps, self.rope_base = float(eps), float(rope_base)
        self.bf16 = wd == 1
        raw = np.memmap(path, dtype=np.uint8, mode="r")
        off = [hbytes]

        def take(shape, is_mat):
            n = int(np.prod(shape))
            o = (off[0] + 255) // 256 * 256
            if is_mat and self.bf16:
                bits = np.frombuffer(raw, dtype=np.uint16, count=n, offset=o)
                arr = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
                off[0] = o + 2 * n
            else:
                arr = np.frombuffer(raw, dtype=np.float32, count=n, offset=o).copy()
                off[0] = o + 4 * n
            return arr.reshape(shape)

        total = V * d * (1 + (1 if self.shared_head else nx)) + L * (4 * d * d + 3 * F * d)
        self.f64 = total <= keep_f32_above
        cast = (lambda a: a.astype(np.float64)) if self.f64 else (lambda a: np.ascontiguousarray(a))

        self.embed = cast(take((V, d), True))
        self.attn_norm, self.wq, self.wk, self.wv, self.wo = [], [], [], [], []
        self.mlp_norm, self.wg, self.wu, self.wd = [], [], [], []
        for _ in range(L):
            self.attn_norm.append(take((d,), False).astype(np.float64))
            self.wq.append(cast(take((d, d), True)))
            self.wk.append(cast(take((d, d), True)))
            self.wv.append(cast(take((d, d), True)))
            self.wo.append(cast(take((d, d), True)))
            self.mlp_norm.append(take((d,), False).astype(np.float64))
            self.wg.append(cast(take((F, d), True)))
            self.wu.append(cast(take((F, d), True)))
            self.wd.append(cast(take((d, F), True)))
        self.gate_w, self.exit_norm, self.head = [], [], []
        self.router_w1, self.router_b1, self.router_w2 = [], [], []
        self.adapter_down, self.adapter_up = [], []
        rr, r = self.router_dim, self.adapter_dim
        for k in range(nx):
            if self.router_mlp:
                self.router_w1.append(take((rr, d), False).astype(np.float64))
                self.router_b1.append(take((rr,), False).astype(np.float64))
                self.router_w2.append(take((rr,), False).astype(np.float64))
            else:
                self.gate_w.append(take((d,), False).astype(np.float64))
            if self.shared_head:
                if k < nx - 1:
                    self.adapter_down.append(take((r, d), True).astype(np.float64))
                    self.adapter_up.append(take((d, r), True).astype(np.float64))
            else:
                self.exit_norm.append(take((d,), False).astype(np.float64))
                self.head.append(cast(take((V, d), True)))
        if self.shared_head:
            self.final_norm = take((d,), False).astype(np.float64)
            shared = cast(take((V, d), True))
            self.head = [shared] * nx
            self.exit_norm = [self.final_norm] * nx
        del raw

    def segment_layers(self, s: int) -> range:
        """0-based layer indices of segment s (0-based): the layers between exits s-1 and s."""
        lo = 0 if s == 0 else self.exit_layers[s - 1]
        return range(lo, self.exit_layers[s])


def lin(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """x @ W^T in float64 (W stored as [out][in])."""
    return x @ W.T.astype(np.float64, copy=False)


# --------------------------------------------------------------------------------------------
# textbook pieces of the LLaMA-2 layer [Results]
# --------------------------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half rotary embedding.  x: [r, H, hd], pos: [r] 0-based positions.

    Pair (i, i + hd/2) is rotated by angle pos * base^(-2i/hd)."""
    hd = x.shape[-1]
    half = hd // 2
    theta = base ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None, None] * theta[None, None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Row i (query at position pos[i]) attends to keys/values at positions 0..pos[i].

    q: [r, H, hd]; K, V: [n, H, hd] holding at least positions 0..max(pos).
    Returns [r, H, hd]: softmax(q K^T / sqrt(hd)) V per head, keys past pos[i] masked."""
    r, H, hd = q.shape
    n = int(np.max(pos)) + 1
    out = np.empty_like(q)
    mask = np.arange(n)[None, :] > np.asarray(pos)[:, None]         # [r, n]
    for h in range(H):
        s = q[:, h, :] @ K[:n, h, :].T / math.sqrt(hd)                # [r, n]
        s = np.where(mask, -np.inf, s)
        out[:, h, :] = softmax(s) @ V[:n, h, :]
    return out


# --------------------------------------------------------------------------------------------
# state: per-layer KV cache [Piggy, Contrib]
# --------------------------------------------------------------------------------------------


class KVCache:
    def __init__(self, M: OracleModel, max_ctx: int):
        self.K = np.zeros((M.L, max_ctx, M.H, M.hd), dtype=np.float64)
        self.V = np.zeros((M.L, max_ctx, M.H, M.hd), dtype=np.float64)
        self.written = np.zeros((M.L, max_ctx), dtype=bool)


def layer_rows(M: OracleModel, l: int, X: np.ndarray, pos: Sequence[int], kv: KVCache) -> np.ndarray:
    """Decoder layer l (0-based) on rows X [r, d] at positions pos (ascending).

    Pre-norm LLaMA-2 block: RMSNorm -> q,k,v -> RoPE -> store k,v at pos ->
    causal attention over positions <= pos[i] -> +o W_o^T -> RMSNorm ->
    + (silu(m W_g^T) * (m W_u^T)) W_d^T.  Rows are a causal chunk: a row sees the
    keys of the chunk rows before it and not those after it."""
    pos = np.asarray(pos, dtype=np.int64)
    r = X.shape[0]
    a = rmsnorm(X, M.attn_norm[l], M.eps)
    q = lin(a, M.wq[l]).reshape(r, M.H, M.hd)
    k = lin(a, M.wk[l]).reshape(r, M.H, M.hd)
    v = lin(a, M.wv[l]).reshape(r, M.H, M.hd)
    q = rope(q, pos, M.rope_base)
    k = rope(k, pos, M.rope_base)
    kv.K[l, pos] = k
    kv.V[l, pos] = v
    kv.written[l, pos] = True
    o = causal_attention(q, kv.K[l], kv.V[l], pos)
    X = X + lin(o.reshape(r, M.d), M.wo[l])
    m = rmsnorm(X, M.mlp_norm[l], M.eps)
    X = X + lin(silu(lin(m, M.wg[l])) * lin(m, M.wu[l]), M.wd[l])
    return X


# --------------------------------------------------------------------------------------------
# exits: router, stick-breaking probabilities, per-exit distributions, mixture [Arch]
# --------------------------------------------------------------------------------------------


def router_logit(M: OracleModel, k: int, h: np.ndarray) -> float:
    """The router's pre-sigmoid output at exit k (0-based, k < N_V - 1) [Arch]: a linear
    gate g_k . h + b_k, or the router MLP w2_k . silu(W1_k h + b1_k) + b_k."""
    if M.router_mlp:
        hidden = silu(M.router_w1[k] @ np.asarray(h, dtype=np.float64) + M.router_b1[k])
        return float(np.dot(M.router_w2[k], hidden)) + M.gate_bias[k]
    return float(np.dot(M.gate_w[k], h)) + M.gate_bias[k]


def gate(M: OracleModel, k: int, h: np.ndarray) -> float:
    """Router output w_k = sigmoid(router logit) for k < N_V - 1 (0-based); w_{N_V} = 1."""
    if k == M.n_exits - 1:
        return 1.0
    z = router_logit(M, k, h)
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    ez = math.exp(z)                       # z = -inf gives exactly 0
    return ez / (1.0 + ez)


def exit_probs(w: Sequence[float]) -> List[float]:
    """p_k = w_k * prod_{j<k} (1 - w_j), with the last w fixed to 1."""
    p, rest = [], 1.0
    for wk in w:
        p.append(wk * rest)
        rest *= 1.0 - wk
    return p


def adapter(M: OracleModel, k: int, h: np.ndarray) -> np.ndarray:
    """Adapter of intermediate exit k (shared head) [Arch, shared head]: a residual
    bottleneck MLP h + U_k silu(D_k h) that maps the exit's hidden state towards the
    geometry the final head expects; the last exit uses h as it is."""
    h = np.asarray(h, dtype=np.float64)
    if k == M.n_exits - 1:
        return h
    return h + M.adapter_up[k] @ silu(M.adapter_down[k] @ h)


def head_logits(M: OracleModel, k: int, h: np.ndarray) -> np.ndarray:
    """Logits of exit k: its own RMSNorm and LM head applied to h, or (shared head) the
    final RMSNorm and LM head applied to the exit's adapter output."""
    if M.shared_head:
        return lin(rmsnorm(adapter(M, k, h), M.final_norm, M.eps), M.head[k])
    return lin(rmsnorm(h, M.exit_norm[k], M.eps), M.head[k])


def mixture(pis: Sequence[np.ndarray], p: Sequence[float]) -> np.ndarray:
    """pi_mix = sum_k p_k pi_k."""
    out = np.zeros_like(pis[0])
    for pk, pik in zip(p, pis):
        out = out + pk * pik
    return out


def walk_gates(w: Sequence[float], u: Sequence[float]) -> int:
    """Exit reached by the gate walk: first k with u_k < w_k, else the last exit (0-based).

    P(exit = k) = w_k prod_{j<k}(1 - w_j) = p_k, so drawing the exit this way and
    then the token from pi_k samples pi_mix exactly."""
    n = len(w)
    for k in range(n - 1):
        if float(u[k]) < w[k]:
            return k
    return n - 1


def inverse_cdf(pi: np.ndarray, u: float) -> int:
    """Smallest i with u < F(i), F the float64 running sum of pi in token-id order;
    if rounding leaves F(V-1) <= u, the largest i with pi(i) > 0."""
    F = np.cumsum(np.asarray(pi, dtype=np.float64))
    i = int(np.searchsorted(F, float(u), side="right"))
    if i < len(F):
        return i
    return int(np.nonzero(np.asarray(pi) > 0)[0][-1])


# --------------------------------------------------------------------------------------------
# sequential full-depth generation (mode 1)
# --------------------------------------------------------------------------------------------


@dataclass
class StepOut:
    pos: int
    token: int
    exit: int                      # 1-based exit index (1..N_V)
    w: List[float]                 # router outputs, w[-1] = 1
    p: List[float]                 # exit probabilities
    logits: List[np.ndarray]       # per exit
    pis: List[np.ndarray]          # per exit, float64 softmax
    h: List[np.ndarray]            # hidden state after each exit's last layer
    u: np.ndarray


@dataclass
class SeqState:
    kv: KVCache
    n: int = 0                     # positions consumed so far


def new_state(M: OracleModel, max_ctx: int) -> SeqState:
    return SeqState(KVCache(M, max_ctx), 0)


def embed(M: OracleModel, tok: int) -> np.ndarray:
    return np.asarray(M.embed[int(tok)], dtype=np.float64)[None, :]


def prefill(M: OracleModel, st: SeqState, tokens: Sequence[int]) -> None:
    """Every layer over the given prompt positions (a causal chunk)."""
    n = len(tokens)
    if n == 0:
        return
    pos = np.arange(st.n, st.n + n)
    X = np.asarray(M.embed[np.asarray(tokens, dtype=np.int64)], dtype=np.float64)
    for l in range(M.L):
        X = layer_rows(M, l, X, pos, st.kv)
    st.n += n


def decode_step(M: OracleModel, st: SeqState, y: int, u: Sequence[float],
                all_heads: bool = True) -> StepOut:
    """Consume token y at the next position, full depth, and sample the next token."""
    pos = st.n
    x = embed(M, y)
    hs = []
    ex = set(M.exit_layers)
    for l in range(M.L):
        x = layer_rows(M, l, x, [pos], st.kv)
        if (l + 1) in ex:
            hs.append(x[0].copy())
    w = [gate(M, k, hs[k]) for k in range(M.n_exits)]
    p = exit_probs(w)
    e = walk_gates(w, u)
    heads = range(M.n_exits) if all_heads else [e]
    logits = [None] * M.n_exits
    pis = [None] * M.n_exits
    for k in heads:
        logits[k] = head_logits(M, k, hs[k])
        pis[k] = softmax(logits[k])
    tok = inverse_cdf(pis[e], float(u[3]))
    st.n += 1
    return StepOut(pos, tok, e + 1, w, p, logits, pis, hs, np.asarray(u))


def generate(M: OracleModel, prompt: Sequence[int], U: np.ndarray, max_ctx: int = None,
             forced: Optional[Sequence[int]] = None, all_heads: bool = True):
    """Prefill prompt[:-1], then one decode step per row of U (U[t] = 4 uniforms).

    The input of step 0 is prompt[-1]; the input of step t > 0 is the token sampled
    at step t-1, or forced[t-1] when forced tokens are given."""
    steps = len(U)
    st = new_state(M, max_ctx or (len(prompt) + steps))
    prefill(M, st, prompt[:-1])
    y = int(prompt[-1])
    outs = []
    for t in range(steps):
        o = decode_step(M, st, y, U[t], all_heads=all_heads)
        outs.append(o)
        y = o.token if forced is None else int(forced[t])
    return outs, st


# --------------------------------------------------------------------------------------------
# forward-only training objective [Arch, training part]
# --------------------------------------------------------------------------------------------


@dataclass
class LossOut:
    L_mix: float           # mean over positions of -log pi_mix(x_{t+1} | x_{1:t})
    L_compute: float       # mean over positions of sum_k p_k * l_k / L
    L_total: float         # L_mix + beta * L_compute
    nll_mix: np.ndarray    # [n-1] per-position -log pi_mix
    depth: np.ndarray      # [n-1] per-position expected normalised depth
    logp: np.ndarray       # [n-1][N_V] log pi_k(x_{t+1})
    w: np.ndarray          # [n-1][N_V] router outputs


def log_softmax_at(z: np.ndarray, y: int) -> float:
    z = np.asarray(z, dtype=np.float64)
    mx = float(np.max(z))
    return float(z[y] - mx - math.log(float(np.sum(np.exp(z - mx)))))


def mixture_loss(M: OracleModel, tokens: Sequence[int], beta: float = 0.0) -> LossOut:
    """The mixture objective on a token sequence, forward only: positions t = 0..n-2 run
    every layer (a causal chunk), each exit k gives w_k and log pi_k(x_{t+1}); the
    stick-breaking p_k mix them: L_mix is the cross-entropy of pi_mix and L_compute the
    expected exit depth l_k / L, both averaged over the n-1 positions."""
    tokens = [int(t) for t in tokens]
    n = len(tokens)
    r = n - 1
    kv = KVCache(M, r)
    X = np.asarray(M.embed[np.asarray(tokens[:r], dtype=np.int64)], dtype=np.float64)
    pos = np.arange(r)
    logp = np.zeros((r, M.n_exits))
    w = np.zeros((r, M.n_exits))
    k = 0
    for l in range(M.L):
        X = layer_rows(M, l, X, pos, kv)
        if l + 1 == M.exit_layers[k]:
            for i in range(r):
                w[i, k] = gate(M, k, X[i])
                logp[i, k] = log_softmax_at(head_logits(M, k, X[i]), tokens[i + 1])
            k += 1
    nll = np.zeros(r)
    depth = np.zeros(r)
    for i in range(r):
        p = exit_probs(list(w[i]))
        terms = [math.log(p[j]) + logp[i, j] for j in range(M.n_exits) if p[j] > 0.0]
        mx = max(terms)
        nll[i] = -(mx + math.log(sum(math.exp(t - mx) for t in terms)))
        depth[i] = sum(p[j] * M.exit_layers[j] / M.L for j in range(M.n_exits))
    L_mix, L_comp = float(np.mean(nll)), float(np.mean(depth))
    return LossOut(L_mix, L_comp, L_mix + beta * L_comp, nll, depth, logp, w)


def boundary_distances(o: StepOut, token: int, exit_: int) -> dict:
    """How close the draw that produced (token, exit_) sits to this step's decision
    boundaries: per walked gate |u_k - w_k|, and for the token the distance of u_4
    to the CDF interval [F(token-1), F(token)) of the exit's distribution."""
    gates = [abs(float(o.u[k]) - o.w[k]) for k in range(min(exit_, len(o.w) - 1))]
    pi = o.pis[exit_ - 1]
    tok_d = None
    if pi is not None:
        F = np.cumsum(pi)
        lo = F[token - 1] if token > 0 else 0.0
        hi = F[token]
        u4 = float(o.u[3])
        tok_d = min(abs(u4 - lo), abs(hi - u4))
    return {"gates": gates, "token": tok_d}
