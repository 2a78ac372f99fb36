"""Helpers that compare the HIP path (through the C ABI) with the oracle.

The oracle decodes on its own (its own samples).  The device is fed the oracle's
tokens as next inputs (nv_step_forced), so both consume the same context at every
step even where a draw lands near a decision boundary; the device's own draw at each
step is then compared with the oracle's.

Token and exit rule: they must be equal, except that a difference is accepted when
the draw lies within `band` of the oracle's decision boundary (|u_k - w_k| for a
walked gate, distance of u_4 to the oracle CDF interval of either token).  Such
draws are counted and reported.  On bf16 paths a difference is also accepted when the
draw lies between the oracle's and the device's gate value, or inside the CDF shift
that the device's tolerance-checked logits imply; `finish` bounds how often that may
happen and how far the device's gate values may sit from the oracle's.

Tensor comparisons are made per row (one position, or one (position, head) of the KV
cache), so that an error confined to a few decoded or deferred rows is not diluted by
hundreds of prompt rows.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from oracle import model as om

BAND = 1e-5
# The device's token must be the inverse-CDF draw of its own (reported, float32) logits:
# its float32 exponentials summed in float64 put each CDF boundary within ~1e-7 of the
# float64 CDF of those logits, so only draws this close to a boundary may differ.
SELF_BAND = 1e-6
# bf16 paths: largest accepted |w_device - w_oracle| of a walked gate.  The 1.5B model's
# residual stream has norm ~85-180 after a segment, so bf16 rounding in 12-48 layers moves
# g . h by a few 1e-3 (measured up to 5.9e-3).
GATE_BOUND_BF16 = 1e-2


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def row_rel(a, b, width: int) -> np.ndarray:
    """Relative error of every row of `width` values: ||a_i - b_i|| / ||b_i||."""
    a = np.asarray(a, np.float64).reshape(-1, width)
    b = np.asarray(b, np.float64).reshape(-1, width)
    return np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-300)


def row_rel_max(a, b, width: int) -> float:
    r = row_rel(a, b, width)
    return float(r.max()) if r.size else 0.0


@dataclass
class StepCheck:
    steps: int = 0
    exit_equal: int = 0
    token_equal: int = 0
    near_boundary: int = 0
    unexplained: List[str] = field(default_factory=list)
    max_logit_rel: float = 0.0
    max_gate_abs: float = 0.0
    max_cdf_shift: float = 0.0
    logit_explained: int = 0
    gate_explained: int = 0
    self_near: int = 0             # draws within SELF_BAND of a boundary of the device's own CDF

    def summary(self) -> str:
        return (f"steps {self.steps} exits equal {self.exit_equal} tokens equal {self.token_equal} "
                f"near-boundary(1e-5) {self.near_boundary} within-cdf-shift {self.logit_explained} "
                f"within-gate-shift {self.gate_explained} "
                f"max logit rel {self.max_logit_rel:.2e} max gate abs {self.max_gate_abs:.2e} "
                f"max cdf shift {self.max_cdf_shift:.2e} self-near(1e-6) {self.self_near}")

    def finish(self, logit_tol: float, gate_bound: float = GATE_BOUND_BF16, max_logit_explained=1,
               max_gate_explained: int = 1) -> None:
        """Assert the run's outcome: no unexplained mismatch, logits within `logit_tol`,
        walked gates within `gate_bound` of the oracle's, and at most the given number of
        draws accepted only through the widened (bf16) bands (max_logit_explained None: any
        number, for vocabularies whose token intervals are narrower than the CDF shift the
        logit tolerance allows; each such draw still has to be the exact draw of the
        device's own logits)."""
        print(self.summary())
        assert not self.unexplained, self.unexplained
        assert self.max_logit_rel < logit_tol, self.max_logit_rel
        assert self.max_gate_abs < gate_bound, self.max_gate_abs
        if max_logit_explained is not None:
            assert self.logit_explained <= max_logit_explained, self.logit_explained
        assert self.gate_explained <= max_gate_explained, self.gate_explained


def cdf_shift(g_logits, pi_oracle) -> float:
    """Largest gap between the CDF implied by the device's logits and the oracle's CDF
    (float64, token-id order)."""
    z = np.asarray(g_logits, np.float64)
    e = np.exp(z - z.max())
    return float(np.max(np.abs(np.cumsum(e / e.sum()) - np.cumsum(pi_oracle))))


def check_step(t: int, o: om.StepOut, g_tok: int, g_exit: int, g_logits, g_w, res: StepCheck,
               band: float = BAND, logit_band: bool = False) -> None:
    """logit_band: for reduced-precision paths, also accept a token difference when the
    draw lies within the CDF shift that the device's (tolerance-checked) logits imply, and
    an exit difference when the draw lies between the device's and the oracle's gate value."""
    res.steps += 1
    u = o.u
    # the device's own decisions are exact: its exit is the walk over the gate values it
    # reports, its token the inverse CDF of the logits it reports
    own_exit = next((k + 1 for k in range(3) if np.isfinite(g_w[k]) and float(u[k]) < float(g_w[k])), 4)
    if own_exit != g_exit:
        res.unexplained.append(f"step {t}: device exit {g_exit} is not the walk over its own gates ({own_exit})")
        return
    if g_logits is not None:
        z = np.asarray(g_logits, np.float64)
        e = np.exp(z - z.max())
        Fd = np.cumsum(e / e.sum())
        own_tok = om.inverse_cdf(e / e.sum(), float(u[3]))
        if own_tok != g_tok:
            lo = Fd[g_tok - 1] if g_tok > 0 else 0.0
            dist = min(abs(float(u[3]) - lo), abs(Fd[g_tok] - float(u[3])))
            if dist < SELF_BAND:
                res.self_near += 1
            else:
                res.unexplained.append(f"step {t}: device token {g_tok} is not the draw of its own logits "
                                       f"({own_tok}, distance {dist:.3g})")
                return
    # gates: the device reports w for every gate it walked
    for k in range(min(g_exit, 3)):           # gates the device walked
        if np.isfinite(g_w[k]):
            res.max_gate_abs = max(res.max_gate_abs, abs(float(g_w[k]) - o.w[k]))
    if g_exit == o.exit:
        res.exit_equal += 1
    else:
        k = min(g_exit, o.exit) - 1              # the gate where the two walks part
        dist = abs(float(u[k]) - o.w[k])
        wshift = abs(float(g_w[k]) - o.w[k]) if (logit_band and np.isfinite(g_w[k])) else 0.0
        if dist < band:
            res.near_boundary += 1
        elif dist <= wshift <= GATE_BOUND_BF16:  # the draw lies between the two gate values
            res.gate_explained += 1
        else:
            res.unexplained.append(f"step {t}: exit device {g_exit} oracle {o.exit} (gate distance {dist:.3g})")
            return
    # token: compare with the oracle's draw from the exit the device used
    pi = o.pis[g_exit - 1]
    want = om.inverse_cdf(pi, float(u[3]))
    if g_logits is not None:
        res.max_logit_rel = max(res.max_logit_rel, rel(g_logits, o.logits[g_exit - 1]))
    if g_tok == want:
        res.token_equal += 1
        return
    F = np.cumsum(pi)
    u4 = float(u[3])
    d1 = om.boundary_distances(o, g_tok, g_exit)["token"]
    d2 = min(abs(u4 - (F[want - 1] if want > 0 else 0.0)), abs(F[want] - u4))
    shift = cdf_shift(g_logits, pi) if (logit_band and g_logits is not None) else 0.0
    res.max_cdf_shift = max(res.max_cdf_shift, shift)
    if min(d1, d2) < band:
        res.near_boundary += 1
    elif min(d1, d2) < shift:
        res.logit_explained += 1
    else:
        res.unexplained.append(f"step {t}: token device {g_tok} oracle {want} (cdf distance {min(d1, d2):.3g})")


def kv_rows_worst(lib, h, seq: int, st, layers, positions) -> float:
    """Largest per-(position, head) relative error of K and V over `layers` at the given
    positions (device after a flush against the oracle's cache `st`)."""
    positions = np.asarray(sorted(positions), dtype=np.int64)
    if positions.size == 0:
        return 0.0
    p0, p1 = int(positions[0]), int(positions[-1]) + 1
    worst = 0.0
    for l in layers:
        k, v = lib.nv_debug_kv(h, seq, l, p0, p1 - p0)
        sel = positions - p0
        hd = k.shape[-1]
        worst = max(worst, row_rel_max(k[sel], st.kv.K[l, positions], hd),
                    row_rel_max(v[sel], st.kv.V[l, positions], hd))
    return worst


def decoded_kv_report(lib, h, seq: int, st, layers, pos0: int, exits, seg_layers: int) -> dict:
    """Per-row KV errors at the decoded positions pos0, pos0+1, ..., split by how each
    (position, layer) was computed: 'direct' when the position's own token reached the
    layer, 'deferred' when it ran later in a catch-up chunk or at the flush; plus the
    prompt rows before pos0.  Returns the worst value of each group."""
    out = {"direct": 0.0, "deferred": 0.0, "prompt": 0.0}
    for l in layers:
        s = l // seg_layers
        direct = [pos0 + t for t, e in enumerate(exits) if s < e]
        deferred = [pos0 + t for t, e in enumerate(exits) if s >= e]
        out["direct"] = max(out["direct"], kv_rows_worst(lib, h, seq, st, [l], direct))
        out["deferred"] = max(out["deferred"], kv_rows_worst(lib, h, seq, st, [l], deferred))
        out["prompt"] = max(out["prompt"], kv_rows_worst(lib, h, seq, st, [l], range(pos0)))
    return out


def hidden_rows_worst(lib, h, seq: int, outs, pos0: int) -> float:
    """After a flush every decoded position has completed the last layer: its hidden row
    must equal the oracle's state after the last layer (per-row relative error)."""
    n = len(outs)
    got = lib.nv_debug_hidden(h, seq, pos0, n)
    want = np.stack([o.h[-1] for o in outs])
    return row_rel_max(got, want, want.shape[-1])


def run_forced(h, lib, outs: List[om.StepOut], seq_index: int = 0, batch: int = 1, other_inputs=None):
    """Step the device along the oracle's tokens; returns per-step (token, exit, logits, w)."""
    recs = []
    for t, o in enumerate(outs):
        U = np.zeros((batch, 4), np.float32)
        U[seq_index] = o.u
        nxt = np.zeros(batch, np.int32)
        nxt[seq_index] = o.token
        tok, ex = lib.nv_step_forced(h, U, nxt)
        recs.append((int(tok[seq_index]), int(ex[seq_index]), lib.nv_debug_logits(h, seq_index),
                     lib.nv_debug_gates(h, seq_index)))
    return recs
