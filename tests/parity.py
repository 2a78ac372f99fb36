"""Helpers that compare the HIP path (through the C ABI) with the oracle.

The oracle decodes on its own (its own samples).  The device is fed the oracle's
tokens as next inputs (nv_step_forced), so both consume the same context at every
step even where a draw lands near a decision boundary; the device's own draw at each
step is then compared with the oracle's.

Token and exit rule: they must be equal, except that a difference is accepted when
the draw lies within `band` of the oracle's decision boundary (|u_k - w_k| for a
walked gate, distance of u_4 to the oracle CDF interval of either token).  Such
draws are counted and reported.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from oracle import model as om

BAND = 1e-5


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


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

    def summary(self) -> str:
        return (f"steps {self.steps} exits equal {self.exit_equal} tokens equal {self.token_equal} "
                f"near-boundary(1e-5) {self.near_boundary} within-cdf-shift {self.logit_explained} "
                f"within-gate-shift {self.gate_explained} "
                f"max logit rel {self.max_logit_rel:.2e} max gate abs {self.max_gate_abs:.2e} "
                f"max cdf shift {self.max_cdf_shift:.2e}")


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
        elif dist <= wshift:                     # the draw lies between the two gate values
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
