"""Deferred-schedule simulator of N-vium decoding (oracle mode 2).

TEST INFRASTRUCTURE (see oracle/model.py).

Follows the "Inferenz: Piggybacking" part of section 2 of the gist.science
technical summary and the abstract: when a token exits at node k its layers
above the exit are not run; when a later token reaches those depths, the
deferred tokens' hidden states are concatenated with the current token's and
run together, so that every layer's KV cache ends up complete.

Bookkeeping (a reading of that passage): segment s (0-based) is the run of
layers between exits s-1 and s.  A frontier f[s] per segment says that every
position < f[s] has completed segment s.  Frontiers never increase with s
(a position that passed segment s+1 passed segment s), so the positions pending
at segment s form the contiguous range [f[s], p] once the current position p
arrives there.  Each position keeps one hidden state: the output of the last
segment it completed.  A flush runs, for s = 1, 2, ..., every pending range up to
the last consumed position, with no gates and no heads.

Two chunk orders are offered: "row" runs the chunk one position at a time
through all of the segment's layers (the same arithmetic as mode 1, so results
are bit-identical to it); "layer" runs the whole chunk through one layer at a
time as a causal batch (the order a batched device implementation uses).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

from .model import (OracleModel, embed, gate, head_logits, inverse_cdf, layer_rows,
                    new_state, prefill, softmax)


@dataclass
class DeferredRun:
    tokens: List[int]
    exits: List[int]                  # 1-based
    chunk_rows: List[List[int]]       # per step, rows run at each reached segment
    frontiers: List[List[int]]        # per step, frontiers after the step
    state: object                     # SeqState (KV cache)
    hidden: dict                      # position -> last hidden state


def _run_segment(M: OracleModel, s: int, H: dict, lo: int, hi: int, kv, order: str) -> None:
    """Run segment s over positions lo..hi-1 (ascending), updating H in place."""
    if hi <= lo:
        return
    layers = M.segment_layers(s)
    if order == "row":
        for q in range(lo, hi):
            x = H[q][None, :]
            for l in layers:
                x = layer_rows(M, l, x, [q], kv)
            H[q] = x[0]
    elif order == "layer":
        pos = list(range(lo, hi))
        X = np.stack([H[q] for q in pos])
        for l in layers:
            X = layer_rows(M, l, X, pos, kv)
        for i, q in enumerate(pos):
            H[q] = X[i]
    else:
        raise ValueError(order)


def generate_deferred(M: OracleModel, prompt: Sequence[int], U: np.ndarray, max_ctx: int = None,
                      forced: Sequence[int] = None, flush: bool = True,
                      order: str = "row") -> DeferredRun:
    steps = len(U)
    st = new_state(M, max_ctx or (len(prompt) + steps))
    prefill(M, st, prompt[:-1])
    P = len(prompt) - 1
    nseg = M.n_exits
    f = [P] * nseg
    H = {}
    y = int(prompt[-1])
    tokens, exits, rows_log, front_log = [], [], [], []
    for t in range(steps):
        p = P + t
        H[p] = embed(M, y)[0]
        u = U[t]
        rows = []
        e = nseg - 1
        for s in range(nseg):
            rows.append(p + 1 - f[s])
            _run_segment(M, s, H, f[s], p + 1, st.kv, order)
            f[s] = p + 1
            if s < nseg - 1:
                if float(u[s]) < gate(M, s, H[p]):      # stop at this exit
                    e = s
                    break
        tok = inverse_cdf(softmax(head_logits(M, e, H[p])), float(u[3]))
        tokens.append(tok)
        exits.append(e + 1)
        rows_log.append(rows)
        front_log.append(list(f))
        y = tok if forced is None else int(forced[t])
    st.n = P + steps
    if flush:
        end = P + steps
        for s in range(nseg):
            _run_segment(M, s, H, f[s], end, st.kv, order)
            f[s] = end
    return DeferredRun(tokens, exits, rows_log, front_log, st, H)
