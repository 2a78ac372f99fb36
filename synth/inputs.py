"""Seeded synthetic decode inputs: prompts and per-step uniforms.

The pages measure on C4 text with the LLaMA-2 tokenizer; with random-init
weights, throughput depends only on shapes, context lengths and the exit
pattern, so token ids are drawn i.i.d. uniform over the vocabulary instead.

  prompts   numpy default_rng(prompt_seed): for a range of prompt lengths the
            lengths are drawn first (integers, inclusive range), then each
            sequence's token ids in order.
  uniforms  numpy default_rng(uniform_seed).random((steps, batch, 4), float32),
            values in [0, 1): entries 0..2 walk the three intermediate gates,
            entry 3 draws the token.
"""
from __future__ import annotations

from typing import List

import numpy as np

from .configs import Workload


def prompts(w: Workload) -> List[np.ndarray]:
    rng = np.random.default_rng(w.prompt_seed)
    if w.prompt_len is not None:
        lens = [w.prompt_len] * w.batch
    else:
        lo, hi = w.prompt_len_range
        lens = [int(x) for x in rng.integers(lo, hi + 1, size=w.batch)]
    return [rng.integers(0, w.model.vocab, size=n, dtype=np.int64).astype(np.int32) for n in lens]


def uniforms(w: Workload, steps: int = None) -> np.ndarray:
    steps = w.decode_steps if steps is None else steps
    rng = np.random.default_rng(w.uniform_seed)
    return rng.random((steps, w.batch, 4), dtype=np.float32)
