"""Named model shapes and decode workloads (pure data, no model arithmetic).

Five workloads share one model family: a LLaMA-2-style decoder whose depth is cut
into four equal segments, each ending in an exit (halting gate + own LM head).  A sixth
(E) uses the exit form of the N-vium pages instead: every exit reads the one final LM
head through a light adapter MLP, and the halting gate is a small router MLP.

  T  tiny fp32 model, batch 1, 64-token prompt, 64 decode steps
  A  1.5B bf16 model, batch 1, 512-token prompt, 512 decode steps
  B  model A with every intermediate gate bias at -inf (all mass on exit 4)
  C  model A, 16 independent sequences, prompt lengths uniform in [256, 1024],
     256 decode steps each
  D  model A with exit mass skewed early, batch 1, 8192-token prompt, 256 steps
  E  model A with a shared head + adapters (bottleneck 192) and router MLPs (hidden 64),
     batch 1, 512-token prompt, 512 steps

Gate biases.  Each intermediate gate is sigmoid(g_k . h + b_k); with the linear
term at zero the conditional stop probability of gate k is sigmoid(b_k), and the
marginal exit masses follow from the stick-breaking product.  The biases below
are the logits of the conditional stop probabilities that give the stated
marginal masses at a zero linear term:
  masses (0.4, 0.25, 0.2, 0.15): conditional stops 0.4, 0.25/0.6, 0.2/0.35
  masses (0.6, 0.2, 0.1, 0.1):   conditional stops 0.6, 0.2/0.4,  0.1/0.2
With random-init weights the residual stream after a segment has norm ~85-180, so the
linear term g_k . h (g_k ~ N(0, 0.02^2)) of the 1.5B model has a standard deviation of
1.2-1.7 and a nonzero mean, and sigmoid(b_k) alone does not give the stated masses.  The
1.5B workloads therefore use calibrated biases: the b_k for which the mean of p_k over the
oracle's hidden states at the positions the workload decodes (511-1022 after the 512-token
prompt, 8191-8446 after the 8192-token one; the linear term drifts with the position and
with the prompt, so the workload's own prompt comes first and seeded uniform-random tokens
stand in for the drawn ones) equals the stated mass (tests/golden/make_gate_bias.py writes them, with the samples, to
tests/golden/gate_bias_1p5b.json).  The tiny model's linear term is small, so it keeps the
zero-linear-term biases.  Benchmarks report the realised exit histogram.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

NEG_INF = float("-inf")

# logit(0.4), logit(5/12), logit(4/7)
BIAS_MASS_40_25_20_15 = (math.log(0.4 / 0.6), math.log(5.0 / 7.0), math.log(4.0 / 3.0))
# logit(0.6), logit(0.5), logit(0.5)
BIAS_MASS_60_20_10_10 = (math.log(0.6 / 0.4), 0.0, 0.0)
# 1.5B model, calibrated on the oracle's hidden states at the decode positions of workload A
# (also used by the other 512-token-prompt workloads and C) and of workload D
# (tests/golden/gate_bias_1p5b.json)
BIAS_CAL_1P5B_40_25_20_15 = (-0.7148283503446942, -2.054615047072935, 0.9033168998118104)
BIAS_CAL_1P5B_60_20_10_10 = (-0.34100759331458186, -1.1546249822822858, -0.2721350662432206)
# every intermediate gate closed: sigmoid(-inf) = 0
BIAS_ALL_LAST = (NEG_INF, NEG_INF, NEG_INF)


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    ffn: int
    vocab: int
    wdtype: str                      # "f32" or "bf16": storage type of matrices
    gate_bias: Tuple[float, float, float]
    n_exits: int = 4
    norm_eps: float = 1e-5
    rope_base: float = 1e4
    init_std: float = 0.02
    seed: int = 0
    head: str = "own"                # "own": a norm + LM head per exit; "shared": one final
                                     # norm + LM head, intermediate exits through an adapter
    adapter_dim: int = 0             # adapter bottleneck width (head "shared")
    router: str = "linear"           # "linear": sigmoid(g.h + b); "mlp": sigmoid(w2.silu(W1 h + b1) + b)
    router_dim: int = 0              # router hidden width (router "mlp")

    @property
    def exit_layers(self) -> Tuple[int, ...]:
        """1-based index of the layer after which exit k (1..n_exits) sits."""
        step = self.n_layers // self.n_exits
        return tuple(step * (k + 1) for k in range(self.n_exits))

    @property
    def seg_layers(self) -> int:
        return self.n_layers // self.n_exits


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int
    prompt_len: Optional[int]                 # fixed prompt length, or None
    prompt_len_range: Optional[Tuple[int, int]] = None   # inclusive range, drawn per sequence
    decode_steps: int = 0
    prompt_seed: int = 1
    uniform_seed: int = 2
    note: str = ""

    @property
    def max_prompt(self) -> int:
        if self.prompt_len is not None:
            return self.prompt_len
        return self.prompt_len_range[1]

    @property
    def max_ctx(self) -> int:
        return self.max_prompt + self.decode_steps


TINY = ModelShape(n_layers=8, d_model=128, n_heads=4, head_dim=32, ffn=352, vocab=512,
                  wdtype="f32", gate_bias=BIAS_MASS_40_25_20_15)
M15B = ModelShape(n_layers=48, d_model=1536, n_heads=12, head_dim=128, ffn=4096, vocab=32000,
                  wdtype="bf16", gate_bias=BIAS_CAL_1P5B_40_25_20_15)

WORKLOADS = {
    "T": Workload("T", TINY, batch=1, prompt_len=64, decode_steps=64,
                  note="tiny fp32 N-vium, batch 1, prompt 64, decode 64"),
    "A": Workload("A", M15B, batch=1, prompt_len=512, decode_steps=512,
                  note="1.5B bf16 N-vium, batch 1, prompt 512, decode 512, exit mass ~[.4,.25,.2,.15]"),
    "B": Workload("B", replace(M15B, gate_bias=BIAS_ALL_LAST), batch=1, prompt_len=512,
                  decode_steps=512,
                  note="1.5B bf16, gate biases -inf (exit 4 forced), batch 1, prompt 512, decode 512"),
    "C": Workload("C", M15B, batch=16, prompt_len=None, prompt_len_range=(256, 1024),
                  decode_steps=256,
                  note="1.5B bf16, 16 independent sequences, prompts uniform in [256,1024], decode 256"),
    "D": Workload("D", replace(M15B, gate_bias=BIAS_CAL_1P5B_60_20_10_10), batch=1, prompt_len=8192,
                  decode_steps=256,
                  note="1.5B bf16, batch 1, prompt 8192, decode 256, exit mass ~[.6,.2,.1,.1]"),
    "E": Workload("E", replace(M15B, gate_bias=BIAS_MASS_40_25_20_15, head="shared", adapter_dim=192, router="mlp",
                                 router_dim=64), batch=1,
                  prompt_len=512, decode_steps=512,
                  note="1.5B bf16, shared LM head + adapters (192), router MLPs (64), batch 1, prompt 512, "
                       "decode 512, exit mass ~[.4,.25,.2,.15]"),
    "L": Workload("L", M15B, batch=1, prompt_len=2048, decode_steps=0,
                  note="mixture objective (L_mix + beta L_compute, forward) over one 2048-token sequence, "
                       "1.5B bf16, every exit's router and head at every position"),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def tiny_variant(**model_overrides) -> ModelShape:
    """A tiny model with some fields changed (tests use e.g. vocab=16 or fewer layers)."""
    return replace(TINY, **model_overrides)
