"""Writes loss_1p5b_a128.json: the oracle's mixture objective (beta 0.5) on the first
128 tokens of the 1.5B single-sequence workload's synthetic prompt, with its per-position
router outputs, log pi_k of the targets, -log pi_mix and expected depths.  Calls only the
oracle and the seeded generators.  Run from the repository root:
    python -m tests.golden.make_loss_1p5b [weights_dir]"""
import json
import os
import sys

from oracle import model as om
from synth import cached_weights, prompts, workload

N_TOKENS, BETA = 128, 0.5


def main(weights_dir: str) -> None:
    w = workload("A")
    tokens = [int(t) for t in prompts(w)[0][:N_TOKENS]]
    M = om.OracleModel(cached_weights(w.model, weights_dir))
    r = om.mixture_loss(M, tokens, BETA)
    out = {"workload": "A", "model": "1.5B bf16 own heads, linear gates", "n_tokens": N_TOKENS, "beta": BETA,
           "tokens": tokens, "L_mix": r.L_mix, "L_compute": r.L_compute, "L_total": r.L_total,
           "w": r.w.tolist(), "logp": r.logp.tolist(), "nll_mix": r.nll_mix.tolist(), "depth": r.depth.tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "loss_1p5b_a128.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print(path, r.L_mix, r.L_compute)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "/tmp/nvium_weights")
