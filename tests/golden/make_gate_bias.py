"""Gate biases that realise the stated exit masses on the 1.5B model (calls only oracle/).

With random-init weights the residual stream after a segment has norm ~85-180, so the
linear term g_k . h of a gate (g_k ~ N(0, 0.02^2)) has a standard deviation near 2 and
sigmoid(b_k) alone does not give the stated marginal exit masses.  The marginal mass of
exit k is the mean over tokens of p_k = w_k prod_{j<k} (1 - w_j), with w_k = sigmoid(g_k .
h^(l_k) + b_k) (gist.science summary, section 2 "Methodik", part "Architektur": equation
for p_k).  The linear term drifts with the position (gate 1's mean falls from about +1.2
at positions 64-164 to -1.0 at 896-1023), so each workload is calibrated where it decodes.
This script runs the oracle's float64 forward over each workload's own prompt followed by
its decode steps' worth of seeded uniform-random tokens (stand-ins for the drawn tokens,
which random-init heads spread near-uniformly over the vocabulary), through the first three
segments (the gates need no more); it keeps z_k = g_k . h^(l_k) at the positions the decode
steps consume, and solves, exit by exit, for the b_k whose sample mean of p_k equals the
stated mass (p_k is increasing in b_k when the earlier biases are fixed; bisection in
float64):
  A (512-token prompt, 512 steps):   positions 511..1022, continuation default_rng(3)
  D (8192-token prompt, 256 steps):  positions 8191..8446, continuation default_rng(4)

    python tests/golden/make_gate_bias.py       # writes tests/golden/gate_bias_1p5b.json
"""
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import model as om                       # noqa: E402
from synth import M15B, cached_weights, prompts, workload   # noqa: E402

MASSES = {"A": (0.4, 0.25, 0.2, 0.15), "D": (0.6, 0.2, 0.1, 0.1)}
SAMPLES = {"A": 3, "D": 4}     # seed of the continuation tokens


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def solve_biases(z: np.ndarray, masses) -> list:
    """z: [n][3] linear terms; the biases b_1..b_3 whose sample-mean exit masses equal
    masses[0..2] (the last exit takes the rest)."""
    rest = np.ones(z.shape[0])
    out = []
    for k in range(3):
        target = masses[k]
        lo, hi = -60.0, 60.0
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if float(np.mean(rest * sig(z[:, k] + mid))) < target:
                lo = mid
            else:
                hi = mid
        b = 0.5 * (lo + hi)
        out.append(b)
        rest = rest * (1.0 - sig(z[:, k] + b))
    return out


def sample_z(M, tokens: np.ndarray, first_pos: int) -> np.ndarray:
    """The gates' linear terms z_k = g_k . h^(l_k) (k < 3) at positions first_pos..len-2 of
    `tokens`, from the oracle's layers (a causal chunk per layer)."""
    n = len(tokens) - 1
    kv = om.KVCache(M, n)
    pos = np.arange(n)
    X = np.asarray(M.embed[tokens[:n]], dtype=np.float64)
    z = np.zeros((n, 3))
    for l in range(M.exit_layers[2]):
        X = om.layer_rows(M, l, X, pos, kv)
        for k in range(3):
            if l + 1 == M.exit_layers[k]:
                z[:, k] = X @ M.gate_w[k]
        print(f"{len(tokens)} tokens: layer {l + 1}/{M.exit_layers[2]}", flush=True)
    return z[first_pos:]


def main():
    path = cached_weights(M15B)
    M = om.OracleModel(path)
    res = {"source": "tests/golden/make_gate_bias.py (oracle float64 forward, 1.5B model, seed-0 weights)"}
    for name, seed in SAMPLES.items():
        wl = workload(name)
        prompt = prompts(wl)[0].astype(np.int64)
        cont = np.random.default_rng(seed).integers(0, M.V, size=wl.decode_steps)
        tokens = np.concatenate([prompt, cont])
        first = len(prompt) - 1
        zs = sample_z(M, tokens, first)
        assert len(zs) == wl.decode_steps
        b = solve_biases(zs, MASSES[name])
        res[name] = {"prompt": f"workload {name}'s prompt ({len(prompt)} tokens), then {wl.decode_steps} "
                               f"uniform-random tokens, numpy default_rng({seed})",
                     "positions": [first, first + wl.decode_steps - 1], "mass": list(MASSES[name]), "bias": b,
                     "z_mean": [float(np.mean(zs[:, k])) for k in range(3)],
                     "z_std": [float(np.std(zs[:, k])) for k in range(3)],
                     "z": [[round(float(v), 9) for v in row] for row in zs]}
        print(name, "biases", b, flush=True)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gate_bias_1p5b.json")
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
