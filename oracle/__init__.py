"""CPU oracle of the N-vium decode step (float64 NumPy).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg import it; the HIP path never does.

Parity status per function (pins are in tests/test_oracle_*.py):
  rmsnorm, silu, softmax, causal_attention   pinned: torch.nn.functional routines
  rope                                       pinned: complex-rotation form + relative-position invariance
  layer_rows, prefill, decode_step           pinned: independent torch LLaMA forward (strict generalisation),
                                             every exit's hidden state and logits at its exit layer
  gate, exit_probs                           pinned: closed forms (sum to 1, stated exit masses)
  walk_gates, inverse_cdf, mixture           pinned: brute force + chi-square against pi_mix
  generate_deferred                          pinned: bit-identity with sequential decoding,
                                             brute force over forced exit patterns
  head_logits (every exit)                   pinned: the textbook forward's exit norm + head at each
                                             exit layer (test_exit4_is_standard_transformer)
  router_logit/gate, router MLP form         pinned: closed forms (zero output layer, zero first
                                             layer, one active weight per layer)
  adapter, head_logits, shared-head form     pinned: closed form with one active weight per
                                             matrix; identity adapters give the textbook
                                             forward's exit logits
  sampling and deferral, second form         pinned: chi-square against pi_mix and p_k;
                                             bit-identity with sequential decoding
  mixture_loss (L_mix, L_compute)            pinned: closed gates / open first gate give the
                                             textbook forward's cross-entropy and depth 1 / l_1/L;
                                             Jensen bounds; exp(-nll) equals the sampler's pi_mix
"""
from . import model, deferred  # noqa: F401
