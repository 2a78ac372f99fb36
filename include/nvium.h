/*
 * nvium.h -- C ABI of the N-vium mixture-of-exits decode library (HIP, gfx950).
 *
 * The method (arXiv 2605.13190, "N-vium: Mixture-of-Exits Transformer for
 * Accelerated Exact Generation"): a LLaMA-2-style decoder is cut into four depth
 * segments; after each segment an exit holds a router w_k (here the linear gate
 * sigmoid(g_k . h + b_k), the last one fixed to 1) and its own RMSNorm + LM head.
 * The next-token distribution is the mixture pi_mix = sum_k p_k pi_k with the
 * stick-breaking weights p_k = w_k prod_{j<k}(1 - w_j) (gist.science technical
 * summary, section 2 "Methodik", part "Architektur", equations for p_k and
 * pi_mix).  A token is drawn exactly from pi_mix by walking the gates with
 * caller-supplied uniforms and sampling only the head where the walk stops
 * (same summary, section 3, "exact sampling"; abstract).  The layers above that
 * exit are deferred and run later, as a causal chunk concatenated with the
 * following tokens that reach those depths, so that every layer's KV cache is
 * complete (section 2, part "Inferenz: Piggybacking"; abstract).
 *
 * Conventions for every call:
 *   - Host pointers belong to the caller and are read or written only during
 *     the call.  Device memory belongs to the model (inside the caller's arena
 *     when one is given) and is released by nv_free.
 *   - Every call is synchronous with respect to the host: results are in host
 *     memory when it returns.  Work is issued on the stream given to nv_load.
 *   - One model handle must not be used from two threads at once.
 *   - Errors return a negative nv_status; nv_last_error gives the text.  After
 *     NV_EDEVICE (any HIP runtime error) the handle can only be freed.
 */
#ifndef NVIUM_H
#define NVIUM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nv_model nv_model;

typedef enum nv_status {
    NV_OK = 0,
    NV_EINVAL = -1,     /* bad argument: NULL pointer, uniform outside [0,1) or NaN,
                           token id >= vocab, sequence index out of range */
    NV_ESTATE = -2,     /* call not valid in the current state (e.g. step before prefill,
                           prefilled sequences not numbered 0..n-1) */
    NV_ECAPACITY = -3,  /* a sequence would exceed max_ctx positions, or an arena too small */
    NV_EIO = -4,        /* weights file missing, truncated or inconsistent */
    NV_EDEVICE = -5     /* HIP runtime error; the handle is no longer usable */
} nv_status;

/* Model shape, as read from the weights file. */
typedef struct nv_config {
    int32_t n_layers, d_model, n_heads, head_dim, ffn, vocab, n_exits;
    int32_t wdtype;                 /* 0: fp32 matrices and KV; 1: bf16 matrices and KV */
    float norm_eps, rope_base;
    int32_t exit_layer[4];          /* 1-based layer after which exit k sits */
    float gate_bias[4];             /* b_k; the last is +inf (w = 1) */
    int32_t head_form;              /* 0: own RMSNorm + LM head per exit; 1: one final RMSNorm + LM
                                       head, exits 1..3 reach it through the adapter MLP
                                       h + U_k silu(D_k h) */
    int32_t adapter_dim;            /* adapter bottleneck r (head_form 1) */
    int32_t router_form;            /* 0: w_k = sigmoid(g_k . h + b_k); 1: router MLP,
                                       w_k = sigmoid(w2_k . silu(W1_k h + b1_k) + b_k) */
    int32_t router_dim;             /* router hidden width (router_form 1) */
} nv_config;

/* Device bytes nv_load needs for this weights file at this capacity
 * (weights + KV caches + hidden states + workspaces), or 0 if the file
 * cannot be read.  Lets a caller allocate the arena (e.g. a torch tensor). */
size_t nv_mem_required(const char *weights_path, int32_t max_batch, int32_t max_ctx);

/* Load a weights file (layout in synth/weights.py of this repository) and
 * allocate state for up to max_batch sequences of up to max_ctx positions each.
 *   device_arena: device memory of at least nv_mem_required() bytes owned by
 *                 the caller and kept alive until nv_free, or NULL to let the
 *                 library allocate (hipMalloc).
 *   hip_stream:   a hipStream_t to issue all work on, or NULL for the null stream.
 * Environment, read here (and, for the sizes, by nv_mem_required; set it the
 * same way for both calls):
 *   NVIUM_MFMA_MIN_ROWS  rows from which products use the matrix cores (default 9;
 *                        0: never), for tests of the vector-ALU paths;
 *   NVIUM_SK_MIN_ROWS, NVIUM_SK_MAX_ROWS  row groups that take the split-K
 *                        matrix-core product when K is a multiple of 512 (default 5
 *                        and 64; 0: never);
 *   NVIUM_SK_NTB=a,b     16-column tiles per split-K block with / without RMSNorm
 *                        (1 or 2; default 2,1);
 *   NVIUM_SCHED_AGE      nv_generate's greedy aging weight (default 16);
 *   NVIUM_SEGMENT=1      one-row decode segments in the persistent segment kernel;
 *   NVIUM_LOSS_ROWS      rows per head pass of nv_mixture_loss (default: as many as
 *                        a 256 MiB logits workspace holds, at least 256).
 * Errors: NV_EINVAL (NULL path/out, sizes < 1), NV_EIO (file), NV_ECAPACITY
 * (arena too small), NV_EDEVICE. */
nv_status nv_load(const char *weights_path, int32_t max_batch, int32_t max_ctx,
                  void *device_arena, size_t arena_bytes, void *hip_stream,
                  nv_model **out);

void nv_free(nv_model *m);

/* Text of the last error on this handle ("" if none).  Valid until the next call. */
const char *nv_last_error(const nv_model *m);

nv_status nv_get_config(const nv_model *m, nv_config *out);

/* Start (or restart) sequence `seq` with prompt tokens[0..n-1], n >= 1.
 * Positions 0..n-2 run through every layer (building their KV); tokens[n-1]
 * becomes the pending input that the next nv_step consumes at position n-1.
 * Source: a forward pass both builds every layer's K/V and predicts the next token
 * (gist.science summary, section 1); the prompt has no token to exit, so it runs at
 * full depth and leaves complete caches (section 2, part "Inferenz: Piggybacking").
 * Restarting drops the sequence's KV, deferred states and frontiers.
 * Errors: NV_EINVAL (seq out of range, NULL tokens, n < 1, token >= vocab),
 * NV_ECAPACITY (n > max_ctx), NV_EDEVICE. */
nv_status nv_prefill(nv_model *m, int32_t seq, const int32_t *tokens, int32_t n);

/* One decode step for every prefilled sequence 0..n_seq-1 in lock-step.
 * Source: the mixture output and its stick-breaking weights (gist.science summary,
 * section 2 "Methodik", part "Architektur", equations for p_k and pi_mix); drawing exactly
 * from the mixture by walking the gates and sampling only the stopping exit (section 3,
 * "Exakte Sampling-Mischung"; abstract); the layers a token skips run later with the next
 * token that reaches them, as one causal chunk (section 2, part "Inferenz: Piggybacking").
 *   uniforms   [n_seq][4] float32 in [0,1): u[0..2] walk gates 1..3 (stop at gate
 *              k iff u[k-1] < w_k), u[3] draws the token by inverse CDF of the
 *              stopping exit's softmax in token-id order (smallest id i with
 *              u[3] < F(i)).
 *   tokens_out [n_seq] sampled next token; it becomes the pending input.
 *   exits_out  [n_seq] exit the token came from, 1..4.
 * Layers above the exit are deferred; they run when a later token of the same
 * sequence reaches them, or at nv_flush.
 * Errors: NV_EINVAL (NULL pointers, bad uniforms), NV_ESTATE (no prefilled
 * sequence, or prefilled indices not contiguous from 0), NV_ECAPACITY (a
 * sequence has no free position), NV_EDEVICE. */
nv_status nv_step(nv_model *m, const float *uniforms, int32_t *tokens_out, int32_t *exits_out);

/* nv_step with the next inputs given by the caller (teacher forcing): sampling
 * and deferral happen exactly as in nv_step and tokens_out/exits_out report the
 * draw, but next_inputs[i] (< vocab) becomes sequence i's pending input instead
 * of the sampled token.  Used to score a given continuation. */
nv_status nv_step_forced(nv_model *m, const float *uniforms, const int32_t *next_inputs,
                         int32_t *tokens_out, int32_t *exits_out);

/* Scheduling policies of nv_generate. */
#define NV_SCHED_LOCKSTEP 0  /* rounds: every listed sequence's token runs segment 1, then the
                                ones still going run segment 2, ...; one token per sequence per
                                round (what repeated nv_step calls do) */
#define NV_SCHED_GREEDY 1    /* each tick runs the segment with the highest
                                (waiting sequences + 16 x the longest wait there, in ticks;
                                the environment variable NVIUM_SCHED_AGE read by nv_load
                                sets the weight); ties go to the deeper segment */

/* Batched decoding where sequences advance through the segments independently (the
 * gptget.net summary's limitations section names the batched-inference strategy as
 * needing change, since tokens of one batch are sampled at different exits).  Sequences seqs[0..n_seq-1]
 * (distinct, prefilled, in any order and any subset of the handle's slots) each
 * generate n_tokens tokens.  A tick runs one segment for every listed sequence whose
 * current token waits there, each with its deferred rows as one causal chunk, then
 * that segment's gate; sequences that stop get their exit head and draw, and their
 * next token enters segment 1 at a later tick.  `policy` chooses the tick's segment.
 *   uniforms   [n_seq][n_tokens][4] float32 in [0,1): token t of sequence seqs[i] uses
 *              uniforms[i][t] exactly as nv_step uses its row (gates walked with
 *              u[0..2], inverse CDF with u[3]).
 *   tokens_out [n_seq][n_tokens], exits_out [n_seq][n_tokens] (1..4).
 * Each sequence's tokens and exits are those of n_tokens nv_step calls with the same
 * uniforms (the kernels may group rows differently, so floating-point results can
 * differ in the last bits).  The last token becomes the pending input.  nv_debug_gates
 * reports NaN afterwards for the listed sequences.
 * Errors: NV_EINVAL (NULL pointers, n_seq outside 1..max_batch, index out of range or
 * repeated, n_tokens < 0, bad uniform, unknown policy), NV_ESTATE (a listed sequence is
 * not prefilled), NV_ECAPACITY (a sequence would pass max_ctx), NV_EDEVICE. */
nv_status nv_generate(nv_model *m, const int32_t *seqs, int32_t n_seq, int32_t n_tokens,
                      const float *uniforms, int32_t policy, int32_t *tokens_out, int32_t *exits_out);

/* The mixture objective on a token sequence, forward only (gist.science technical
 * summary, section 2 "Methodik", part "Training": L_total = L_mix + beta * L_compute;
 * L_mix is the cross-entropy of pi_mix, L_compute the expected exit depth).
 * Sequence `seq` is prefilled with tokens[0..n-1] exactly as nv_prefill does
 * (afterwards it can decode), and after each segment every position t = 0..n-2
 * evaluates that exit's router w_k and log pi_k(tokens[t+1]).
 *   out      [3] host float64: L_mix = mean_t -log sum_k p_k pi_k(tokens[t+1]),
 *            L_compute = mean_t sum_k p_k l_k / L (l_k = exit k's last layer),
 *            L_total = L_mix + beta * L_compute.
 *   per_pos  NULL, or host float64 [n-1][10]: w_1..w_4 (w_4 = 1), log pi_1..4 of
 *            the target, -log pi_mix of the target, expected depth.
 * Errors: NV_EINVAL (seq out of range, NULL tokens or out, n < 2, token >= vocab,
 * beta not finite), NV_ECAPACITY (n > max_ctx), NV_EDEVICE.  On error the
 * sequence must be prefilled again before it decodes. */
nv_status nv_mixture_loss(nv_model *m, int32_t seq, const int32_t *tokens, int32_t n, double beta,
                          double *out, double *per_pos);

/* Run every deferred segment of sequence `seq` (-1: all prefilled sequences)
 * over all consumed positions, with no gates and no heads.  Afterwards every
 * layer's KV is complete for every consumed position.  A second flush is a
 * no-op.  Source: the deferred rows are the ones piggybacking would fill with the next
 * deeper token; running them at once gives the complete, exact cache the method promises
 * (gist.science summary, section 2, part "Inferenz: Piggybacking", "Ergebnis"; section 3,
 * "Vollständige KV-Wiederherstellung").
 * Errors: NV_EINVAL (seq out of range), NV_EDEVICE. */
nv_status nv_flush(nv_model *m, int32_t seq);

/* ---- one exit's draw on caller buffers --------------------------------------- */

/* Bytes of device workspace nv_exit_draw needs for a vocabulary of `vocab` ids (0 if
 * vocab is not a positive multiple of 8 up to 65536). */
size_t nv_exit_draw_workspace(int32_t vocab);

/* One exit's head and draw for one hidden row, the step nv_step takes for a sequence that
 * stops at an exit (gist.science technical summary of the pages, section 2, part
 * "Architektur": every exit has its own head; section 3: the exit's distribution is sampled
 * exactly).  logits = W_head . RMSNorm(h) (RMSNorm weight norm_w, epsilon eps), then token =
 * the smallest id i with u < F(i), F the running sum of softmax(logits) in id order
 * (float32 exponentials, float64 sums and comparison); if rounding leaves u at or past the
 * total, the last id with nonzero mass.
 *   h         device float32 [d]: the residual stream after the exit's last layer
 *   norm_w    device float32 [d]
 *   head_w    device [vocab][d]: bf16 bit patterns if wdtype is 1, float32 if 0
 *   u         the uniform, in [0, 1)
 *   logits    device float32 [vocab], written
 *   token     device int32 [1], written
 *   workspace device memory of at least nv_exit_draw_workspace(vocab) bytes (scratch: the
 *             head product's per-block softmax partials), owned by the caller
 *   hip_stream the hipStream_t to enqueue on (NULL: the null stream)
 * Shapes: d a multiple of 8 (bf16) or 4 (float32), d <= 4096 (bf16) or 2048 (float32);
 * vocab a multiple of 8, at most 65536.  The call only enqueues work (it does not wait, and
 * it allocates nothing); the outputs are valid once the stream has run it.  Errors:
 * NV_EINVAL (NULL pointer, shape, u outside [0,1) or NaN, eps <= 0), NV_ECAPACITY
 * (workspace too small), NV_EDEVICE (a launch failed). */
nv_status nv_exit_draw(const float *h, const float *norm_w, const void *head_w, int32_t wdtype, int32_t d,
                       int32_t vocab, float eps, float u, float *logits, int32_t *token, void *workspace,
                       size_t workspace_bytes, void *hip_stream);

/* nv_exit_draw for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments
 * without the workspace.  Its scratch is a 64 KiB array inside the library, one per GPU,
 * held until the process ends (vocab up to 65536, as for nv_exit_draw).  It allocates
 * nothing and only enqueues work.  Calls that overlap on one GPU (on different streams or
 * threads) share that array and race; serialize them.  Errors: as nv_exit_draw, and
 * NV_EDEVICE if the array's device address cannot be obtained. */
nv_status nv_exit_draw_static(const float *h, const float *norm_w, const void *head_w, int32_t wdtype,
                              int32_t d, int32_t vocab, float eps, float u, float *logits, int32_t *token,
                              void *hip_stream);

/* ---- inspection (not on the timed path) ------------------------------------ */

/* Positions consumed so far (prompt prefix + decode steps) and the four
 * frontiers: every position < frontier[s] has completed segment s+1. */
nv_status nv_debug_frontiers(nv_model *m, int32_t seq, int32_t *n_consumed, int32_t frontier[4]);

/* Logits (float32, [vocab]) of the exit that produced the last step's token. */
nv_status nv_debug_logits(nv_model *m, int32_t seq, float *out);

/* Router outputs w_1..w_4 of the last step (float64; NaN for gates not reached,
 * w_4 = 1 when exit 4 was reached). */
nv_status nv_debug_gates(nv_model *m, int32_t seq, double *out);

/* K and V of layer `layer` (0-based) for positions pos0..pos0+n-1, as float32
 * [n][n_heads][head_dim] each (K after RoPE). */
nv_status nv_debug_kv(nv_model *m, int32_t seq, int32_t layer, int32_t pos0, int32_t n,
                      float *k_out, float *v_out);

/* Hidden states (float32 [n][d_model]) of positions pos0..pos0+n-1: the output
 * of the last segment each position completed. */
nv_status nv_debug_hidden(nv_model *m, int32_t seq, int32_t pos0, int32_t n, float *out);

/* ---- kernel timing (measurement; adds events between launches) ------------------ */

/* Kernel classes timed by nv_timing_*: */
#define NV_TIME_BLOCK_GEMM 0   /* the transformer-block skinny GEMMs (QKV, O, gate/up, down) */
#define NV_TIME_ATTENTION 1    /* RoPE + KV append, chunked attention, split combine */
#define NV_TIME_EXIT_HEAD 2    /* exit RMSNorm + LM-head GEMV */
#define NV_TIME_OTHER 3        /* embedding gather, router gates, sampling */
#define NV_TIME_CLASSES 4

/* on == 1: from now on bracket every kernel launch with HIP events on the model's
 * stream (hipExtLaunchKernelGGL's start/stop events: launch to completion, as a
 * profiler's kernel trace counts it) and accumulate per-class device time, launch counts
 * and algorithmic bytes (bytes each launch must move at minimum: weights read once,
 * activations in/out, keys/values read).  on == 2: the same, and the decode products and
 * attention kernels also record per-block device clock stamps (first block start to last
 * block end), folded by one small kernel after each launch, which perturbs the event
 * durations; take events and spans from separate passes.  on == 0: stop.  Either way the
 * counters restart at zero.  Other values: NV_EINVAL. */
nv_status nv_timing_enable(nv_model *m, int32_t on);

/* Totals since nv_timing_enable: ms[k] device milliseconds, bytes[k] algorithmic
 * bytes and launches[k] launches of class k, for k < NV_TIME_CLASSES. */
nv_status nv_timing_read(nv_model *m, double *ms, double *bytes, int64_t *launches);

/* The same totals per kernel symbol, as text: one line per kernel,
 * "class<TAB>launches<TAB>device ms<TAB>algorithmic bytes<TAB>span ms<TAB>symbol\n"
 * (device ms from the events; span ms the summed stamp spans, -1 for kernels without
 * stamps; symbols as profilers print them).  NV_ECAPACITY if `cap` bytes cannot hold it. */
nv_status nv_timing_kernels(nv_model *m, char *out, size_t cap);

#ifdef __cplusplus
}
#endif

#endif /* NVIUM_H */
