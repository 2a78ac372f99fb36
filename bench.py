#!/usr/bin/env python3
"""Decode throughput of the N-vium mixture-of-exits step on one MI355X.

Workload (default "A"): the 1.5B N-vium (48 layers, d 1536, 12 x 128 heads, SwiGLU
4096, vocab 32000, bf16 weights and KV), batch 1, a 512-token uniform-random
prompt, then `--steps` decode steps (512 = the full workload) with seeded uniforms;
random-init weights (seed 0), exit mass ~[.4,.25,.2,.15].  A step is one nv_step:
embed, every reached segment with its deferred chunk, the gates walked, one exit
head and the draw.  Inputs are resident in device memory before timing starts.

Printed: one JSON line.  `value` = generated tokens/s over the timed steps.
Beside it: the same kernels with every intermediate gate closed (all tokens exit at
4, standard decode), per-kernel device time from a second, identical pass (device
wall-clock stamps per block for the decode GEMMs and attention, HIP events for the
rest; roofline of the dominant block GEMM against 8 TB/s), and the CPU oracle timed
on a bounded sample of the same decode.

Workload "C" (--workload C) decodes 16 sequences with nv_generate's greedy segment
scheduling; lock-step scheduling, nv_step and exit-4-forced decoding are timed beside it.
Workload "L" (--workload L) times the mixture objective instead: a step is one
nv_mixture_loss over a 2048-token sequence on the same 1.5B model (full-depth causal
pass, every exit's router and head at every position); `value` = scored positions/s,
roofline of the dominant block GEMM against the bf16 matrix-core peak.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SPANS = False          # --spans: also a pass with per-block device clock stamps
EVENTS_PASSES = 0      # --events-passes: events passes of a decode (0: enough for 100 steps)
TIMING_NOTE = ("avg_launch_us: hipExtLaunchKernelGGL start/stop events on each launch on the model's stream, "
               "in untimed passes identical to the timed one (decode: as many as make 100 steps or more; launch "
               "to completion, as a rocprofv3 kernel trace counts it); avg_span_us (with --spans): first block start to last block end from device "
               "clock stamps, in a further untimed pass of its own")
# exit masses the workloads state (the gate biases are calibrated to give them)
STATED_MASS = {"A": (0.4, 0.25, 0.2, 0.15), "C": (0.4, 0.25, 0.2, 0.15), "D": (0.6, 0.2, 0.1, 0.1),
               "E": (0.4, 0.25, 0.2, 0.15)}
MFMA_BF16_TFLOPS = 2500.0
KERNEL_SOURCES = ("mixture_exits_transformer_amd/csrc/nv_kernels.hip",
                  "mixture_exits_transformer_amd/csrc/nv_segment.hip",
                  "mixture_exits_transformer_amd/csrc/nv_device.h",
                  "mixture_exits_transformer_amd/csrc/nv_internal.h")


def kernel_source_sha1():
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled(kname, field):
    """(value, source) of `field` for kernel symbol `kname` from the machine-readable block
    of a committed summary under profiles/ (rocprofv3 counters or kernel trace), or None
    when none covers this kernel or the kernel sources changed since it was taken."""
    import glob
    sha = kernel_source_sha1()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        kv = {}
        with open(path) as f:
            for line in f:
                k, sep, v = line.partition(": ")
                if sep and k in ("kernel", "kernel_source_sha1", field):
                    kv[k] = v.strip()
        if kv.get("kernel") == kname and kv.get("kernel_source_sha1") == sha and field in kv:
            return float(kv[field]), os.path.relpath(path, ROOT)
    return None


def counted_traffic(kname):
    """HBM bytes per launch of `kname` from the committed FETCH_SIZE/WRITE_SIZE summaries."""
    r = profiled(kname, "traffic_bytes_per_launch")
    return (int(r[0]), r[1]) if r else None


def profile_fields(kname, bytes_per_launch, peak):
    """The committed rocprofv3 kernel-trace average of the dominant symbol, beside the
    live events figure (the events average moves by several per cent between runs of
    the same code; the profiler's kernel durations much less)."""
    r = profiled(kname, "rocprof_avg_us")
    if not r:
        return {"rocprof_avg_us": None, "rocprof_frac": None, "rocprof_source": None}
    return {"rocprof_avg_us": r[0], "rocprof_frac": round(bytes_per_launch / (r[0] * 1e-6) / 1e9 / peak, 4),
            "rocprof_source": r[1]}


def calibration_copy(out):
    """One 1 GiB device-to-device copy after the timed work: the reference that scales the
    HBM byte counters (FETCH_SIZE, WRITE_SIZE) of a profiled run."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    out["calibration_copy_bytes"] = 1 << 30
    # the same copy timed (three more, events on torch's stream): HBM read + write rate of a
    # plain device copy, a practical ceiling beside the 8 TB/s data-sheet peak
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(3):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    out["calibration_copy_GBps"] = round(3 * 2 * (1 << 30) / (t0.elapsed_time(t1) * 1e-3) / 1e9, 1)


class paused_gc:
    """Timed regions run with Python's cyclic garbage collector paused (after a collection):
    one full collection in an interpreter that holds torch takes about 40 ms, and it landed
    inside one of the 512 timed decode steps (8 % of the run)."""

    def __enter__(self):
        gc.collect()
        gc.disable()

    def __exit__(self, *exc):
        gc.enable()


CALIBRATION_SAMPLE = os.path.join(ROOT, "tests", "golden", "gate_bias_1p5b.json")


def expected_window_mass(wl, p0, n):
    """Mean stick-breaking exit probabilities over decode positions p0 .. p0+n-1, from the
    stored gate-calibration sample: the gate logits g_k . h at those positions, taken on the
    workload's prompt followed by uniform stand-in tokens (the run draws its own tokens, so
    its hidden states differ), with the workload's biases.  None when the sample does not
    cover the window.  The stated mass holds on average over the whole calibrated range; a
    short window sees the drift of the router's linear term with the position."""
    import numpy as np
    try:
        with open(CALIBRATION_SAMPLE) as f:
            cal = json.load(f).get(wl.name)
    except OSError:
        return None
    if not cal:
        return None
    lo, hi = cal["positions"]
    if p0 < lo or p0 + n - 1 > hi:
        return None
    z = np.asarray(cal["z"], dtype=np.float64)[p0 - lo:p0 - lo + n]
    w = 1.0 / (1.0 + np.exp(-(z + np.asarray(wl.model.gate_bias, dtype=np.float64))))
    p = np.empty((n, 4))
    rest = np.ones(n)
    for k in range(3):
        p[:, k] = rest * w[:, k]
        rest = rest * (1.0 - w[:, k])
    p[:, 3] = rest
    return {"value": [round(float(x), 4) for x in p.mean(axis=0)],
            "positions": [p0, p0 + n - 1],
            "source": "gate-calibration sample (tests/golden/gate_bias_1p5b.json): oracle hidden states on "
                      "the workload's prompt plus uniform stand-in tokens, not this run's draws"}


def run_decode(lib, h, prompt, U, steps, warmup):
    """Warm up, restart the sequence, then time `steps` decode steps: once through
    nv_generate (the library's decode loop: one call, draws read back through its ring of
    pinned buffers) and once as a loop of nv_step calls from Python (one synchronous call
    per token).  Both run the same computation and give the same tokens and exits.
    Returns (generate seconds, nv_step-loop seconds, exits)."""
    import torch
    lib.nv_prefill(h, 0, prompt)
    for t in range(warmup):
        lib.nv_step(h, U[t:t + 1])
    lib.nv_prefill(h, 0, prompt)
    with paused_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, ex = lib.nv_generate(h, [0], U[None, :steps, :], lib.SCHED_GREEDY)
        torch.cuda.synchronize()
        dt_g = time.perf_counter() - t0
    exits = [int(e) for e in ex.ravel()]
    lib.nv_prefill(h, 0, prompt)
    exits_s = []
    with paused_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            _, e = lib.nv_step(h, U[t:t + 1])
            exits_s.append(int(e[0]))
        torch.cuda.synchronize()
        dt_s = time.perf_counter() - t0
    assert exits_s == exits, "nv_generate and the nv_step loop took different exits"
    return dt_g, dt_s, exits


def two_pass_timing(lib, h, setup, work, passes=1):
    """Per-launch device timing of `work` (after `setup`) in `passes` untimed passes with
    HIP events only (summed: the events average of one short pass moves by a few per cent
    from one pass to the next); with --spans, one more pass with per-block device clock
    stamps as well (the small kernel that folds each launch's stamps perturbs the events,
    so the spans come from a pass of their own).  Returns the events passes' class totals
    and per-kernel rows, each with the stamp pass's summed span (ms) of the same symbol
    scaled to the same launch count, or None."""
    tim, acc = None, {}
    for _ in range(passes):
        setup()
        lib.nv_timing_enable(h, 1)
        work()
        t1 = lib.nv_timing_read(h)
        tim = t1 if tim is None else {c: tuple(a + b for a, b in zip(tim[c], t1[c])) for c in tim}
        for k in lib.nv_timing_kernels(h):
            key = (k[0], k[4])
            n, ms, by = acc.get(key, (0, 0.0, 0.0))
            acc[key] = (n + k[1], ms + k[2], by + k[3])
        lib.nv_timing_enable(h, 0)
    ker = [(c, n, ms, by, name) for (c, name), (n, ms, by) in acc.items()]
    if not SPANS:
        return tim, [k + (None,) for k in ker]
    setup()
    lib.nv_timing_enable(h, 2)
    work()
    spans = {(k[0], k[4]): (k[1], k[5]) for k in lib.nv_timing_kernels(h)}
    lib.nv_timing_enable(h, 0)
    rows = []
    for k in ker:
        n2, span = spans.get((k[0], k[4]), (0, None))
        rows.append(k + (span * k[1] / n2 if span is not None and n2 else None,))
    return tim, rows


def events_passes(steps):
    """Events passes for a decode of `steps` steps: at least about 100 steps in all
    (--events-passes sets the count instead)."""
    if EVENTS_PASSES:
        return EVENTS_PASSES
    return max(1, -(-100 // max(steps, 1)))


def timing_pass(lib, h, prompt, U, steps):
    """The same decode again with per-launch device timing (events, then stamps)."""
    def work():
        for t in range(steps):
            lib.nv_step(h, U[t:t + 1])
    return two_pass_timing(lib, h, lambda: lib.nv_prefill(h, 0, prompt), work, events_passes(steps))


def cpu_baseline(wl, path, prompt, U, budget_s):
    """The oracle (float64 NumPy) on the host: decode steps after an untimed prefill."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import model as om
    M = om.OracleModel(path)
    st = om.new_state(M, len(prompt) + len(U))
    om.prefill(M, st, prompt[:-1])
    y = int(prompt[-1])
    n = 0
    t0 = time.perf_counter()
    while n < len(U):
        o = om.decode_step(M, st, y, U[n], all_heads=False)
        y = o.token
        n += 1
        if time.perf_counter() - t0 > budget_s and n >= 2:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "precision": "float64 (the oracle as written: sequential, full depth, all exits' heads skipped but "
                         "the stopping one; slower than a float32 CPU implementation would be)",
            "sample": f"{n} decode steps of workload {wl.name} (positions {len(prompt) - 1}.."
                      f"{len(prompt) - 2 + n}) after an untimed {len(prompt) - 1}-token prefill, "
                      f"{dt:.1f} s"}


def loss_cpu_baseline(path, tokens, budget_tokens):
    """The oracle's mixture_loss on the first `budget_tokens` tokens of the sequence."""
    from threadpoolctl import threadpool_info

    from oracle import model as om
    M = om.OracleModel(path)
    t0 = time.perf_counter()
    om.mixture_loss(M, tokens[:budget_tokens], 0.5)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": (budget_tokens - 1) / dt, "unit": "scored tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"mixture_loss over the first {budget_tokens} tokens ({budget_tokens - 1} positions, every "
                      f"exit's router and head) of the same sequence, {dt:.1f} s"}


def bench_loss(args, wl):
    """Mixture objective: a step is one nv_mixture_loss over the whole sequence (the
    full-depth causal pass over n-1 positions, each exit's router and head at every
    position, log-softmax at the target, the mixture and the means)."""
    import torch

    from mixture_exits_transformer_amd import lib
    from synth import cached_weights, prompts
    tokens = prompts(wl)[0]
    n = len(tokens)
    steps = args.steps if args.steps is not None else 10
    warmup = args.warmup if args.warmup is not None else 2
    path = cached_weights(wl.model)
    h = lib.nv_load(path, 1, n)
    for _ in range(warmup):
        lib.nv_mixture_loss(h, 0, tokens, 0.5)
    with paused_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            L = lib.nv_mixture_loss(h, 0, tokens, 0.5)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
    tim, ker = two_pass_timing(lib, h, lambda: None, lambda: lib.nv_mixture_loss(h, 0, tokens, 0.5))
    lib.nv_free(h)
    m = wl.model
    d, F, Lr, V, r = m.d_model, m.ffn, m.n_layers, m.vocab, n - 1
    # dominant kernel: the block-GEMM product symbol with the most device time.  The long-chunk
    # GEMM is instantiated per epilogue (template argument EPI: 1 residual = O and down,
    # 2 SwiGLU = gate/up, 3 QKV), so each symbol's algorithmic FLOPs follow from it.
    per_epi = {1: 2.0 * r * Lr * (d * d + F * d), 2: 2.0 * r * Lr * 2 * F * d, 3: 2.0 * r * Lr * 3 * d * d}
    gemms = sorted([k for k in ker if k[0] == "block_gemm" and "k_gemm_bf16<" in k[4]], key=lambda k: -k[2])
    _, nl, ms, by, kname, span = gemms[0]
    epi = int(kname.split("k_gemm_bf16<")[1].split(">")[0].split(",")[2]) if "k_gemm_bf16<" in kname else None
    assert epi in per_epi, f"dominant block GEMM {kname} is not the long-chunk kernel"
    flops = per_epi[epi]
    # algorithmic bytes: weights once, the bf16 rows, the outputs (fp32, read and written
    # for a residual; SwiGLU written as the down product's bf16 rows; q in fp32 and K, V in
    # bf16 for QKV)
    per_epi_bytes = {1: Lr * (2 * d * d + 2 * d * F + r * d * 2 + r * F * 2 + 2 * r * d * 8),
                     2: Lr * (2 * F * d * 2 + r * d * 2 + r * F * 2),
                     3: Lr * (3 * d * d * 2 + r * d * 2 + r * d * 4 + r * 2 * d * 2)}
    bytes_per_launch = per_epi_bytes[epi] / nl
    achieved = flops / (ms * 1e-3) / 1e12
    all_flops = 2.0 * r * Lr * (4 * d * d + 3 * d * F)
    counted = counted_traffic(kname)
    top = sorted(ker, key=lambda k: -k[2])[:8]
    total_flops = all_flops + 2.0 * r * 4 * V * d + 2.0 * Lr * m.n_heads * m.head_dim * r * (r + 1)
    out = {
        "metric": "mixture-objective scored tokens/s (forward L_mix + beta L_compute), 1.5B bf16",
        "value": round(steps * r / dt, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(dt / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m.wdtype,
        "data": "synthetic: uniform-random token ids (seed 1), random-init N(0,0.02) weights",
        "config": {"workload": f"{wl.name}: {wl.note}", "batch": 1, "tokens": n, "positions": r},
        "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 1), "peak": MFMA_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_TFLOPS, 4),
                     "traffic": counted[0] if counted else None,
                     "traffic_source": counted[1] if counted else None,
                     "launches": nl, "avg_launch_us": round(ms / max(nl, 1) * 1e3, 3),
                     "flops_per_launch": round(flops / max(nl, 1)), "bytes_per_launch": round(bytes_per_launch)},
        "block_gemm_all_TFLOPs": round(all_flops / (tim["block_gemm"][0] * 1e-3) / 1e12, 1),
        "pass_TFLOPs": round(total_flops / (dt / steps) / 1e12, 1),
        "L": [round(x, 6) for x in L],
        "top_kernels": [{"kernel": k[4], "class": k[0], "launches": k[1],
                         "avg_us": round(k[2] / max(k[1], 1) * 1e3, 3)} for k in top],
        "kernel_classes_ms_per_step": {k: round(v[0], 4) for k, v in tim.items()},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = loss_cpu_baseline(path, tokens, args.cpu_loss_tokens)
    if args.calibrate_copy:
        calibration_copy(out)
    print(json.dumps(out), flush=True)


def bench_batch(args, wl):
    """Batched decode (workload C: 16 independent sequences): a step is one token for
    every sequence.  `value` uses nv_generate with the greedy tick policy (sequences
    advance through the segments independently); beside it the lock-step policy, a
    loop of nv_step calls, and exit-4-forced decoding."""
    import numpy as np
    import torch
    from dataclasses import replace

    from mixture_exits_transformer_amd import lib
    from synth import cached_weights, prompts, uniforms
    from synth.configs import BIAS_ALL_LAST
    ps = prompts(wl)
    B = wl.batch
    steps = args.steps if args.steps is not None else wl.decode_steps
    warmup = args.warmup if args.warmup is not None else 8
    U = np.ascontiguousarray(uniforms(wl, steps=steps + warmup).transpose(1, 0, 2))   # [B][steps+warmup][4]
    Uw, Ut = np.ascontiguousarray(U[:, steps:]), np.ascontiguousarray(U[:, :steps])
    max_ctx = max(len(p) for p in ps) + max(steps, warmup)
    slots = list(range(B))
    path = cached_weights(wl.model)

    def prefill_all(h):
        for i, p in enumerate(ps):
            lib.nv_prefill(h, i, p)

    def timed_generate(h, policy):
        prefill_all(h)
        if warmup:
            lib.nv_generate(h, slots, Uw, policy)
        prefill_all(h)
        with paused_gc():
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            toks, exs = lib.nv_generate(h, slots, Ut, policy)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
        return dt, exs

    h = lib.nv_load(path, B, max_ctx)
    dt_g, ex_g = timed_generate(h, lib.SCHED_GREEDY)
    dt_l, ex_l = timed_generate(h, lib.SCHED_LOCKSTEP)
    prefill_all(h)
    with paused_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            lib.nv_step(h, Ut[:, t, :])
        torch.cuda.synchronize()
        dt_s = time.perf_counter() - t0
    tim, ker = two_pass_timing(lib, h, lambda: prefill_all(h), lambda: lib.nv_generate(h, slots, Ut, lib.SCHED_GREEDY))
    lib.nv_free(h)
    base = None
    if not args.no_baseline:
        h4 = lib.nv_load(cached_weights(replace(wl.model, gate_bias=BIAS_ALL_LAST)), B, max_ctx)
        dt4, ex4 = timed_generate(h4, lib.SCHED_LOCKSTEP)
        lib.nv_free(h4)
        assert set(ex4.ravel().tolist()) == {4}
        base = B * steps / dt4
    tok_s = B * steps / dt_g
    gemms = sorted([k for k in ker if k[0] == "block_gemm"], key=lambda k: -k[2])
    _, nl, ms, by, kname, span = gemms[0]
    achieved = by / (ms * 1e-3) / 1e9
    counted = counted_traffic(kname)
    top = sorted(ker, key=lambda k: -k[2])[:8]
    out = {
        "metric": "generated tokens/s over 16 sequences, 1.5B, greedy segment scheduling vs lock-step; "
                  "achieved HBM GB/s",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(dt_g / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.model.wdtype,
        "data": "synthetic: uniform-random token ids, seeded uniforms, random-init N(0,0.02) weights",
        "config": {"workload": f"{wl.name}: {wl.note}", "batch": B, "prompts": [len(p) for p in ps],
                   "decode_steps": steps},
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counted[0] if counted else None,
                     "traffic_source": counted[1] if counted else None,
                     "launches": nl, "avg_launch_us": round(ms / max(nl, 1) * 1e3, 3),
                     "avg_span_us": round(span / max(nl, 1) * 1e3, 3) if span else None,
                     "bytes_per_launch": round(by / max(nl, 1)), "timing": TIMING_NOTE},
        "lockstep_policy_tokens_per_s": round(B * steps / dt_l, 2),
        "nv_step_loop_tokens_per_s": round(B * steps / dt_s, 2),
        "greedy_vs_lockstep": round(dt_l / dt_g - 1.0, 4),
        "exit4_forced_tokens_per_s": round(base, 2) if base else None,
        "speedup_vs_exit4": round(tok_s / base - 1.0, 4) if base else None,
        "exit_histogram": [int(x) for x in np.bincount(ex_g.ravel(), minlength=5)[1:]],
        "lockstep_exit_histogram": [int(x) for x in np.bincount(ex_l.ravel(), minlength=5)[1:]],
        "top_kernels": [{"kernel": k[4], "class": k[0], "launches": k[1],
                         "avg_us": round(k[2] / max(k[1], 1) * 1e3, 3),
                         "GBps": round(k[3] / (k[2] * 1e-3) / 1e9, 1) if k[2] > 0 else None} for k in top],
        "kernel_classes_ms_per_step": {k: round(v[0] / steps, 4) for k, v in tim.items()},
    }
    if not args.no_cpu:
        j = int(np.argmin([len(p) for p in ps]))
        cb = cpu_baseline(wl, path, ps[j], Ut[j], args.cpu_budget)
        cb["sample"] = f"sequence {j} alone: " + cb["sample"]
        out["cpu_baseline"] = cb
    if args.calibrate_copy:
        calibration_copy(out)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="decode steps (default: the workload's, 512 for A); loss passes (10)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 16; loss passes 2)")
    ap.add_argument("--workload", default="A",
                    help="A, B, D, E (decode, batch 1), C (16 sequences) or L (mixture objective)")
    ap.add_argument("--cpu-loss-tokens", type=int, default=40, help="oracle sample for workload L")
    ap.add_argument("--no-baseline", action="store_true", help="skip the exit-4-forced run")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--spans", action="store_true",
                    help="also time first block start to last block end (device stamps) in a pass of its own")
    ap.add_argument("--events-passes", type=int, default=0,
                    help="events passes of a decode (default: enough for 100 steps)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    global SPANS, EVENTS_PASSES
    SPANS = args.spans
    EVENTS_PASSES = max(0, args.events_passes)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the decode path "
              f"runs on a single GPU", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from dataclasses import replace

    from mixture_exits_transformer_amd import lib
    from synth import cached_weights, prompts, uniforms, workload
    from synth.configs import BIAS_ALL_LAST

    torch.cuda.set_device(0)
    wl = workload(args.workload)
    if wl.name == "L":
        return bench_loss(args, wl)
    if wl.batch > 1:
        return bench_batch(args, wl)
    steps = args.steps if args.steps is not None else wl.decode_steps
    warmup = args.warmup if args.warmup is not None else 16
    prompt = prompts(wl)[0]
    U = uniforms(wl, steps=max(steps, warmup))[:, 0, :]
    max_ctx = len(prompt) + max(steps, warmup)

    path = cached_weights(wl.model)
    h = lib.nv_load(path, 1, max_ctx)
    dt, dt_s, exits = run_decode(lib, h, prompt, U, steps, warmup)
    tim, ker = timing_pass(lib, h, prompt, U, steps)
    lib.nv_free(h)
    tok_s = steps / dt

    base = base_s = None
    if not args.no_baseline:
        m4 = replace(wl.model, gate_bias=BIAS_ALL_LAST)
        h4 = lib.nv_load(cached_weights(m4), 1, max_ctx)
        dt4, dt4_s, ex4 = run_decode(lib, h4, prompt, U, steps, warmup)
        lib.nv_free(h4)
        assert set(ex4) == {4}
        base = steps / dt4
        base_s = steps / dt4_s

    # dominant kernel: the block-GEMM or attention symbol with the most device time (the
    # one-row gate/up product at a 512-token prompt, the decode attention at 8192)
    gemms = sorted([k for k in ker if k[0] in ("block_gemm", "attention")], key=lambda k: -k[2])
    _, nl, ms, by, kname, span = gemms[0]
    achieved = by / (ms * 1e-3) / 1e9
    counted = counted_traffic(kname)
    top = sorted(ker, key=lambda k: -k[2])[:8]
    hist = np.bincount(np.asarray(exits), minlength=5)[1:]
    window_mass = expected_window_mass(wl, len(prompt) - 1, steps)
    out = {
        "metric": "generated tokens/s, 1.5B bs=1, vs exit-4-forced decode; achieved HBM GB/s",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(dt / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.model.wdtype,
        "data": "synthetic: uniform-random token ids, seeded uniforms, random-init N(0,0.02) weights",
        "config": {"workload": f"{wl.name}: {wl.note}" + (
                       f"; timed: decode steps 1-{steps} of {wl.decode_steps} (positions {len(prompt) - 1}-"
                       f"{len(prompt) - 2 + steps})" if steps < wl.decode_steps else ""),
                   "batch": wl.batch, "prompt": len(prompt), "decode_steps": steps},
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counted[0] if counted else None,
                     "traffic_source": counted[1] if counted else None,
                     "launches": nl, "avg_launch_us": round(ms / max(nl, 1) * 1e3, 3),
                     "avg_span_us": round(span / max(nl, 1) * 1e3, 3) if span else None,
                     "bytes_per_launch": round(by / max(nl, 1)), "timing": TIMING_NOTE,
                     **profile_fields(kname, by / max(nl, 1), HBM_PEAK_GBS)},
        "block_gemm_all": {"achieved_GBps": round(tim["block_gemm"][1] / (tim["block_gemm"][0] * 1e-3) / 1e9, 1),
                           "launches": tim["block_gemm"][2]},
        "top_kernels": [{"kernel": k[4], "class": k[0], "launches": k[1],
                         "avg_us": round(k[2] / max(k[1], 1) * 1e3, 3),
                         "GBps": round(k[3] / (k[2] * 1e-3) / 1e9, 1) if k[2] > 0 else None} for k in top],
        "kernel_classes_ms_per_step": {k: round(v[0] / (steps * events_passes(steps)), 4) for k, v in tim.items()},
        "events_passes": events_passes(steps),
        "decode_api": "nv_generate (one sequence); nv_step_loop_tokens_per_s: one nv_step call per token",
        "nv_step_loop_tokens_per_s": round(steps / dt_s, 2),
        "exit4_forced_tokens_per_s": round(base, 2) if base else None,
        "exit4_forced_nv_step_loop_tokens_per_s": round(base_s, 2) if base else None,
        "speedup_vs_exit4": round(tok_s / base - 1.0, 4) if base else None,
        "exit_histogram": [int(x) for x in hist],
        "exit_mass_stated": list(STATED_MASS.get(wl.name, ())) or None,
        "exit_mass_realised": [round(float(x) / steps, 4) for x in hist],
        "exit_mass_expected_window": window_mass,
        "mean_segments_per_token": round(float(np.mean(exits)), 4),
        # the step's cost per segment a token runs: tokens/s moves with the realised exit mix
        # (which last-bit rounding changes on random-init weights), this figure does not
        "ms_per_segment_token": round(1e3 / tok_s / float(np.mean(exits)), 4),
        "exit4_ms_per_segment_token": round(1e3 / base / 4.0, 4) if base else None,
        "pages_reference": "57.9% wall-clock speedup at 1.5B on unspecified hardware (context only)",
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, path, prompt, U[:steps], args.cpu_budget)
    if args.calibrate_copy:
        calibration_copy(out)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
