"""Seeded random-init weights and the on-disk weights file (".nvw").

File layout (little-endian), read independently by the C loader and by the
oracle's own reader:

  offset  field
  0       char[8]  magic "NVIUMW01"
  8       int32    header bytes (256)
  12      int32    n_layers L
  16      int32    d_model d
  20      int32    n_heads H
  24      int32    head_dim hd           (H * hd == d)
  28      int32    ffn F
  32      int32    vocab V
  36      int32    n_exits (4)
  40      int32    matrix dtype: 0 = fp32, 1 = bf16
  44      float32  RMSNorm eps
  48      float32  RoPE base
  52      int32[4] exit layer (1-based layer index after which exit k sits)
  68      float32[4] gate bias b_k (entry 4 is +inf: the last gate is fixed to 1)
  84      int32    head form: 0 = own norm + LM head per exit, 1 = shared final norm + LM
                   head, intermediate exits through an adapter MLP
  88      int32    adapter bottleneck r (head form 1)
  92      int32    router form: 0 = linear gate, 1 = router MLP
  96      int32    router hidden width rr (router form 1)
  100..255 zero
  256...  tensors, each starting at a multiple of 256 bytes, in this order:
          embed      [V][d]       matrix dtype
          per layer l = 0..L-1:
            attn_norm [d]         fp32
            wq, wk, wv, wo [d][d] matrix dtype (row = output feature)
            mlp_norm  [d]         fp32
            wg, wu    [F][d]      matrix dtype
            wd        [d][F]      matrix dtype
          per exit k = 0..3:
            router form 0: gate_w [d]          fp32 (zeros for the last exit: unused)
            router form 1: router_w1 [rr][d]   fp32 (zeros for the last exit)
                           router_b1 [rr]      fp32 (zeros)
                           router_w2 [rr]      fp32 (zeros for the last exit)
            head form 0:   exit_norm [d]       fp32
                           head      [V][d]    matrix dtype
            head form 1, k < 3: adapter_down [r][d]  matrix dtype
                                adapter_up   [d][r]  matrix dtype
          head form 1, after the exits:
            final_norm [d]        fp32
            head       [V][d]     matrix dtype

Values: tensor number i in the order above (0-based, norm vectors included) is
drawn from numpy.random.default_rng([seed, i]).standard_normal(float32) * 0.02;
RMSNorm weights are 1; the last exit's gate vector (or router tensors) and router
biases are 0.  bf16 matrices are the round-to-nearest-even bf16 of those float32
values.
"""
from __future__ import annotations

import hashlib
import os
import struct
import tempfile
import threading
from typing import Iterator, List, Tuple

import numpy as np

from .configs import ModelShape

MAGIC = b"NVIUMW01"
HEADER_BYTES = 256
ALIGN = 256


def tensor_specs(m: ModelShape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) in file order; kind is 'mat', 'norm' or 'gate'."""
    d, F, V = m.d_model, m.ffn, m.vocab
    specs = [("embed", (V, d), "mat")]
    for l in range(m.n_layers):
        specs += [
            (f"l{l}.attn_norm", (d,), "norm"),
            (f"l{l}.wq", (d, d), "mat"),
            (f"l{l}.wk", (d, d), "mat"),
            (f"l{l}.wv", (d, d), "mat"),
            (f"l{l}.wo", (d, d), "mat"),
            (f"l{l}.mlp_norm", (d,), "norm"),
            (f"l{l}.wg", (F, d), "mat"),
            (f"l{l}.wu", (F, d), "mat"),
            (f"l{l}.wd", (d, F), "mat"),
        ]
    for k in range(m.n_exits):
        last = k == m.n_exits - 1
        if m.router == "mlp":
            rr = m.router_dim
            specs += [
                (f"x{k}.router_w1", (rr, d), "zero" if last else "gate"),
                (f"x{k}.router_b1", (rr,), "zero"),
                (f"x{k}.router_w2", (rr,), "zero" if last else "gate"),
            ]
        else:
            specs += [(f"x{k}.gate_w", (d,), "zero" if last else "gate")]
        if m.head == "shared":
            if not last:
                specs += [
                    (f"x{k}.adapter_down", (m.adapter_dim, d), "mat"),
                    (f"x{k}.adapter_up", (d, m.adapter_dim), "mat"),
                ]
        else:
            specs += [
                (f"x{k}.exit_norm", (d,), "norm"),
                (f"x{k}.head", (V, d), "mat"),
            ]
    if m.head == "shared":
        specs += [("final_norm", (d,), "norm"), ("head", (V, d), "mat")]
    return specs


def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (uint16). Inputs are finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def header_bytes(m: ModelShape) -> bytes:
    wd = {"f32": 0, "bf16": 1}[m.wdtype]
    hdr = MAGIC + struct.pack(
        "<9i2f", HEADER_BYTES, m.n_layers, m.d_model, m.n_heads, m.head_dim, m.ffn, m.vocab,
        m.n_exits, wd, m.norm_eps, m.rope_base)
    hdr += struct.pack("<4i", *m.exit_layers)
    biases = list(m.gate_bias) + [float("inf")]
    hdr += struct.pack("<4f", *biases)
    hdr += struct.pack("<4i", 1 if m.head == "shared" else 0, m.adapter_dim if m.head == "shared" else 0,
                       1 if m.router == "mlp" else 0, m.router_dim if m.router == "mlp" else 0)
    return hdr + b"\0" * (HEADER_BYTES - len(hdr))


def _tensor_values(m: ModelShape, idx: int, shape, kind: str) -> np.ndarray:
    n = int(np.prod(shape))
    if kind == "norm":
        return np.ones(n, dtype=np.float32)
    if kind == "zero":
        return np.zeros(n, dtype=np.float32)
    rng = np.random.default_rng([m.seed, idx])
    return rng.standard_normal(n, dtype=np.float32) * np.float32(m.init_std)


def _encode(m: ModelShape, vals: np.ndarray, kind: str) -> bytes:
    if kind == "mat" and m.wdtype == "bf16":
        return f32_to_bf16_bits(vals).tobytes()
    return vals.astype(np.float32).tobytes()


def file_size(m: ModelShape) -> int:
    off = HEADER_BYTES
    for _, shape, kind in tensor_specs(m):
        el = 2 if (kind == "mat" and m.wdtype == "bf16") else 4
        off = _align(off) + int(np.prod(shape)) * el
    return _align(off)


def write_weights(m: ModelShape, path: str, threads: int = 8) -> str:
    """Write the seeded weights of model `m` to `path` (atomically)."""
    specs = tensor_specs(m)
    offsets = []
    off = HEADER_BYTES
    for _, shape, kind in specs:
        el = 2 if (kind == "mat" and m.wdtype == "bf16") else 4
        off = _align(off)
        offsets.append(off)
        off += int(np.prod(shape)) * el
    total = _align(off)
    tmp = path + f".tmp{os.getpid()}"
    with open(tmp, "wb") as f:
        f.truncate(total)
    mm = np.memmap(tmp, dtype=np.uint8, mode="r+", shape=(total,))
    mm[:HEADER_BYTES] = np.frombuffer(header_bytes(m), dtype=np.uint8)

    lock = threading.Lock()
    next_idx = [0]

    def worker():
        while True:
            with lock:
                i = next_idx[0]
                next_idx[0] += 1
            if i >= len(specs):
                return
            _, shape, kind = specs[i]
            data = _encode(m, _tensor_values(m, i, shape, kind), kind)
            mm[offsets[i]:offsets[i] + len(data)] = np.frombuffer(data, dtype=np.uint8)

    th = [threading.Thread(target=worker) for _ in range(max(1, threads))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    mm.flush()
    del mm
    os.replace(tmp, path)
    return path


def shape_key(m: ModelShape) -> str:
    return hashlib.sha1(repr(m).encode()).hexdigest()[:12]


def _tensor_key(m: ModelShape) -> str:
    """Key of the tensor values alone (the gate biases live in the header)."""
    from dataclasses import replace
    return shape_key(replace(m, gate_bias=(0.0, 0.0, 0.0)))


def cached_weights(m: ModelShape, cache_dir: str = None) -> str:
    """Path of the weights file for `m`, writing it once per cache directory.  A model
    that differs from a cached one only in its gate biases is made by copying that file
    and rewriting the header's bias field."""
    import shutil
    cache_dir = cache_dir or os.environ.get("NVIUM_WEIGHTS_DIR") or os.path.join(
        tempfile.gettempdir(), "nvium_weights")
    os.makedirs(cache_dir, exist_ok=True)
    stem = f"nvium-{m.n_layers}x{m.d_model}-{m.wdtype}-{_tensor_key(m)}"
    path = os.path.join(cache_dir, f"{stem}-{shape_key(m)}.nvw")
    size = file_size(m)
    if os.path.exists(path) and os.path.getsize(path) == size:
        return path
    sibling = next((os.path.join(cache_dir, f) for f in sorted(os.listdir(cache_dir))
                    if f.startswith(stem + "-") and f.endswith(".nvw")
                    and os.path.getsize(os.path.join(cache_dir, f)) == size), None)
    if sibling is None:
        return write_weights(m, path)
    tmp = path + f".tmp{os.getpid()}"
    shutil.copyfile(sibling, tmp)
    with open(tmp, "r+b") as f:
        f.write(header_bytes(m))
    os.replace(tmp, path)
    return path
