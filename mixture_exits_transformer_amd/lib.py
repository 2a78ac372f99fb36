"""ctypes binding of libnvium (include/nvium.h): the same entry points, argument
marshalling only.  PyTorch provides the device arena and the stream.

Every function raises NvError on a non-zero status.  Nothing here computes: if the
shared library is missing, loading fails with an error (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# NVIUM_LIBRARY names another build of the same library (for example one built with host
# sanitizers); by default the in-tree build is loaded
LIB_PATH = os.environ.get("NVIUM_LIBRARY") or os.path.join(HERE, "libnvium.so")

NV_OK, NV_EINVAL, NV_ESTATE, NV_ECAPACITY, NV_EIO, NV_EDEVICE = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "NV_OK", -1: "NV_EINVAL", -2: "NV_ESTATE", -3: "NV_ECAPACITY", -4: "NV_EIO",
                -5: "NV_EDEVICE"}


class NvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class nv_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_exits", ctypes.c_int32), ("wdtype", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("exit_layer", ctypes.c_int32 * 4),
                ("gate_bias", ctypes.c_float * 4), ("head_form", ctypes.c_int32), ("adapter_dim", ctypes.c_int32),
                ("router_form", ctypes.c_int32), ("router_dim", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_F32P = ctypes.POINTER(ctypes.c_float)
_F64P = ctypes.POINTER(ctypes.c_double)

_SIGS = {
    "nv_mem_required": (ctypes.c_size_t, [ctypes.c_char_p, ctypes.c_int32, ctypes.c_int32]),
    "nv_load": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t, _P,
                               ctypes.POINTER(_P)]),
    "nv_free": (None, [_P]),
    "nv_last_error": (ctypes.c_char_p, [_P]),
    "nv_get_config": (ctypes.c_int, [_P, ctypes.POINTER(nv_config)]),
    "nv_prefill": (ctypes.c_int, [_P, ctypes.c_int32, _I32P, ctypes.c_int32]),
    "nv_step": (ctypes.c_int, [_P, _F32P, _I32P, _I32P]),
    "nv_step_forced": (ctypes.c_int, [_P, _F32P, _I32P, _I32P, _I32P]),
    "nv_generate": (ctypes.c_int, [_P, _I32P, ctypes.c_int32, ctypes.c_int32, _F32P, ctypes.c_int32, _I32P,
                                   _I32P]),
    "nv_mixture_loss": (ctypes.c_int, [_P, ctypes.c_int32, _I32P, ctypes.c_int32, ctypes.c_double, _F64P, _F64P]),
    "nv_flush": (ctypes.c_int, [_P, ctypes.c_int32]),
    "nv_debug_frontiers": (ctypes.c_int, [_P, ctypes.c_int32, _I32P, _I32P]),
    "nv_debug_logits": (ctypes.c_int, [_P, ctypes.c_int32, _F32P]),
    "nv_debug_gates": (ctypes.c_int, [_P, ctypes.c_int32, _F64P]),
    "nv_debug_kv": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _F32P,
                                   _F32P]),
    "nv_debug_hidden": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _F32P]),
    "nv_exit_draw_workspace": (ctypes.c_size_t, [ctypes.c_int32]),
    "nv_exit_draw": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                    ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "nv_exit_draw_static": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_float, ctypes.c_float, _P, _P, _P]),
    "nv_timing_enable": (ctypes.c_int, [_P, ctypes.c_int32]),
    "nv_timing_read": (ctypes.c_int, [_P, _F64P, _F64P, ctypes.POINTER(ctypes.c_int64)]),
    "nv_timing_kernels": (ctypes.c_int, [_P, ctypes.c_char_p, ctypes.c_size_t]),
}
TIME_CLASSES = ("block_gemm", "attention", "exit_head", "other")
EXPORTED = tuple(_SIGS)


def library(path: str = None):
    """Load libnvium.so (built by mixture_exits_transformer_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m mixture_exits_transformer_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _check(h, status: int):
    if status != NV_OK:
        msg = library().nv_last_error(h).decode() if h else ""
        raise NvError(status, msg)


class Handle:
    """An nv_model* plus the torch objects it borrows (arena, stream)."""

    def __init__(self, ptr, arena=None, stream=None):
        self.ptr = ptr
        self.arena = arena
        self.stream = stream
        cfg = nv_config()
        _check(ptr, library().nv_get_config(ptr, ctypes.byref(cfg)))
        self.cfg = cfg

    @property
    def vocab(self):
        return self.cfg.vocab


def nv_mem_required(path: str, max_batch: int, max_ctx: int) -> int:
    return int(library().nv_mem_required(path.encode(), max_batch, max_ctx))


def nv_load(path: str, max_batch: int, max_ctx: int, device: str = "cuda:0", use_torch=True,
            stream=None) -> Handle:
    """Load weights.  With use_torch the device arena is a torch uint8 tensor on `device`
    and work goes on `stream` (default: torch's current stream there); without it the
    library allocates with hipMalloc and uses the null stream."""
    lib = library()
    arena = None
    arena_ptr, arena_bytes, stream_ptr = None, 0, None
    if use_torch:
        import torch
        dev = torch.device(device)
        need = nv_mem_required(path, max_batch, max_ctx)
        if need == 0:
            raise NvError(NV_EIO, f"cannot read weights header of {path}")
        arena = torch.empty(need, dtype=torch.uint8, device=dev)
        arena_ptr, arena_bytes = arena.data_ptr(), need
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        stream_ptr = stream.cuda_stream
    out = _P()
    st = lib.nv_load(path.encode(), max_batch, max_ctx, arena_ptr, arena_bytes, stream_ptr,
                     ctypes.byref(out))
    if st != NV_OK:
        msg = lib.nv_last_error(out).decode() if out else ""
        if out:
            lib.nv_free(out)
        raise NvError(st, msg)
    return Handle(out, arena, stream)


def nv_free(h: Handle) -> None:
    if h.ptr:
        library().nv_free(h.ptr)
        h.ptr = None
        h.arena = None


def nv_last_error(h: Handle) -> str:
    return library().nv_last_error(h.ptr).decode()


def nv_prefill(h: Handle, seq: int, tokens) -> None:
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    _check(h.ptr, library().nv_prefill(h.ptr, seq, _ptr(t, ctypes.c_int32), len(t)))


def nv_step(h: Handle, uniforms) -> Tuple[np.ndarray, np.ndarray]:
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(-1, 4)
    n = u.shape[0]
    tok = np.empty(n, np.int32)
    ex = np.empty(n, np.int32)
    _check(h.ptr, library().nv_step(h.ptr, _ptr(u, ctypes.c_float), _ptr(tok, ctypes.c_int32),
                                    _ptr(ex, ctypes.c_int32)))
    return tok, ex


def nv_step_forced(h: Handle, uniforms, next_inputs) -> Tuple[np.ndarray, np.ndarray]:
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(-1, 4)
    n = u.shape[0]
    f = np.ascontiguousarray(next_inputs, dtype=np.int32).reshape(n)
    tok = np.empty(n, np.int32)
    ex = np.empty(n, np.int32)
    _check(h.ptr, library().nv_step_forced(h.ptr, _ptr(u, ctypes.c_float), _ptr(f, ctypes.c_int32),
                                           _ptr(tok, ctypes.c_int32), _ptr(ex, ctypes.c_int32)))
    return tok, ex


SCHED_LOCKSTEP, SCHED_GREEDY = 0, 1


def nv_generate(h: Handle, seqs, uniforms, policy: int = SCHED_GREEDY) -> Tuple[np.ndarray, np.ndarray]:
    """uniforms [n_seq][n_tokens][4] -> (tokens, exits), each [n_seq][n_tokens]."""
    q = np.ascontiguousarray(seqs, dtype=np.int32).reshape(-1)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    assert u.ndim == 3 and u.shape[0] == len(q) and u.shape[2] == 4, u.shape
    tok = np.zeros(u.shape[:2], np.int32)
    ex = np.zeros(u.shape[:2], np.int32)
    _check(h.ptr, library().nv_generate(h.ptr, _ptr(q, ctypes.c_int32), len(q), u.shape[1], _ptr(u, ctypes.c_float),
                                        policy, _ptr(tok, ctypes.c_int32), _ptr(ex, ctypes.c_int32)))
    return tok, ex


def nv_mixture_loss(h: Handle, seq: int, tokens, beta: float = 0.0, per_pos: bool = False):
    """(L_mix, L_compute, L_total), and with per_pos the [n-1][10] rows w_1..4,
    log pi_1..4 of the target, -log pi_mix, expected depth.  Prefills `seq` with tokens."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.empty(3, np.float64)
    pp = np.empty((max(len(t) - 1, 0), 10), np.float64) if per_pos else None
    _check(h.ptr, library().nv_mixture_loss(h.ptr, seq, _ptr(t, ctypes.c_int32), len(t), float(beta),
                                            _ptr(out, ctypes.c_double),
                                            _ptr(pp, ctypes.c_double) if per_pos else None))
    return (tuple(float(x) for x in out), pp) if per_pos else tuple(float(x) for x in out)


def _dptr(t) -> int:
    """Device address of a torch tensor (or an int address)."""
    return t if isinstance(t, int) else t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def nv_exit_draw_workspace(vocab: int) -> int:
    return int(library().nv_exit_draw_workspace(vocab))


def nv_exit_draw(h, norm_w, head_w, wdtype: int, d: int, vocab: int, eps: float, u: float, logits, token,
                 workspace, workspace_bytes: int, stream=None) -> None:
    """Enqueue one exit's head + draw on device buffers (torch tensors or addresses); the
    outputs `logits` [vocab] float32 and `token` [1] int32 are valid once the stream has run it."""
    st = library().nv_exit_draw(_dptr(h), _dptr(norm_w), _dptr(head_w), wdtype, d, vocab, eps, u, _dptr(logits),
                                _dptr(token), _dptr(workspace), workspace_bytes, _stream_ptr(stream))
    if st != NV_OK:
        raise NvError(st, "nv_exit_draw")


def nv_exit_draw_static(h, norm_w, head_w, wdtype: int, d: int, vocab: int, eps: float, u: float, logits, token,
                        stream=None) -> None:
    """nv_exit_draw with the library's own per-GPU scratch (allocates nothing; calls that
    overlap on one GPU race)."""
    st = library().nv_exit_draw_static(_dptr(h), _dptr(norm_w), _dptr(head_w), wdtype, d, vocab, eps, u,
                                       _dptr(logits), _dptr(token), _stream_ptr(stream))
    if st != NV_OK:
        raise NvError(st, "nv_exit_draw_static")


def nv_get_config(h: Handle) -> nv_config:
    """The model shape read from the weights file."""
    c = nv_config()
    _check(h.ptr, library().nv_get_config(h.ptr, ctypes.byref(c)))
    return c


def nv_flush(h: Handle, seq: int = -1) -> None:
    _check(h.ptr, library().nv_flush(h.ptr, seq))


def nv_debug_frontiers(h: Handle, seq: int) -> Tuple[int, np.ndarray]:
    n = ctypes.c_int32()
    f = np.empty(4, np.int32)
    _check(h.ptr, library().nv_debug_frontiers(h.ptr, seq, ctypes.byref(n), _ptr(f, ctypes.c_int32)))
    return int(n.value), f


def nv_debug_logits(h: Handle, seq: int) -> np.ndarray:
    out = np.empty(h.cfg.vocab, np.float32)
    _check(h.ptr, library().nv_debug_logits(h.ptr, seq, _ptr(out, ctypes.c_float)))
    return out


def nv_debug_gates(h: Handle, seq: int) -> np.ndarray:
    out = np.empty(4, np.float64)
    _check(h.ptr, library().nv_debug_gates(h.ptr, seq, _ptr(out, ctypes.c_double)))
    return out


def nv_debug_kv(h: Handle, seq: int, layer: int, pos0: int, n: int) -> Tuple[np.ndarray, np.ndarray]:
    c = h.cfg
    k = np.empty((n, c.n_heads, c.head_dim), np.float32)
    v = np.empty((n, c.n_heads, c.head_dim), np.float32)
    _check(h.ptr, library().nv_debug_kv(h.ptr, seq, layer, pos0, n, _ptr(k, ctypes.c_float),
                                        _ptr(v, ctypes.c_float)))
    return k, v


def nv_debug_hidden(h: Handle, seq: int, pos0: int, n: int) -> np.ndarray:
    out = np.empty((n, h.cfg.d_model), np.float32)
    _check(h.ptr, library().nv_debug_hidden(h.ptr, seq, pos0, n, _ptr(out, ctypes.c_float)))
    return out


def nv_timing_enable(h: Handle, on=True) -> None:
    """on: False/0 stop, True/1 events, 2 events and per-block device stamps."""
    _check(h.ptr, library().nv_timing_enable(h.ptr, int(on)))


def nv_timing_read(h: Handle) -> dict:
    """{class: (device ms, algorithmic bytes, launches)} since nv_timing_enable."""
    ms = np.zeros(4, np.float64)
    by = np.zeros(4, np.float64)
    n = np.zeros(4, np.int64)
    _check(h.ptr, library().nv_timing_read(h.ptr, _ptr(ms, ctypes.c_double), _ptr(by, ctypes.c_double),
                                           _ptr(n, ctypes.c_int64)))
    return {c: (float(ms[i]), float(by[i]), int(n[i])) for i, c in enumerate(TIME_CLASSES)}


def nv_timing_kernels(h: Handle) -> list:
    """[(class, launches, device ms, algorithmic bytes, symbol, span ms or None)] since
    nv_timing_enable; device ms is launch to completion (HIP events), span ms the first
    block start to last block end (device stamps) of the kernels that record them."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(h.ptr, library().nv_timing_kernels(h.ptr, buf, len(buf)))
    out = []
    for line in buf.value.decode().splitlines():
        k, n, ms, by, span, name = line.split("\t", 5)
        out.append((TIME_CLASSES[int(k)], int(n), float(ms), float(by), name, float(span) if float(span) >= 0 else None))
    return out
