"""N-vium mixture-of-exits decode step on MI355X (gfx950): HIP kernels behind a C ABI.

The library is libnvium.so in this directory (built by `build.py`); `lib` is its
ctypes binding, with the same entry point names as include/nvium.h.
"""
from . import lib  # noqa: F401
from .lib import (NvError, nv_debug_frontiers, nv_debug_gates, nv_debug_hidden,  # noqa: F401
                  nv_debug_kv, nv_debug_logits, nv_exit_draw, nv_exit_draw_static, nv_exit_draw_workspace, nv_flush, nv_free,
                  nv_generate, nv_get_config, nv_last_error, nv_load, nv_mem_required, nv_mixture_loss,
                  nv_prefill, nv_step, nv_step_forced, nv_timing_enable, nv_timing_kernels, nv_timing_read)
