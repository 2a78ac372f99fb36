"""The C ABI library loads, exports every entry point include/nvium.h declares, and
rejects bad weights files before touching a device (no GPU needed)."""
import os
import re

import numpy as np
import pytest

from synth import TINY, cached_weights, file_size

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    src = open(os.path.join(ROOT, "include", "nvium.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nv_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    from mixture_exits_transformer_amd import lib
    L = lib.library()
    names = declared_entry_points()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(lib.EXPORTED)


def test_mem_required(weights_dir):
    from mixture_exits_transformer_amd import lib
    p = cached_weights(TINY, weights_dir)
    assert lib.nv_mem_required("/nonexistent/file.nvw", 1, 16) == 0
    assert lib.nv_mem_required(p, 0, 16) == 0
    a = lib.nv_mem_required(p, 1, 128)
    b = lib.nv_mem_required(p, 2, 128)
    # at least the weights, KV (8 layers x 2 x 128 positions x 128 floats) and hidden states
    assert a > file_size(TINY) + 8 * 2 * 128 * 128 * 4 + 128 * 128 * 4
    assert b > a


@pytest.mark.parametrize("damage", ["missing", "magic", "truncated", "shape", "form"])
def test_bad_weights_file_is_eio(weights_dir, tmp_path, damage):
    from mixture_exits_transformer_amd import lib
    src = cached_weights(TINY, weights_dir)
    p = str(tmp_path / "w.nvw")
    data = bytearray(open(src, "rb").read())
    if damage == "magic":
        data[0:8] = b"XXXXXXXX"
    elif damage == "truncated":
        data = data[: len(data) // 2]
    elif damage == "shape":
        data[16:20] = np.int32(100).tobytes()       # d_model not n_heads * head_dim
    elif damage == "form":
        data[84:88] = np.int32(2).tobytes()         # no head form 2
    if damage != "missing":
        open(p, "wb").write(data)
    with pytest.raises(lib.NvError) as e:
        lib.nv_load(p, 1, 16, use_torch=False)
    assert e.value.status == lib.NV_EIO


def test_null_arguments_are_einval():
    from mixture_exits_transformer_amd import lib
    L = lib.library()
    out = lib._P()
    assert L.nv_load(None, 1, 16, None, 0, None, lib.ctypes.byref(out)) == lib.NV_EINVAL
    assert L.nv_step(None, None, None, None) == lib.NV_EINVAL
    assert L.nv_flush(None, 0) == lib.NV_EINVAL
    assert L.nv_mixture_loss(None, 0, None, 0, 0.0, None, None) == lib.NV_EINVAL
