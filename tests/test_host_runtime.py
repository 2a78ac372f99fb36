"""libnvium's host runtime under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

nv_runtime.cpp is built with g++ over a host stand-in for the device (tests/host/
mock_device.cpp) and driven through its C ABI by tests/host/drive.cpp.  The stand-in checks
the plan of every launch: row tables, the order of the block products on each hidden-state
row, that every key an attention item reads has its K/V written at that layer (the K/V the
deferred layers must complete, gist.science summary, section 3 on complete KV recovery),
that the key splits of a row block tile its causal range, and that the split merges read
only partials the attention wrote.  The driver checks tokens, exits, the token fed back at
the next position, the per-segment frontiers and that flushing completes every layer.

Shapes: the tiny model (float32, head_dim 32), its bf16 form on each matrix-product path, the
shared-head / adapter / router-MLP form with ragged loss passes, and a 4-layer bf16 model with
head_dim 128 at an 8K context (prompts longer than the 4096-row launch group, 128 key splits)
and on the one-launch-per-segment kernel, and with the split-K decode product taking
groups of 5-64 rows (its MLP width 512 is one K slice).

The whole library with host sanitizers is checked by an opt-in test (about 2.5 minutes of
hipcc): NVIUM_SANITIZE_LIBRARY=1 builds it and runs tests/test_abi_cpu.py against it.
"""
import os
import subprocess
import sys

import pytest

from synth import TINY, cached_weights, tiny_variant
from tests.host.build import ASAN_RUNTIME, build_driver, build_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MODELS = {
    "tiny": TINY,
    "bf16": tiny_variant(wdtype="bf16", ffn=384),
    "forms": tiny_variant(head="shared", adapter_dim=16, router="mlp", router_dim=8),
    "hd128": tiny_variant(n_layers=4, d_model=256, n_heads=2, head_dim=128, ffn=512, vocab=512, wdtype="bf16"),
}

CASES = [
    # model, max_batch, max_ctx, prompt lengths, environment
    ("tiny", 4, 256, "40,17,3,100", {}),
    ("bf16", 4, 256, "40,17,3,100", {}),
    ("bf16", 4, 256, "40,17,3,100", {"NVIUM_MFMA_MIN_ROWS": "1"}),
    ("bf16", 4, 256, "40,17,3,100", {"NVIUM_MFMA_MIN_ROWS": "0"}),
    ("forms", 3, 128, "20,9,64", {"NVIUM_LOSS_ROWS": "7"}),
    ("hd128", 2, 8500, "8200,300", {}),
    ("hd128", 2, 1200, "1000,70", {"NVIUM_SEGMENT": "1"}),
    ("hd128", 4, 600, "40,17,3,100", {"NVIUM_SK_MIN_ROWS": "5", "NVIUM_SK_MAX_ROWS": "64"}),
]

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    return build_driver(str(tmp_path_factory.mktemp("host_driver")))


@pytest.mark.parametrize("model,batch,ctx,lens,env", CASES,
                         ids=[f"{c[0]}-{c[2]}" + "".join(f"-{k[6:].lower()}{v}" for k, v in c[4].items()) for c in CASES])
def test_host_runtime_sanitized(driver, weights_dir, model, batch, ctx, lens, env):
    path = cached_weights(MODELS[model], weights_dir)
    e = dict(os.environ)
    for k in ("NVIUM_MFMA_MIN_ROWS", "NVIUM_LOSS_ROWS", "NVIUM_SEGMENT", "NVIUM_SK_MIN_ROWS", "NVIUM_SK_MAX_ROWS"):
        e.pop(k, None)
    e.update(SAN_ENV)
    e.update(env)
    r = subprocess.run([driver, path, str(batch), str(ctx), lens], env=e, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:]
    assert r.stdout.rstrip().endswith("host runtime checks passed")


@pytest.mark.skipif(os.environ.get("NVIUM_SANITIZE_LIBRARY") != "1",
                    reason="opt-in (NVIUM_SANITIZE_LIBRARY=1): builds the whole library with hipcc, ~2.5 min")
def test_abi_under_sanitized_library(tmp_path):
    lib = build_library(str(tmp_path / "lib"))
    e = dict(os.environ)
    e.update({"NVIUM_LIBRARY": lib, "LD_PRELOAD": ASAN_RUNTIME, "ASAN_OPTIONS": "detect_leaks=0",
              "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")], env=e, cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-4000:]
