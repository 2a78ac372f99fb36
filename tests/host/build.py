"""Host-sanitizer builds of libnvium (no GPU needed to build or run them).

  build_driver(out_dir): nv_runtime.cpp with tests/host/mock_device.cpp and tests/host/drive.cpp,
      compiled by g++ with AddressSanitizer and UndefinedBehaviorSanitizer: the runtime's
      planning and bookkeeping over a host stand-in for the device.
  build_library(out_dir): the whole libnvium.so with hipcc, its host code instrumented with
      AddressSanitizer and UndefinedBehaviorSanitizer (device code as usual); load it into
      Python with the clang sanitizer runtime preloaded (ASAN_RUNTIME) and NVIUM_LIBRARY
      pointing at it.

    python tests/host/build.py <out_dir>          # both, then prints the commands to run
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "mixture_exits_transformer_amd", "csrc")
INC = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ASAN_RUNTIME = os.path.join(ROCM, "llvm", "lib", "clang", "22", "lib", "linux", "libclang_rt.asan-x86_64.so")

GXX_FLAGS = ["-std=c++17", "-O0", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
             "-I", CSRC, "-I", INC]
# host code only: every sanitizer flag goes to the host compilation
HIPCC_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fsanitize=address",
               "-Xarch_host", "-fsanitize=undefined",
               "-I", CSRC, "-I", INC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}")


def build_driver(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    srcs = [os.path.join(CSRC, "nv_runtime.cpp"), os.path.join(HERE, "mock_device.cpp"), os.path.join(HERE, "drive.cpp")]
    objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in srcs]
    with ThreadPoolExecutor(len(srcs)) as ex:
        list(ex.map(lambda so: _run(["g++"] + GXX_FLAGS + ["-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    exe = os.path.join(out_dir, "drive")
    _run(["g++", "-fsanitize=address,undefined", "-o", exe] + objs)
    return exe


def build_library(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    jobs = []
    for src in ("nv_kernels.hip", "nv_segment.hip", "nv_exit_op.hip", "nv_runtime.cpp"):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append((obj, [hipcc] + HIPCC_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(len(jobs)) as ex:
        list(ex.map(lambda j: _run(j[1]), jobs))
    lib = os.path.join(out_dir, "libnvium.so")
    # the sanitizer runtime is not linked in: the process that loads the library preloads it
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + [j[0] for j in jobs])
    return lib


if __name__ == "__main__":
    out = sys.argv[1] if len(sys.argv) > 1 else "/tmp/nvium_sanitize"
    exe = build_driver(os.path.join(out, "driver"))
    lib = build_library(os.path.join(out, "lib"))
    print(f"driver: {exe} <weights file> <max_batch> <max_ctx> <prompt lengths>")
    print(f"library: NVIUM_LIBRARY={lib} LD_PRELOAD={ASAN_RUNTIME} ASAN_OPTIONS=detect_leaks=0 "
          f"python -m pytest tests/test_abi_cpu.py")
