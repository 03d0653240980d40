"""The host layer (argument checks, capacity, workspace plans, statistics
bookkeeping, training helpers) built with AddressSanitizer on the host side
only and run over tests/asan_host_exercise.cpp.  No GPU: the exercise program only takes
paths that return before any kernel launch.  The kernels' objects are the
ones the regular build wrote (_build/obj)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OBJ = os.path.join(ROOT, "_build", "obj")
OUT = os.path.join(ROOT, "_build", "asan")
KERNEL_OBJS = ["routing.o", "ffn_grouped.o", "combine.o", "backward.o"]


def test_host_layer_under_asan():
    if not all(os.path.exists(os.path.join(OBJ, o)) for o in KERNEL_OBJS):
        pytest.skip("kernel objects not built (run __graft_entry__.build())")
    os.makedirs(OUT, exist_ok=True)
    # host side instrumented; the device side of each file compiles as usual
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-I", os.path.join(ROOT, "include")]
    api_o = os.path.join(OUT, "moe_api_asan.o")
    r = subprocess.run([HIPCC, *common, *asan, "-x", "hip", "-c",
                        os.path.join(ROOT, "sparse_mixture_experts_capacity_amd", "csrc",
                                     "moe_api.cpp"), "-o", api_o],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    drv_o = os.path.join(OUT, "asan_host_exercise.o")
    r = subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
                        *asan, "-x", "c++", "-c", os.path.join(ROOT, "tests", "asan_host_exercise.cpp"),
                        "-o", drv_o], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = os.path.join(OUT, "asan_host_exercise")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *asan, drv_o, api_o,
                        *[os.path.join(OBJ, o) for o in KERNEL_OBJS], "-o", exe],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout
    assert "AddressSanitizer" not in r.stderr
