"""Build libtern.so in-tree with hipcc for gfx950 (cross-compiles on a host
without a GPU)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtern.so")
BENCH_LIB = os.path.join(HERE, "libtern_bench.so")  # measurement helper, not the matmul path

# (source, extra flags).  The GEMM keeps its MFMA results in ordinary VGPRs:
# it rescales them with VALU arithmetic right away (per group), and results
# in accumulator registers would need a copy out for each.
SOURCES = [
    ("tern_kernels.hip", []),
    ("tern_gemm.hip", ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"]),
    ("tern_t5.hip", []),
    ("tern_gemv1.hip", []),
    ("tern_api.cpp", []),
    ("tern_codec.cpp", []),
]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed FP32 VALU instructions stay off: the compiler must not form them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]

NOISE = "'-packed-fp32-ops' is not a recognized feature"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if NOISE not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False) -> str:
    """Compile every source and link libtern.so (always recompiles)."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(objdir, src + ".o") for src, _ in SOURCES]
    # the sources compile independently: one hipcc per source, in parallel
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
        jobs = [pool.submit(_run, [hipcc(), *HIPCC_FLAGS, *extra, *inc, "-c", os.path.join(CSRC, src), "-o", obj],
                            verbose)
                for (src, extra), obj in zip(SOURCES, objs)]
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    # the benchmark's read-only streaming kernel, a library of its own
    tmpb = BENCH_LIB + ".tmp"
    _run([hipcc(), *HIPCC_FLAGS, "-shared", os.path.join(CSRC, "tern_bench.hip"), "-o", tmpb], verbose)
    os.replace(tmpb, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
