"""Build libmmrelu.so (the gfx950 HIP library) in-tree with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into ``tiled_matmul_relu_amd/libmmrelu.so``. The C example
(``examples/mmrelu_run.c``, the library used from C without Python) is then
built with gcc against the library into ``_build/mmrelu_run``, and the
matrix-core ceiling probe (``probe/mfma_ceiling.hip``, a measurement used by
``bench.py --mfma-ceiling``) into ``_build/libmfma_ceiling.so``. Run ``python
-m tiled_matmul_relu_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmmrelu.so")
OBJDIR = os.path.join(PKG, "_build")
EXAMPLE = os.path.join(OBJDIR, "mmrelu_run")
PROBE_SRC = os.path.join(PKG, "probe", "mfma_ceiling.hip")
PROBE_LIB = os.path.join(OBJDIR, "libmfma_ceiling.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # hipcc forms packed fp32 instructions on its own; keep them out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


# Per-file compiler options. The four-wave bf16 kernel is built with the
# register-pressure-first scheduler, the build its timings were taken with
# (180 VGPRs against 176 with the default scheduler, same AGPR moves); with
# larger wave tiles the default scheduler shuffled accumulators between AGPRs
# inside the K loop.
FILE_FLAGS = {
    "k_bf16_mfma.hip": ["-mllvm", "--amdgpu-sched-strategy=iterative-minreg"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    build_example()
    build_probe()
    return LIB


def build_probe() -> str:
    """The matrix-core ceiling probe (bench.py --mfma-ceiling), a library of
    its own: it is a measurement, not part of libmmrelu."""
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([hipcc(), *HIPCC_FLAGS, "-shared", PROBE_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe build failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build_example() -> str:
    """Strict C99 with the HIP runtime headers as system headers; the binary
    finds libmmrelu.so next to its own directory's parent ($ORIGIN/..)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C example")
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", "-isystem", os.path.join(ROCM, "include"),
           os.path.join(PKG, "examples", "mmrelu_run.c"), "-o", EXAMPLE, f"-L{PKG}", "-lmmrelu",
           f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", "-Wl,-rpath,$ORIGIN/..",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("C example build failed:\n" + r.stdout + r.stderr)
    return EXAMPLE


if __name__ == "__main__":
    print(build())
