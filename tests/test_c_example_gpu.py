"""The library used from C without Python or torch (needs the GPU): the C
example tiled_matmul_relu_amd/examples/mmrelu_run.c, built by build() into
tiled_matmul_relu_amd/_build/mmrelu_run, allocates device memory with the
HIP runtime, calls mmrelu_f32 / mmrelu_bf16 through the C-ABI and writes C
to a file. It runs here as a child process on inputs from the seeded
generators; its output is compared with the fp64 oracle at the parity
tolerances (fp32 max |C - R| <= 1e-4 sqrt(K); bf16 relative Frobenius
<= 1e-2, elementwise 2^-8 |R| + 1e-6), on an aligned shape and on a ragged
one (odd sizes: the unaligned fp32 and any-layout bf16 kernels)."""
import math
import os
import subprocess

import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tiled_matmul_relu_amd", "_build", "mmrelu_run")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(300, 264, 136), (257, 129, 65)], ids=["aligned", "ragged"])
def test_c_example_matches_oracle(tmp_path, dtype, M, N, K):
    assert os.path.exists(EXE), "C example not built: run build() first"
    a = datagen.normal_f32(71, M, K, 1 / math.sqrt(K))
    b = datagen.normal_f32(72, K, N, 1 / math.sqrt(K))
    if dtype == "bf16":
        a, b = datagen.f32_to_bf16_bits(a), datagen.f32_to_bf16_bits(b)
    pa, pb, pc = (str(tmp_path / n) for n in ("a.bin", "b.bin", "c.bin"))
    a.tofile(pa)
    b.tofile(pb)
    print(f"C example {dtype} {M}x{N}x{K}", flush=True)
    r = subprocess.run([EXE, dtype, str(M), str(N), str(K), pa, pb, pc], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    c = np.fromfile(pc, dtype=np.float32 if dtype == "f32" else np.uint16).reshape(M, N)
    ref = oracle.mmrelu(a, b)
    if dtype == "f32":
        assert np.abs(c.astype(np.float64) - ref).max() <= 1e-4 * math.sqrt(K)
    else:
        cf = datagen.bf16_bits_to_f32(c).astype(np.float64)
        assert np.linalg.norm(cf - ref) / np.linalg.norm(ref) <= 1e-2
        assert np.all(np.abs(cf - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    assert np.all(c.astype(np.float64) >= 0) if dtype == "f32" else np.all(datagen.bf16_bits_to_f32(c) >= 0)


def test_c_example_reports_bad_arguments(tmp_path):
    """Usage errors end with status 1 and a message before any GPU work."""
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    r = subprocess.run([EXE, "f64", "4", "4", "4", "a", "b", "c"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "dtype" in r.stderr
    r = subprocess.run([EXE, "f32", "4", "4", "4", str(tmp_path / "missing"), "b", "c"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 1 and "read" in r.stderr
