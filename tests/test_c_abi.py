"""The C-ABI from plain C: tests/c_abi_client.c includes only
include/mmrelu.h, is compiled as strict C99 with gcc and linked against
libmmrelu.so, and calls the host-side entry points (planning, workspace
sizing, status strings, argument checks that fail before any launch). Each
line it prints must equal the same call made through the Python binding. No
GPU is needed: none of these calls reaches the device."""
import json
import os
import shutil
import subprocess

import pytest

import tiled_matmul_relu_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_client.c")


@pytest.fixture(scope="module")
def client_lines(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib = mm.load_library()
    libdir = os.path.dirname(lib._name)
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_client")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), SRC,
           "-o", exe, "-L", libdir, "-lmmrelu", f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=60).stdout
    return [json.loads(line) for line in out.splitlines()]


def test_c_client_matches_python_binding(client_lines):
    by_call = {}
    for d in client_lines:
        by_call.setdefault(d["call"], []).append(d)
    assert by_call["version"][0]["value"] == mm.version()
    assert by_call["status"][0]["value"] == [mm.status_string(0), mm.status_string(mm.MMRELU_ERR_MISALIGNED),
                                            mm.status_string(99)]
    plans = by_call["plan"]
    assert len(plans) == 8
    shapes = [
        (mm.DTYPE_F32, 256, 256, 256, 256, 256, 256), (mm.DTYPE_F32, 1024, 1024, 1024, 1024, 1024, 1024),
        (mm.DTYPE_F32, 4096, 4096, 4096, 4096, 4096, 4096), (mm.DTYPE_F32, 4097, 3001, 2049, 2049, 3001, 3001),
        (mm.DTYPE_BF16, 8192, 8192, 8192, 8192, 8192, 8192), (mm.DTYPE_BF16, 4097, 3001, 2049, 2049, 3001, 3001),
        (mm.DTYPE_F32, 8192, 1, 8192, 8192, 1, 1),
    ]
    for got, args in zip(plans, shapes):
        want = mm.mmrelu_plan(*args, cus=256)
        assert got["status"] == 0 and got["shape"] == list(args[1:4])
        assert (got["variant"], got["name"], got["grid"], got["waves"]) == (
            want["variant"], want["name"], want["grid"], want["waves"]), (args, got, want)
    assert plans[-1]["status"] == mm.MMRELU_ERR_INVALID_VALUE
    w = by_call["waves"][0]
    assert w["status"] == 0 and tuple(w["value"]) == mm.mmrelu_wave_quantization(3055, 1280)
    ws = by_call["workspace"][0]
    assert ws["status"] == 0
    assert ws["value"] == mm.mmrelu_strided_workspace_size(mm.DTYPE_BF16, mm.ACT_RELU, 0x100000, 0x200000, 0,
                                                           0x300000, 1024, 512, 256, 1, 1024, 512, 1, 512, 1)
    assert ws["value"] >= 1024 * 256 * 2           # the transposed A is copied once
    assert by_call["checks"][0]["value"] == [mm.MMRELU_ERR_INVALID_VALUE, mm.MMRELU_ERR_NULL_POINTER,
                                             mm.MMRELU_ERR_MISALIGNED, mm.MMRELU_ERR_INVALID_VALUE]
