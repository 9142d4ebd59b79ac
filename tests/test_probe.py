"""The matrix-core ceiling probe library (a measurement for bench.py, not part
of libmmrelu) on the CPU: it is built, exports its one entry point, and
rejects bad arguments before launching anything."""
import ctypes
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tiled_matmul_relu_amd", "_build", "libmfma_ceiling.so")


def load():
    assert os.path.exists(PROBE), "run build() first"
    lib = ctypes.CDLL(PROBE)
    fn = lib.mfma_ceiling_bf16
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return fn


def test_probe_rejects_bad_arguments_before_launch():
    fn = load()
    p = 1 << 20   # a 16-byte aligned stand-in address; never dereferenced, every call below is refused
    ok = dict(a=p, b=p, na=64, nb=64, shape=16, tiles=4, slabs=1, out=p)

    def call(**kw):
        a = {**ok, **kw}
        return fn(a["a"], a["b"], a["na"], a["nb"], a["shape"], a["tiles"], a["slabs"], a["out"], None)

    assert call(a=None) == 1
    assert call(b=None) == 1
    assert call(out=None) == 1
    assert call(na=7) == 1
    assert call(nb=0) == 1
    assert call(tiles=0) == 1
    assert call(slabs=-1) == 1
    assert call(shape=8) == 1
    assert call(a=p + 2) == 1        # A not 16-byte aligned
    assert call(b=p + 8) == 1
