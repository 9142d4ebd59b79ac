#!/usr/bin/env python3
"""Benchmark of C = relu(A·B) on one MI355X through the gfx950 C-ABI library.

A step is one call of the library on the headline workload: bf16 inputs and
output, fp32 accumulation, M = N = K = 8192, entries N(0,1)/sqrt(K) rounded
to bf16, seeded synthetic data already resident in HBM. The fp32 4096^3
U(-1,1) workload is timed the same way and reported beside it.

Prints one JSON line: throughput (TFLOP/s, 2MNK per step), the roofline
object for the dominant kernel (achieved FLOP/s per launch from HIP events on
the launch stream against the bf16 dense matrix-core peak) and the CPU
baseline (the fp64 oracle timed on a bounded sample of the same workload on
this host's cores), whose result is compared with the timed output (parity).

Order of the GPU work: the headline's W warm-up and K timed calls run twice
in a row, first as `cold_start` (the board's power management settles over
the first ~25 calls of a process), then for `value`; then the matrix-core
ceiling probe, the all-zero power check and the fp32 workload.
"""
import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # MI355X dense matrix-core peaks
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "bf16": ["tiled_matmul_relu_amd/csrc/k_bf16_pingpong.hip", "tiled_matmul_relu_amd/csrc/device_common.hpp"],
    "f32": ["tiled_matmul_relu_amd/csrc/k_f32_mfma.hip", "tiled_matmul_relu_amd/csrc/device_common.hpp"],
}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kind: str, kernel_name: str):
    """HBM bytes per launch from committed counter runs, or None when the
    kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_hash(kind):
        return None
    return rec.get("bytes_per_launch")


def read_counters(path, counter):
    """Per-kernel lists of one counter's per-dispatch values from a rocprofv3
    counter_collection.csv."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def calibrated_counters(fetch_csv, write_csv, calib_mib):
    """FETCH_SIZE and WRITE_SIZE per kernel name (KiB per dispatch, lists),
    and the factors that turn them into bytes: each counter is scaled by what
    it reads for the calibration copy of calib_mib MiB in the same run, whose
    true traffic is calib_mib MiB read and calib_mib MiB written."""
    fetch = read_counters(fetch_csv, "FETCH_SIZE")
    write = read_counters(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k]
    if len(copy) != 1 or copy[0] not in write:
        raise SystemExit(f"counters: expected one copy kernel in the counter files, found {copy}")
    # The calibration copy is the largest copy dispatch of the run (inputs
    # may also be staged through small copy kernels).
    calib = calib_mib * (1 << 20)
    return fetch, write, calib / (max(fetch[copy[0]]) * 1024), calib / (max(write[copy[0]]) * 1024)


def counter_summary(fetch_csv, write_csv, calib_mib):
    """One JSON line per mmrelu kernel in two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE) of the same command: calibrated HBM bytes read and written
    per dispatch (mean over its dispatches)."""
    fetch, write, f_fac, w_fac = calibrated_counters(fetch_csv, write_csv, calib_mib)
    for name in sorted(fetch):
        if "mmrelu" not in name or name not in write:
            continue
        fv, wv = fetch[name], write[name]
        print(json.dumps({"kernel_symbol": name.split(">(")[0] + ">", "dispatches": min(len(fv), len(wv)),
                          "fetch_bytes": round(sum(fv) / len(fv) * 1024 * f_fac),
                          "write_bytes": round(sum(wv) / len(wv) * 1024 * w_fac),
                          "fetch_scale": round(f_fac, 4), "write_scale": round(w_fac, 4)}))


def record_traffic(fetch_csv, write_csv, calib_mib, command):
    """Write profiles/traffic.json from two rocprofv3 --pmc runs of this script
    (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch) that included the
    calibration copy of calib_mib MiB (--calib-copy-mib). Each counter is scaled
    by what it reads for that copy, whose true traffic is calib_mib MiB read and
    calib_mib MiB written."""
    import datagen
    import tiled_matmul_relu_amd as mm
    fetch, write, f_fac, w_fac = calibrated_counters(fetch_csv, write_csv, calib_mib)
    recs = {}
    for kind, cid in (("bf16", 5), ("f32", 3)):
        cfg = datagen.CONFIGS[cid]
        plan = mm.mmrelu_plan(mm.DTYPE_BF16 if kind == "bf16" else mm.DTYPE_F32, cfg.M, cfg.N, cfg.K,
                              cfg.lda, cfg.ldb, cfg.ldc)
        family = plan["name"].split("<")[0]          # the planner's kernel for this workload
        names = [k for k in fetch if family + "<" in k]
        if len(names) != 1 or names[0] not in write:
            raise SystemExit(f"record-traffic: expected one {family} kernel, found {names}")
        fv, wv = fetch[names[0]], write[names[0]]
        fb = sum(fv) / len(fv) * 1024 * f_fac
        wb = sum(wv) / len(wv) * 1024 * w_fac
        s_in = 2 if kind == "bf16" else 4
        recs[plan["name"]] = {
            "kernel_symbol": names[0].split(">(")[0] + ">",
            "workload": cfg.name,
            "source_sha256": source_hash(kind),
            "bytes_per_launch": round(fb + wb),
            "fetch_bytes_per_launch": round(fb),
            "write_bytes_per_launch": round(wb),
            "algorithmic_bytes": s_in * (cfg.M * cfg.K + cfg.K * cfg.N) + s_in * cfg.M * cfg.N,
            "dispatches": min(len(fv), len(wv)),
            "fetch_scale": round(f_fac, 4),
            "write_scale": round(w_fac, 4),
            "calibration": f"{calib_mib} MiB device-to-device copy in the same run",
            "command": command,
        }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(recs, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(recs, indent=1, sort_keys=True))


def calib_copy(mib, torch):
    """One device-to-device copy of mib MiB (a kernel of known traffic, for
    scaling memory counters); returns the bytes copied."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return n * 4


def to_device(x, torch):
    import numpy as np
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def prepare_workload(cfg, torch, mm, datagen):
    """Host inputs of a workload, their device copies, a NaN-filled C and the
    call's arguments on torch's current stream."""
    a, b = datagen.make_inputs(cfg)
    da, db = to_device(a, torch), to_device(b, torch)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    c = torch.full((cfg.M, cfg.ldc), float("nan"), dtype=dt, device="cuda")
    stream = torch.cuda.current_stream()
    fn = mm.mmrelu_f32 if cfg.dtype == "f32" else mm.mmrelu_bf16
    args = (da.data_ptr(), db.data_ptr(), c.data_ptr(), cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb, cfg.ldc,
            stream.cuda_stream)
    plan = mm.mmrelu_plan(mm.DTYPE_F32 if cfg.dtype == "f32" else mm.DTYPE_BF16, cfg.M, cfg.N, cfg.K,
                          cfg.lda, cfg.ldb, cfg.ldc)
    return {"cfg": cfg, "fn": fn, "args": args, "stream": stream, "plan": plan, "inputs": (a, b),
            "da": da, "db": db, "c": c}


def time_calls(w, steps, warmup, torch, mm):
    """W warm-up calls, then `steps` calls back to back between two HIP events
    on the launch stream (the timed region: ms per call = elapsed / steps),
    then `steps` more calls with an event after each, for the distribution
    of single calls (mean, median, P95)."""
    cfg, fn, args, stream = w["cfg"], w["fn"], w["args"], w["stream"]
    for _ in range(warmup):
        rc = fn(*args)
        if rc != mm.MMRELU_OK:
            raise RuntimeError(mm.status_string(rc))
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn(*args)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn(*args)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    per_call = {"calls": steps, "mean_ms": round(sum(t) / steps, 4), "median_ms": round(median(t), 4),
                "p95_ms": round(t[min(steps - 1, int(math.ceil(0.95 * steps)) - 1)], 4),
                "tflops_median": round(cfg.flops / (median(t) * 1e-3) / 1e12, 2)}
    return {"ms": ms, "tflops": cfg.flops / (ms * 1e-3) / 1e12, "per_call": per_call}


def time_workload(cfg, steps, warmup, torch, mm, datagen):
    """prepare_workload, then time_calls; returns both records merged."""
    w = prepare_workload(cfg, torch, mm, datagen)
    return {**w, **time_calls(w, steps, warmup, torch, mm)}


def median(sorted_t):
    n = len(sorted_t)
    return sorted_t[n // 2] if n % 2 else 0.5 * (sorted_t[n // 2 - 1] + sorted_t[n // 2])


def mfma_ceiling(da, db, steps, warmup, torch):
    """The bf16 matrix cores alone on the workload's own operand values
    (probe/mfma_ceiling.hip): 1024 workgroups shaped like the 256 x 256 tiles
    of the 8192^3 product, each wave issuing that product's MFMAs on operands
    loaded once from A and B, no memory traffic in the loop. Timed like the
    product (HIP events on the launch stream), for both MFMA shapes and for
    all-zero operands. Returns TFLOP/s per case."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiled_matmul_relu_amd", "_build",
                        "libmfma_ceiling.so")
    lib = ctypes.CDLL(path)
    lib.mfma_ceiling_bf16.restype = ctypes.c_int
    lib.mfma_ceiling_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    tiles, slabs = 1024, 256                      # 8192^3: (32 x 32) tiles of 256 x 256, 256 slabs of 32
    flops = 2.0 * 256 * 256 * 32 * slabs * tiles
    out = torch.empty(tiles * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    za, zb = torch.zeros_like(da), torch.zeros_like(db)
    res = {}
    for name, a, b in (("workload", da, db), ("zeros", za, zb)):
        for shape in (16, 32):
            def call():
                rc = lib.mfma_ceiling_bf16(a.data_ptr(), b.data_ptr(), a.numel(), b.numel(), shape, tiles, slabs,
                                           out.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"mfma_ceiling_bf16 returned {rc}")
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            for _ in range(steps):
                call()
            end.record(stream)
            torch.cuda.synchronize()
            ms = start.elapsed_time(end) / steps
            res[f"{name}_{shape}x{shape}"] = round(flops / (ms * 1e-3) / 1e12, 1)
    return res


def per_call_stats(cfg, steps, warmup, torch, mm, datagen, variant=None, act="relu", bias=False, cold=False):
    """Per-call HIP-event times (ms) of one workload: mean, median, P95, and
    the rates derived from the median. act/bias select the fused epilogue
    (the default is relu(A·B)). With cold, the same calls are timed once more
    with a 512 MiB scratch write before each (larger than the 256 MB
    Infinity Cache and the 8 x 4 MB of L2), so every call starts with its
    operands in HBM only; the write itself is outside the events."""
    a, b = datagen.make_inputs(cfg)
    da, db = to_device(a, torch), to_device(b, torch)
    dbias = None
    if bias:
        bv = datagen.normal_f32(cfg.seed_b + 7, 1, cfg.N, 0.5).ravel()
        dbias = to_device(datagen.f32_to_bf16_bits(bv) if cfg.dtype == "bf16" else bv, torch)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    c = torch.empty((cfg.M, cfg.ldc), dtype=dt, device="cuda")
    stream = torch.cuda.current_stream()
    kind = mm.DTYPE_F32 if cfg.dtype == "f32" else mm.DTYPE_BF16
    code = {"relu": mm.ACT_RELU, "gelu_tanh": mm.ACT_GELU_TANH, "none": mm.ACT_NONE}[act]
    if variant is None:
        fn = mm.mmrelu_fused_f32 if cfg.dtype == "f32" else mm.mmrelu_fused_bf16
        args = (code,)
    else:
        fn = mm.mmrelu_fused_f32_variant if cfg.dtype == "f32" else mm.mmrelu_fused_bf16_variant
        args = (variant, code)
    args += (da.data_ptr(), db.data_ptr(), dbias.data_ptr() if dbias is not None else 0, c.data_ptr(),
             cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb, cfg.ldc, stream.cuda_stream)
    for _ in range(warmup):
        rc = fn(*args)
        if rc != mm.MMRELU_OK:
            raise RuntimeError(mm.status_string(rc))
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn(*args)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    # Back-to-back: the same calls with no event between them, so the
    # queue never waits for an event packet (the per-call times carry a
    # few microseconds of that gap, which matters for short kernels).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    b2b = e0.elapsed_time(e1) / steps
    mean = sum(t) / steps
    med = t[steps // 2] if steps % 2 else 0.5 * (t[steps // 2 - 1] + t[steps // 2])
    p95 = t[min(steps - 1, int(math.ceil(0.95 * steps)) - 1)]
    plan = (mm.mmrelu_plan(kind, cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb, cfg.ldc) if variant is None else
            mm.mmrelu_plan_variant(kind, variant, cfg.M, cfg.N, cfg.K, cfg.lda, cfg.ldb, cfg.ldc))
    alg_bytes = cfg.elem_bytes * (cfg.M * cfg.K + cfg.K * cfg.N + cfg.M * cfg.N)
    tf = cfg.flops / (med * 1e-3) / 1e12
    extra = {}
    if cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        tc = []
        for i in range(steps):
            scratch.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            tc.append(e0.elapsed_time(e1))
        del scratch
        tc.sort()
        cmed = tc[steps // 2] if steps % 2 else 0.5 * (tc[steps // 2 - 1] + tc[steps // 2])
        extra["cold_cache"] = {"what": "per call, after a 512 MiB scratch write (operands in HBM only)",
                               "mean_ms": round(sum(tc) / steps, 5), "median_ms": round(cmed, 5),
                               "p95_ms": round(tc[min(steps - 1, int(math.ceil(0.95 * steps)) - 1)], 5),
                               "tflops_median": round(cfg.flops / (cmed * 1e-3) / 1e12, 3),
                               "alg_gbs_median": round(alg_bytes / (cmed * 1e-3) / 1e9, 1)}
    return {**extra, "workload": cfg.name, "act": act, "bias": bool(bias), "M": cfg.M, "N": cfg.N, "K": cfg.K, "lda": cfg.lda, "ldb": cfg.ldb, "ldc": cfg.ldc,
            "dtype": cfg.dtype, "kernel": plan["name"], "grid": plan["grid"], "waves": plan["waves"],
            "idle_slots_last_wave": plan["idle_slots_last"], "steps": steps, "warmup": warmup,
            "mean_ms": round(mean, 5), "median_ms": round(med, 5), "p95_ms": round(p95, 5),
            "tflops_median": round(tf, 3), "pct_of_peak": round(100 * tf / PEAK_TFLOPS[cfg.dtype], 2),
            "alg_gbs_median": round(alg_bytes / (med * 1e-3) / 1e9, 1),
            "b2b_ms": round(b2b, 5), "alg_gbs_b2b": round(alg_bytes / (b2b * 1e-3) / 1e9, 1)}


LAYOUTS = {   # name: (A stored as, B stored as, C stored as); "col" = the transpose's row-major storage
    "NN": ("row", "row", "row"), "TN": ("col", "row", "row"), "NT": ("row", "col", "row"),
    "TT": ("col", "col", "row"), "TT_Ccol": ("col", "col", "col"), "NN_Ccol": ("row", "row", "col"),
}


def layout_stats(cfg, name, steps, warmup, torch, mm, datagen):
    """Per-call and back-to-back times of one workload with its operands and
    output stored in the layout `name` (general-stride entry points, the
    workspace allocated once outside the timed calls)."""
    import numpy as np
    a, b = datagen.make_inputs(cfg)
    la, lb, lc = LAYOUTS[name]
    M, N, K = cfg.M, cfg.N, cfg.K
    a = a[:, :K] if cfg.lda != K else a
    b = b[:, :N] if cfg.ldb != N else b
    if la == "col":
        da, sa = to_device(np.ascontiguousarray(a.T), torch), (1, M)
    else:
        da, sa = to_device(np.ascontiguousarray(a), torch), (K, 1)
    if lb == "col":
        db, sb = to_device(np.ascontiguousarray(b.T), torch), (1, K)
    else:
        db, sb = to_device(np.ascontiguousarray(b), torch), (N, 1)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    c = torch.empty((N, M) if lc == "col" else (M, N), dtype=dt, device="cuda")
    sc = (1, M) if lc == "col" else (N, 1)
    kind = mm.DTYPE_F32 if cfg.dtype == "f32" else mm.DTYPE_BF16
    need = mm.mmrelu_strided_workspace_size(kind, mm.ACT_RELU, da.data_ptr(), db.data_ptr(), 0, c.data_ptr(),
                                            M, N, K, *sa, *sb, *sc)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    fn = mm.mmrelu_strided_f32 if kind == mm.DTYPE_F32 else mm.mmrelu_strided_bf16
    stream = torch.cuda.current_stream()
    args = (mm.ACT_RELU, da.data_ptr(), db.data_ptr(), 0, c.data_ptr(), M, N, K, *sa, *sb, *sc,
            ws.data_ptr() if need else 0, need, stream.cuda_stream)
    for _ in range(warmup):
        rc = fn(*args)
        if rc != mm.MMRELU_OK:
            raise RuntimeError(mm.status_string(rc))
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn(*args)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    b2b = e0.elapsed_time(e1) / steps
    med = t[steps // 2]
    return {"workload": cfg.name, "layout": name, "A": la, "B": lb, "C": lc, "workspace_bytes": need,
            "median_ms": round(med, 5), "b2b_ms": round(b2b, 5),
            "tflops_b2b": round(cfg.flops / (b2b * 1e-3) / 1e12, 1)}


ROW_WORKLOADS = [   # (op, dtype, M, N)
    ("softmax", "f32", 8192, 8192), ("softmax", "bf16", 8192, 8192), ("softmax", "f32", 65536, 1024),
    ("softmax", "f32", 1024, 65536), ("row_sum", "f32", 16384, 4096), ("row_sum", "bf16", 16384, 4096),
]


def row_stats(op, dtype, M, N, steps, warmup, torch, mm, datagen):
    """Per-call and back-to-back times of the row softmax or row sum on an
    M x N matrix of N(0, 2^2) values, with algorithmic bytes (one read of X,
    plus one write of Y or of the M sums) against the HBM peak."""
    x = datagen.normal_f32(7000 + M % 97, M, N, 2.0)
    if dtype == "bf16":
        x = datagen.f32_to_bf16_bits(x)
    dx = to_device(x, torch)
    es = 4 if dtype == "f32" else 2
    stream = torch.cuda.current_stream()
    if op == "softmax":
        y = torch.empty_like(dx)
        fn = mm.mmrelu_softmax_rows_f32 if dtype == "f32" else mm.mmrelu_softmax_rows_bf16
        args = (dx.data_ptr(), y.data_ptr(), M, N, N, N, stream.cuda_stream)
        kernel = f"softmax variant {mm.mmrelu_softmax_rows_variant(mm.DTYPE_F32 if dtype == 'f32' else mm.DTYPE_BF16, N, N, N)}"
        alg = 2 * M * N * es
    else:
        y = torch.empty(M, dtype=torch.float32, device="cuda")
        fn = mm.mmrelu_row_sum_f32 if dtype == "f32" else mm.mmrelu_row_sum_bf16
        args = (dx.data_ptr(), y.data_ptr(), M, N, N, stream.cuda_stream)
        kernel = "row_sum"
        alg = M * N * es + 4 * M

    def call():
        rc = fn(*args)
        if rc != mm.MMRELU_OK:
            raise RuntimeError(mm.status_string(rc))

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return t[steps // 2], e0.elapsed_time(e1) / steps

    med, b2b = timed(call)
    r = {"op": op, "dtype": dtype, "M": M, "N": N, "kernel": kernel, "median_ms": round(med, 5),
         "b2b_ms": round(b2b, 5), "alg_bytes": alg, "alg_gbs_b2b": round(alg / (b2b * 1e-3) / 1e9, 1),
         "hbm_frac_b2b": round(alg / (b2b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if op == "softmax":                       # context: the framework's own fused softmax on the same tensor,
        t_out = torch.empty_like(dx)          # and a plain copy (one read, one write: the same bytes)
        _, tb = timed(lambda: torch.softmax(dx, dim=1, out=t_out))
        r["torch_softmax_b2b_ms"] = round(tb, 5)
        _, cb = timed(lambda: t_out.copy_(dx))
        r["copy_b2b_ms"] = round(cb, 5)
    return r


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, a, b, target_s, oracle):
    """The oracle timed on rows [0, r) of the workload, r chosen so that the
    timed part takes about target_s seconds: a calibration run on a few rows
    per thread, one correction if the timed run came out under half the
    target, and whole-matrix repeats if even all rows take under 10 s.
    Returns the baseline record and the oracle's rows [0, r) from the last
    run (fp64), which the caller compares with the timed output."""
    def run(rows):
        t0 = time.perf_counter()
        r = oracle.mmrelu(a, b, M=rows, N=cfg.N, K=cfg.K, lda=cfg.lda, ldb=cfg.ldb)
        return time.perf_counter() - t0, r
    clamp = lambda r: int(min(cfg.M, max(1, r)))
    cal_rows = clamp(max(64, 4 * oracle.num_threads()))
    t_cal, _ = run(cal_rows)
    rows = clamp(target_s / max(t_cal, 1e-6) * cal_rows)
    t, ref = run(rows)
    if t < 0.5 * target_s and rows < cfg.M:
        rows = clamp(rows * target_s / max(t, 1e-6))
        del ref
        t, ref = run(rows)
    reps = 1
    if rows == cfg.M and t < 10.0:
        reps = max(1, math.ceil(10.0 / max(t, 1e-6)))
        for _ in range(reps - 1):
            del ref
            dt, ref = run(rows)
            t += dt
    flops = 2.0 * rows * cfg.N * cfg.K * reps
    what = f"rows 0..{rows - 1} of {cfg.M}" if rows < cfg.M else f"all {cfg.M} rows"
    times = f", computed {reps} times" if reps > 1 else ""
    rec = {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "cpu_model": cpu_model(), "kind": "oracle",
           "sample": f"{what} of the {cfg.name} workload ({rows}x{cfg.N} outputs, K={cfg.K}){times}, fp64 oracle, "
                     f"{t:.1f} s in all"}
    return rec, ref


def parity_of(cfg, c_dev, ref, datagen):
    """The timed output against the oracle's rows [0, r): fp32 max |C - R|
    against 1e-4 sqrt(K); bf16 ||C - R||_F / ||R||_F against 1e-2, and the
    largest element error over its bound 2^-8 |R| + 1e-6."""
    import numpy as np
    rows = ref.shape[0]
    c = c_dev[:rows, :cfg.N]
    if cfg.dtype == "bf16":
        import torch
        c = datagen.bf16_bits_to_f32(c.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    else:
        c = c.cpu().numpy().astype(np.float64)
    out = {"rows_compared": f"0..{rows - 1} of {cfg.M}", "elements": int(c.size),
           "finite": bool(np.isfinite(c).all())}
    d = np.abs(c - ref)
    if cfg.dtype == "f32":
        tol = 1e-4 * math.sqrt(cfg.K)
        out.update({"metric": "max |C - R|", "value": float(d.max()), "tol": tol,
                    "pass": bool(out["finite"] and d.max() <= tol)})
    else:
        rel = float(np.linalg.norm(c - ref) / np.linalg.norm(ref))
        worst = float((d / (2.0 ** -8 * np.abs(ref) + 1e-6)).max())
        out.update({"metric": "||C - R||_F / ||R||_F", "value": rel, "tol": 1e-2,
                    "max_elem_err_over_bound": round(worst, 4),
                    "pass": bool(out["finite"] and rel <= 1e-2 and worst <= 1.0)})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # The first ~25 calls of a fresh process run while clocks and power
    # management settle (up to 30% slower); the defaults time the sustained rate.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle timing")
    ap.add_argument("--no-f32", action="store_true", help="skip the fp32 4096^3 workload")
    ap.add_argument("--no-power-check", action="store_true",
                    help="skip the power-cap checks: the bf16 kernel on all-zero inputs, and the matrix cores alone "
                         "on the workload's values (the MFMA ceiling probe)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a kernel of known traffic, "
                         "for scaling memory counters)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: write profiles/traffic.json from the counter_collection.csv files of "
                         "two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script with --calib-copy-mib")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the benchmark line: per-call statistics (mean, median, P95, algorithmic GB/s, "
                         "grid and wave quantization) of all five workloads, one JSON line each")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line: square sizes 256..8192 and skinny shapes (M or N of "
                         "1..64, the others 8192) in both dtypes, per-call statistics with the bounding roofline "
                         "(MFMA or HBM) and the fraction of it reached, one JSON line each")
    ap.add_argument("--layouts", action="store_true",
                    help="instead of the benchmark line: the bf16 8192^3 and fp32 4096^3 workloads with A, B and C "
                         "stored row- or column-major (NN, TN, NT, TT, TT into a column-major C, NN into a "
                         "column-major C) through the general-stride entry points, one JSON line each")
    ap.add_argument("--rows", action="store_true",
                    help="instead of the benchmark line: the row softmax and row sum (the rungs before the matmul) "
                         "on 8192 x 8192, 65536 x 1024, 1024 x 65536 and 16384 x 4096 matrices, algorithmic GB/s "
                         "against the HBM peak, one JSON line each")
    ap.add_argument("--shapes", default="",
                    help="with --sweep: only these shapes, comma-separated dtype:MxNxK (e.g. f32:1x8192x8192)")
    ap.add_argument("--sweep-steps", type=int, default=0,
                    help="with --sweep: timed calls per shape (default 100, 40 above 2e11 FLOPs)")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: calibrated HBM bytes per dispatch of each mmrelu kernel in the "
                         "counter_collection.csv files of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of a "
                         "command run with --calib-copy-mib, one JSON line each")
    ap.add_argument("--act", choices=["relu", "gelu_tanh", "none"], default="relu",
                    help="with --all-configs: the fused epilogue's activation")
    ap.add_argument("--bias", action="store_true", help="with --all-configs: add a per-column bias")
    ap.add_argument("--cold-cache", action="store_true",
                    help="with --all-configs: also time each call after a 512 MiB scratch write (cold L2 and "
                         "Infinity Cache)")
    ap.add_argument("--traffic-command", default="", help="the profiling command, stored with --record-traffic")
    args = ap.parse_args()

    if args.all_configs:
        import torch
        import datagen
        import tiled_matmul_relu_amd as mm
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(1)
        mm.load_library()
        for ident, cfg in sorted(datagen.CONFIGS.items()):
            print(json.dumps({"config": ident, **per_call_stats(cfg, args.steps, args.warmup, torch, mm, datagen,
                                                                act=args.act, bias=args.bias,
                                                                cold=args.cold_cache)}), flush=True)
        return

    if args.sweep:
        import torch
        import datagen
        import tiled_matmul_relu_amd as mm
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(1)
        mm.load_library()
        if args.calib_copy_mib > 0:
            calib_copy(args.calib_copy_mib, torch)
        todo = []
        for dtype in ("f32", "bf16"):
            shapes = [(n, n, n) for n in (256, 512, 1024, 2048, 4096, 8192)]
            shapes += [(m, 8192, 8192) for m in (1, 8, 16, 32, 64)] + [(8192, n, 8192) for n in (1, 16, 64)]
            shapes += [(1, 16384, 16384), (4, 32768, 4096)]     # few rows, many columns
            # between skinny and square: few output tiles, long K; and the
            # ragged shape (odd leading dimensions)
            shapes += [(128, 8192, 8192), (256, 4096, 4096), (512, 512, 8192), (1024, 1024, 8192), (4097, 3001, 2049)]
            # one GPU's share of an 8-way split of C by rows: 4096^3 fp32, 8192^3 bf16
            shapes += [(512, 4096, 4096) if dtype == "f32" else (1024, 8192, 8192)]
            todo += [(dtype, s) for s in shapes]
        if args.shapes:
            todo = []
            for item in args.shapes.split(","):
                dtype, dims = item.split(":")
                todo.append((dtype, tuple(int(x) for x in dims.split("x"))))
        for dtype, (M, N, K) in todo:
            cfg = datagen.Config(0, f"{dtype}_{M}x{N}x{K}", dtype, M, N, K, K, N, N, "normal_over_sqrtk")
            steps = args.sweep_steps or (40 if cfg.flops > 2e11 else 100)
            r = per_call_stats(cfg, steps, 20, torch, mm, datagen)
            peak = PEAK_TFLOPS[dtype]
            t_mfma = cfg.flops / (peak * 1e12) * 1e3
            t_hbm = cfg.elem_bytes * (M * K + K * N + M * N) / (HBM_PEAK_GBS * 1e9) * 1e3
            r["bound"] = "mfma" if t_mfma >= t_hbm else "hbm"
            r["roofline_frac"] = round(max(t_mfma, t_hbm) / r["median_ms"], 4)
            r["pct_of_hbm_peak"] = round(100 * r["alg_gbs_median"] / HBM_PEAK_GBS, 2)
            r["roofline_frac_b2b"] = round(max(t_mfma, t_hbm) / r["b2b_ms"], 4)
            print(json.dumps(r), flush=True)
        return

    if args.layouts:
        import torch
        import datagen
        import tiled_matmul_relu_amd as mm
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(1)
        mm.load_library()
        for cid in (5, 3):
            cfg = datagen.CONFIGS[cid]
            base = None
            for name in LAYOUTS:
                r = layout_stats(cfg, name, args.sweep_steps or 40, 10, torch, mm, datagen)
                base = base or r["b2b_ms"]
                r["vs_NN"] = round(r["b2b_ms"] / base, 4)
                print(json.dumps(r), flush=True)
        return

    if args.rows:
        import torch
        import datagen
        import tiled_matmul_relu_amd as mm
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(1)
        mm.load_library()
        if args.calib_copy_mib > 0:
            calib_copy(args.calib_copy_mib, torch)
        for op, dtype, M, N in ROW_WORKLOADS:
            print(json.dumps(row_stats(op, dtype, M, N, args.sweep_steps or 50, 10, torch, mm, datagen)), flush=True)
        return

    if args.counter_summary:
        if args.calib_copy_mib <= 0:
            ap.error("--counter-summary needs --calib-copy-mib (the size the profiled runs copied)")
        counter_summary(args.counter_summary[0], args.counter_summary[1], args.calib_copy_mib)
        return

    if args.record_traffic:
        if args.calib_copy_mib <= 0:
            ap.error("--record-traffic needs --calib-copy-mib (the size the profiled runs copied)")
        record_traffic(args.record_traffic[0], args.record_traffic[1], args.calib_copy_mib, args.traffic_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; relu(A·B) shards by rows or columns of C with no "
              "exchange, and no multi-GPU path is built. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import datagen
    import tiled_matmul_relu_amd as mm

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    mm.load_library()

    head = datagen.CONFIGS[5]
    res = prepare_workload(head, torch, mm, datagen)
    # The first calls of a process run while the board's power management
    # settles: after a few fast calls it cuts the clock hard and then
    # releases it over ~25 calls of this kernel (per-call trace 750, 745,
    # 812, 941, 1040, 984, 913, ... 760, 748 us). The same W + K calls are
    # therefore run and timed twice, back to back: first at the process's
    # cold start (reported as cold_start), then again for `value`, the
    # steady state that a job issuing this call repeatedly runs in.
    cold = time_calls(res, args.steps, args.warmup, torch, mm)
    res.update(time_calls(res, args.steps, args.warmup, torch, mm))
    kernel = res["plan"]["name"]
    achieved = res["tflops"]
    traffic = measured_traffic("bf16", kernel)
    out = {
        "metric": "TFLOP/s and % of MI355X MFMA peak for relu(A·B), fp32 4096³ and bf16 8192³",
        "value": round(achieved, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(K) rounded to bf16, resident in HBM)",
        "config": {"workload": "relu(A·B) bf16 in/out, fp32 accumulate, M=N=K=8192, row-major",
                   "M": head.M, "N": head.N, "K": head.K, "lda": head.lda, "ldb": head.ldb, "ldc": head.ldc,
                   "kernel": kernel, "grid": res["plan"]["grid"]},
        "pct_of_peak": round(100 * achieved / PEAK_TFLOPS["bf16"], 2),
        "per_call": res["per_call"],
        "cold_start": {"what": "the same W warm-up and K timed calls at the start of the process, timed the same "
                               "way, before the ones above",
                       "ms_per_step": round(cold["ms"], 4), "value": round(cold["tflops"], 2), "unit": "TFLOP/s",
                       "frac": round(cold["tflops"] / PEAK_TFLOPS["bf16"], 4), "per_call": cold["per_call"]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": traffic},
    }
    if not args.no_power_check:
        # The matrix cores alone on the same operand values: the most any
        # kernel of this product can reach on these inputs under the power
        # cap. Run right after the product, whose power draw it matches, so
        # that it starts in the same settled state.
        mc = mfma_ceiling(res["da"], res["db"], args.steps, args.warmup, torch)
        out["mfma_ceiling"] = {"what": "bf16 MFMAs alone (no memory traffic), the product's per-wave MFMA "
                                       "block on operands loaded from A and B; TFLOP/s per MFMA shape",
                               "unit": "TFLOP/s", **mc,
                               "value_frac_of_ceiling": round(achieved / mc["workload_16x16"], 4)}
        # Same kernel, same shape, all-zero inputs: the matrix cores see no
        # operand toggling, so the board's power cap does not lower the clock.
        # The gap to `value` is the power cost of random operands, not schedule.
        zero = dataclasses.replace(head, name=head.name + "_zeros", dist="zeros")
        rz = time_workload(zero, args.steps, args.warmup, torch, mm, datagen)
        out["power_check"] = {"inputs": "all-zero bf16 A and B, same shape, kernel and launch",
                              "value": round(rz["tflops"], 2), "unit": "TFLOP/s", "ms_per_step": round(rz["ms"], 4),
                              "frac": round(rz["tflops"] / PEAK_TFLOPS["bf16"], 4)}
        del rz
    r32 = None
    if not args.no_f32:
        f = datagen.CONFIGS[3]
        r32 = time_workload(f, args.steps, args.warmup, torch, mm, datagen)
        out["fp32_4096"] = {"value": round(r32["tflops"], 2), "unit": "TFLOP/s", "ms_per_step": round(r32["ms"], 4),
                            "frac": round(r32["tflops"] / PEAK_TFLOPS["f32"], 4), "peak": PEAK_TFLOPS["f32"],
                            "kernel": r32["plan"]["name"], "per_call": r32["per_call"],
                            "traffic": measured_traffic("f32", r32["plan"]["name"])}
    if args.calib_copy_mib > 0:
        out["calib_copy_bytes"] = calib_copy(args.calib_copy_mib, torch)
    if not args.no_cpu_baseline:
        # The oracle on this host's cores: timed as the CPU baseline, and its
        # result compared with the output of the timed calls.
        import oracle
        a, b = res["inputs"]
        out["cpu_baseline"], ref = cpu_baseline(head, a, b, args.cpu_seconds, oracle)
        out["parity"] = parity_of(head, res["c"], ref, datagen)
        del ref
        if r32 is not None:
            # fp32: the first rows of its output, about two seconds of oracle work
            a32, b32 = r32["inputs"]
            t0 = time.perf_counter()
            probe = oracle.mmrelu(a32, b32, M=64, N=f.N, K=f.K, lda=f.lda, ldb=f.ldb)
            rows = int(min(f.M, max(64, 64 * 2.0 / max(time.perf_counter() - t0, 1e-6))))
            ref32 = probe if rows == 64 else oracle.mmrelu(a32, b32, M=rows, N=f.N, K=f.K, lda=f.lda, ldb=f.ldb)
            out["fp32_4096"]["parity"] = parity_of(f, r32["c"], ref32, datagen)
    else:
        out["cpu_baseline"] = None
        out["parity"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
