"""Benchmark: VCS SpMM on the 60,000 x 2,000 count matrix (~6M nonzeros) at
width 16, all four directions, on one MI355X.

A step is one pass of the product path over that matrix in all four
directions: VCSR @ B and B @ VCSC (aligned walks), B @ VCSR and VCSC @ B
(misaligned). The headline runs each direction the fastest deterministic way
the library offers, with each deterministic direction's schedule built for
width 16 (vspmm_schedule_create; the one-time builds and the schedules'
resident bytes are reported separately):
VCSR @ B as the plain aligned walk (B fits in LDS), VCSC @ B as the walk over
the regrouped layout, and B @ VCSR and B @ VCSC over the tiled copy of the
matrix (B's 60,000 rows cut into tiles that fit in LDS). Atomic mode, whose
misaligned products are bound by the GPU's float-atomic request rate, is
timed and reported in the same line.

Inputs are resident in HBM before timing starts. Every product reads its own
copy of the matrix and dense operands, and the copies rotate through more than
1 GB, so no product finds its data in the 256 MB Infinity Cache (cold-HBM
numbers). Each direction's launches run back to back between two HIP events
on the stream the library launches on; its average launch duration is the
elapsed time over the launch count.

Minimum algorithmic bytes of one product = the compressed structure the
product walks (4(n_major+1) + 4 G + 4(G+1) + 4 nnz) + 4 w (n_in + n_out).
value = the four products' minimum bytes / the sum of their average times.

roofline.traffic is the HBM bytes per launch of the dominant kernel, from two
rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of this script, each scaled
by what the same counter reads for a plain device copy of known size
(--copy-calibration). The figures sit in a record under profiles/ keyed by a
hash of the kernel sources; when the sources have changed since, traffic is
null. roofline.secondary is the walk's measured secondary ceiling from the
same kind of record (SQ counters: instructions per entry, VALU busy fraction):
the walk is bound by instruction issue and latency, not by HBM.

Prints ONE JSON line. --gpus above 1 is refused: the benchmark measures one GPU.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HBM GB/s (% of peak) for VCS SpMM 60k×2k, 6M nnz, width 16, 4 directions"
PEAK_GBPS = 8000.0  # MI355X HBM3E

CSRC = os.path.join(ROOT, "sparse_dense_matmul_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# name, layout of the handle, direction, walk used in atomic mode
DIRECTIONS = [
    ("VCSR@B", "vcsr", "AB", "aligned"),
    ("B@VCSR", "vcsr", "BA", "scatter"),
    ("VCSC@B", "vcsc", "AB", "scatter"),
    ("B@VCSC", "vcsc", "BA", "aligned"),
]


def dense_bytes(shape, direction, w):
    m, n = shape
    n_in, n_out = (n, m) if direction == "AB" else (m, n)
    return 4 * w * (n_in + n_out)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256 over the kernel sources (every file under csrc/, by name)."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_record(kernel, direction, width):
    """HBM bytes per launch from the counter record in profiles/, when its
    source hash matches the sources built now; else None."""
    want = kernel_source_hash()
    pat = re.compile(r"^traffic-record:\s*(.*)$")
    for f in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        for line in open(f):
            m = pat.match(line.strip())
            if not m:
                continue
            kv = dict(tok.split("=", 1) for tok in m.group(1).split())
            if (kv.get("kernel") == kernel.replace(" ", "") and kv.get("direction") == direction and
                    int(kv.get("width", -1)) == width and kv.get("source_sha256") == want):
                return int(kv["hbm_bytes"]), os.path.relpath(f, ROOT)
    return None, None


def ceiling_record(kernel):
    """The walk's measured secondary ceiling from the counter record in
    profiles/ (instruction counts per entry and how busy the VALU is), when its
    source hash matches the sources built now; else None."""
    want = kernel_source_hash()
    pat = re.compile(r"^ceiling-record:\s*(.*)$")
    for f in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        for line in open(f):
            m = pat.match(line.strip())
            if not m:
                continue
            kv = dict(tok.split("=", 1) for tok in m.group(1).split())
            if kv.get("kernel") == kernel and kv.get("source_sha256") == want:
                out = {k: float(v) for k, v in kv.items()
                       if k not in ("kernel", "source_sha256", "bound")}
                out["bound"] = kv.get("bound")
                out["source"] = os.path.relpath(f, ROOT)
                return out
    return None


def probe_record():
    """The measured secondary ceilings (LDS and L2 row gathers, global and LDS
    float atomics, empty launches) from the probe record in profiles/, when
    the probe source hashes to the value recorded; else None."""
    h = hashlib.sha256(open(os.path.join(CSRC, "probe.hip"), "rb").read()).hexdigest()
    pat = re.compile(r"^probe-ceilings:\s*(.*)$")
    for f in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        for line in open(f):
            m = pat.match(line.strip())
            if not m:
                continue
            kv = dict(tok.split("=", 1) for tok in m.group(1).split())
            if kv.get("source_sha256") == h:
                out = {k: float(v) for k, v in kv.items() if k != "source_sha256"}
                out["source"] = os.path.relpath(f, ROOT)
                return out
    return None


def copy_calibration(mib):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


def ceilings(reps=20):
    """Measured ceilings of the resources the walks use besides HBM (the
    probe kernels of libvspmm_probe.so, shaped like the aligned walk's inner
    loop): 64-byte row gathers from LDS and from global memory (L2), global
    and LDS float atomics as a width-16 scatter issues them, and back-to-back
    empty launches. Rates are per chip; 'us_per_6M' is the time 6,000,000 such
    rows (or 6M entries' adds at width 16) take at that rate."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_dense_matmul_amd", "libvspmm_probe.so"))
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.vspmm_probe.argtypes = [ci, ci, vp, ci, vp, ci, ci, ci, vp, vp, ci, vp,
                                ctypes.POINTER(ctypes.c_float)]
    lib.vspmm_probe.restype = ci
    dev = torch.device("cuda:0")
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    clk_ghz = 2.4
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rng = np.random.default_rng(5)
    grid = n_cu
    n_win = 4096
    sink = torch.empty(grid * 1024, dtype=torch.float32, device=dev)

    def run(kind, mode, n_rows, iters, table=None, out=None, g=grid):
        idx = torch.from_numpy(rng.integers(0, n_rows, size=n_win * 64).astype(np.int32)).to(dev)
        ms = ctypes.c_float(0)
        st = lib.vspmm_probe(kind, mode, vp(table.data_ptr()) if table is not None else None,
                             n_rows, vp(idx.data_ptr()), n_win, iters, g, vp(sink.data_ptr()),
                             vp(out.data_ptr()) if out is not None else None, reps, stream,
                             ctypes.byref(ms))
        if st != 0:
            raise RuntimeError(f"vspmm_probe(kind={kind}, mode={mode}) failed: {st}")
        return ms.value / reps  # ms per launch

    res = {}
    iters = 512
    rows_per_launch = grid * 16 * iters * 4 * 16  # 16 rows per step per wave
    table = torch.randn(2000 * 16, device=dev)
    for mode, name in ((0, "lds_gather_b128_random_rows"), (1, "lds_gather_b128_conflict_free"),
                       (2, "lds_gather_2xb64_random_rows")):
        ms = run(0, mode, 2000, iters, table=table)
        rate = rows_per_launch / (ms * 1e-3)
        res[name] = {"G_rows_per_s": round(rate / 1e9, 2),
                     "bytes_per_clk_per_CU": round(rate * 64 / (clk_ghz * 1e9 * n_cu), 1),
                     "us_per_6M": round(6e6 / rate * 1e6, 2)}
    for n_rows, name in ((2000, "l2_gather_128KB_table"), (60000, "l2_gather_3.84MB_table")):
        tab = torch.randn(n_rows * 16, device=dev)
        ms = run(1, 0, n_rows, iters // 4, table=tab)
        rate = rows_per_launch / 4 / (ms * 1e-3)
        res[name] = {"G_rows_per_s": round(rate / 1e9, 2), "us_per_6M": round(6e6 / rate * 1e6, 2)}
    for n_rows, name in ((2000, "atomic_f32_w16_128KB_out"), (60000, "atomic_f32_w16_3.84MB_out")):
        out = torch.zeros(n_rows * 16, device=dev)
        it_a = 16
        ms = run(2, 0, n_rows, it_a, out=out)
        entries = grid * 16 * it_a * 64  # 64 entries (rows of 16 adds) per window
        rate = entries / (ms * 1e-3)
        res[name] = {"G_entries_per_s": round(rate / 1e9, 3),
                     "G_instr_per_s": round(rate / 4 / 1e9, 3),
                     "us_per_6M": round(6e6 / rate * 1e6, 1)}
    it_a = 16
    ms = run(4, 0, 2000, it_a)
    rate = grid * 16 * it_a * 64 / (ms * 1e-3)
    res["lds_atomic_f32_w16_128KB_copy"] = {
        "G_entries_per_s": round(rate / 1e9, 3),
        "lanes_per_clk_per_CU": round(rate * 16 / (clk_ghz * 1e9 * n_cu), 3),
        "us_per_6M": round(6e6 / rate * 1e6, 1)}
    res["empty_launch_us"] = round(1e3 * run(3, 0, 1, 0, g=1024), 2)
    return {"device_cus": n_cu, "clock_ghz_assumed": clk_ghz, "grid": grid,
            "threads_per_block": 1024, "reps": reps, "ceilings": res}


def cpu_threads():
    """Host threads for the oracle's timed mode: OMP_NUM_THREADS when set (the
    share of the host's cores a job is given), else every core the process
    may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "").strip()
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(layouts, width, budget_s):
    """The float64 oracle, as it is, on the host: its threaded mode (slices
    split over the host threads, private float64 outputs where the output rows
    are not the slices) over the four directions of the full matrix. One
    warm-up pass, then passes until about budget_s seconds (at least 5); the
    value is the bytes of a pass over the median pass time. A single-threaded
    pass of the sequential oracle is timed too."""
    import oracle

    rng = np.random.default_rng(1)
    threads = cpu_threads()
    ops = []
    for name, layout, direction, _ in DIRECTIONS:
        L = layouts[layout]
        m, n = L.shape
        B = rng.standard_normal((n if direction == "AB" else m, width)).astype(np.float32)
        ops.append((L, direction, B.astype(np.float64)))
    pass_bytes = sum(L.nbytes() + dense_bytes(L.shape, d, width) for L, d, _ in ops)

    def one_pass(fn):
        t0 = time.perf_counter()
        for L, d, B in ops:
            fn(L, d, B)
        return time.perf_counter() - t0

    threaded = lambda L, d, B: oracle.spmm_threaded(L, d, B, threads)
    one_pass(threaded)  # warm-up
    times, spent = [], 0.0
    while len(times) < 5 or spent < budget_s:
        times.append(one_pass(threaded))
        spent += times[-1]
        if len(times) >= 200:
            break
    med = float(np.median(times))
    single = one_pass(lambda L, d, B: oracle.spmm(L, d, B))
    return {"value": round(pass_bytes / med / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "host_cpu_count": os.cpu_count(),
            "single_thread_GBps": round(pass_bytes / single / 1e9, 4),
            "sample": f"median of {len(times)} passes (after one warm-up) of the four directions "
                      f"over the full 60k x 2k matrix at width {width}, float64 C oracle, threaded "
                      f"mode on {threads} threads (host reports {os.cpu_count()} CPUs); "
                      f"{spent:.1f} s timed; one sequential pass took {single:.2f} s"}


def csr64_products(dev, steps):
    """A CSR past 2^31 entries (int64 row pointers, int32 column indices),
    reported beside the headline: 2^21 rows of 1,025 entries (2,149,580,800)
    over 4,096 columns, indices uniform and values U(0,1) drawn on the device
    (seeded). A @ x and x @ A (atomic, and deterministic with the blocks'
    transposes built) at width 1, float32 sums and float32 values summed in
    float64. The matrix (17.2 GB) is far larger than every cache, so each
    product reads it from HBM. Algorithmic bytes: 8(m+1) + 8 nnz + s (n_in +
    n_out), s = 4 or 8."""
    import torch

    import sparse_dense_matmul_amd as sdm

    n_rows, L, n_cols = 2**21, 1025, 4096
    nnz = n_rows * L
    g = torch.Generator(device=dev)
    g.manual_seed(20261202)
    col = torch.empty(nnz, dtype=torch.int32, device=dev)
    val = torch.empty(nnz, dtype=torch.float32, device=dev)
    chunk = 2**28
    for s0 in range(0, nnz, chunk):
        e0 = min(nnz, s0 + chunk)
        col[s0:e0] = torch.randint(0, n_cols, (e0 - s0,), generator=g, device=dev,
                                   dtype=torch.int32)
        val[s0:e0] = torch.rand(e0 - s0, generator=g, device=dev)
    row_ptr = torch.arange(n_rows + 1, dtype=torch.int64, device=dev) * L
    stream = torch.cuda.current_stream(dev)
    out = {}
    steps = max(2, min(steps, 10))
    for tdt, tname in ((torch.float32, "f32"), (torch.float64, "f32 values, f64 sums")):
        A = sdm.CsrMatrix.from_arrays((n_rows, n_cols), row_ptr, col, val, dtype=tdt)
        s = 4 if tdt == torch.float32 else 8
        for direction in ("AB", "BA"):
            n_in, n_out = (n_cols, n_rows) if direction == "AB" else (n_rows, n_cols)
            B = torch.rand(n_in, 1, generator=g, device=dev, dtype=tdt)
            O = torch.empty(n_out, 1, dtype=tdt, device=dev)
            for mode in (["atomic"] if direction == "AB" else ["atomic", "deterministic"]):
                sc = None
                t0 = time.perf_counter()
                if mode == "deterministic":
                    sc = A.schedule(direction, 1)  # the blocks' transposes
                    run = lambda: sc.spmm(B, out=O)
                else:
                    run = lambda: A.spmm(B, direction, mode=mode, out=O)
                run()
                torch.cuda.synchronize()
                first_ms = 1e3 * (time.perf_counter() - t0)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(steps):
                    run()
                b.record(stream)
                torch.cuda.synchronize()
                us = 1e3 * a.elapsed_time(b) / steps
                nbytes = 8 * (n_rows + 1) + 8 * nnz + s * (n_in + n_out)
                key = f"{tname} w=1 {'A@x' if direction == 'AB' else 'x@A'}" + \
                      ("" if direction == "AB" else f" {mode}")
                out[key] = {"us": round(us, 1), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
                if mode == "deterministic":
                    out[key]["schedule_build_plus_first_ms"] = round(first_ms, 1)
                    out[key]["schedule_bytes"] = sc.nbytes
                del sc
        del A
    del col, val, row_ptr
    torch.cuda.empty_cache()
    return {"workload": f"CSR {n_rows} x {n_cols}, {nnz} entries (int64 row pointers, "
                        "3 row blocks), width 1", "products": out}


def csr_products(dev, steps, copies=8):
    """The CSR rows of the path, reported beside the headline (not in it): the
    regridding-shaped operator (20,000 x ~373,500, ~1.1M weights) in float32
    and float64, forward (A @ x) and backprojection (x @ A, misaligned: atomic,
    and deterministic on the built transpose), at widths 1 and 32. Algorithmic
    bytes: 4(m+1) + (4+s) nnz + s w (n_in + n_out), s = 4 or 8."""
    import torch

    import sparse_dense_matmul_amd as sdm
    import workloads as W

    out = {}
    stream = torch.cuda.current_stream(dev)
    # (value type, dense type): float32 values summed in float64 as a third case
    for np_t, d_t, tname in ((np.float32, np.float32, "f32"), (np.float64, np.float64, "f64"),
                             (np.float32, np.float64, "f32 values, f64 sums")):
        _, C = W.config4(np_t)
        m, n = C.shape
        s = np.dtype(d_t).itemsize
        sv = np.dtype(np_t).itemsize
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        tdt = torch.float64 if d_t == np.float64 else torch.float32
        hs = [sdm.CsrMatrix.from_arrays(C.shape, up(C.row_ptr), up(C.col), up(C.val), dtype=tdt)
              for _ in range(copies)]
        for w in (1, 32):
            for direction in ("AB", "BA"):
                n_in, n_out = (n, m) if direction == "AB" else (m, n)
                Bs = [up(np.random.default_rng(k).standard_normal((n_in, w)).astype(d_t))
                      for k in range(copies)]
                Os = [torch.empty((n_out, w), dtype=Bs[0].dtype, device=dev) for _ in range(copies)]
                modes = ["atomic"] if direction == "AB" else ["atomic", "deterministic"]
                for mode in modes:
                    if mode == "deterministic":  # the transposes, built once
                        scs = [h.schedule(direction, w) for h in hs]
                        run = lambda k: scs[k % copies].spmm(Bs[k % copies], out=Os[k % copies])
                    else:
                        scs = None
                        run = lambda k: hs[k % copies].spmm(Bs[k % copies], direction, mode=mode,
                                                            out=Os[k % copies])
                    for k in range(copies):
                        run(k)  # warm-up
                    torch.cuda.synchronize()
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for k in range(steps):
                        run(k)
                    b.record(stream)
                    torch.cuda.synchronize()
                    us = 1e3 * a.elapsed_time(b) / steps
                    nbytes = 4 * (m + 1) + (4 + sv) * C.nnz + s * w * (n_in + n_out)
                    key = f"{tname} w={w} {'A@x' if direction == 'AB' else 'x@A'}" + \
                          ("" if direction == "AB" else f" {mode}")
                    out[key] = {"us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                                "kernel": hs[0].plan_info(w, direction, mode)["kernel_name"]}
                    if scs:
                        out[key]["schedule_bytes"] = scs[0].nbytes
                    del scs
        # the exact transpose on the device (vspmm_transpose_csr), once per copy
        h0 = hs[0]
        ws = h0.workspace("BA")
        t_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
        t_col = torch.empty(C.nnz, dtype=torch.int32, device=dev)
        t_val = torch.empty(C.nnz, dtype=hs[0].val.dtype, device=dev)
        ts = []
        for k in range(copies):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            st = sdm.lib.vspmm_transpose_csr(hs[k]._h, t_ptr.data_ptr(), t_col.data_ptr(),
                                             t_val.data_ptr(), ws.data_ptr(), ws.numel(),
                                             sdm._stream(dev))
            b.record(stream)
            torch.cuda.synchronize()
            if st != 0:
                raise RuntimeError(f"vspmm_transpose_csr failed with status {st}")
            ts.append(a.elapsed_time(b))
        out[f"{tname} transpose"] = {"us": round(1e3 * float(np.median(ts)), 1),
                                     "kernel": "index keys + radix sort + bin starts + emit"}
        del hs, ws
    return {"workload": "CSR regridding operator 20,000 x ~373,500, ~1.1M weights "
                        "(log-normal rows), U(0,1) values; cold copies rotated", "products": out}


def expansions(layouts, dev, steps, copies=8):
    """VCS -> one value per entry on the device (vspmm_expand_vcs), beside the
    headline: the 60k matrix from either layout into CSR or CSC, index-sorted
    or in stored order, cold copies rotated. Bytes: the VCS read once plus
    the expansion written, 4(n_major + 1) + 4 G_k + 4(G_k + 1) + 4 nnz
    + 4(n_out_major + 1) + 8 nnz."""
    import torch

    import sparse_dense_matmul_amd as sdm

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    out = {}
    stream = torch.cuda.current_stream(dev)
    for lay, L in layouts.items():
        hs = [sdm.VcsMatrix.from_arrays(lay, L.shape, *[up(a) for a in (L.major_ptr, L.values,
                                                                       L.value_ptr, L.indices)])
              for _ in range(copies)]
        wss = [h.workspace("BA" if lay == "vcsr" else "AB") for h in hs]
        m, n = L.shape
        for fmt in ("csr", "csc"):
            for sort in (True, False):
                own = (fmt == "csr") == (lay == "vcsr")
                if not own and not sort:
                    continue  # the other format is always index-sorted
                run = lambda k: hs[k % copies].expand(fmt, sort, workspace=wss[k % copies])
                for k in range(copies):
                    run(k)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for k in range(steps):
                    run(k)
                b.record(stream)
                torch.cuda.synchronize()
                us = 1e3 * a.elapsed_time(b) / steps
                nb = L.nbytes() + 4 * ((m if fmt == "csr" else n) + 1) + 8 * L.nnz
                key = f"{lay} -> {fmt}" + ("" if not own else (" sorted" if sort else " stored order"))
                out[key] = {"us": round(us, 1), "GBps": round(nb / (us * 1e-6) / 1e9, 1)}
        del hs, wss
    return {"workload": "the 60k x 2k count matrix, 6,001,332 entries; outputs from torch's "
                        "caching allocator (no device work), workspace given", "products": out}


def time_launches(run, steps, stream):
    """Average microseconds of run() over `steps` back-to-back launches
    between two events (after one untimed call)."""
    import torch
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for k in range(steps):
        run(k)
    b.record(stream)
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / steps


def csr_small_products(dev, steps, copies=16):
    """The 2,000 x 500 CSR (Poisson(10) entries per row, U(0,1) values,
    float32): A @ B and B @ A at width 8, and SpMV (width 1) both ways; B @ A
    atomic and deterministic (through a schedule). Cold copies rotated.
    Algorithmic bytes: 4(m+1) + 8 nnz + 4 w (n_in + n_out)."""
    import torch

    import sparse_dense_matmul_amd as sdm
    import workloads as W

    _, C = W.config1()
    m, n = C.shape
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    hs = [sdm.CsrMatrix.from_arrays(C.shape, up(C.row_ptr), up(C.col), up(C.val))
          for _ in range(copies)]
    stream = torch.cuda.current_stream(dev)
    out = {}
    for w in (1, 8):
        for direction in ("AB", "BA"):
            n_in, n_out = (n, m) if direction == "AB" else (m, n)
            rng = np.random.default_rng(w)
            Bs = [up(rng.standard_normal((n_in, w)).astype(np.float32)) for _ in range(copies)]
            Os = [torch.empty((n_out, w), device=dev) for _ in range(copies)]
            for mode in (["atomic"] if direction == "AB" else ["atomic", "deterministic"]):
                if mode == "deterministic":
                    scs = [h.schedule(direction, w) for h in hs]
                    run = lambda k=0: scs[k % copies].spmm(Bs[k % copies], out=Os[k % copies])
                else:
                    run = lambda k=0: hs[k % copies].spmm(Bs[k % copies], direction,
                                                          out=Os[k % copies])
                us = time_launches(run, steps, stream)
                nb = 4 * (m + 1) + 8 * C.nnz + 4 * w * (n_in + n_out)
                key = f"w={w} {'A@B' if direction == 'AB' else 'B@A'}" + \
                      ("" if direction == "AB" else f" {mode}")
                out[key] = {"us": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                            "kernel": hs[0].plan_info(w, direction, mode)["kernel_name"]}
    return {"workload": f"CSR {m} x {n}, {C.nnz} entries (Poisson(10) per row), float32; "
                        "launch-bound at this size (the matrix is 0.2 MB)", "products": out}


def large_vcs_products(dev, steps, widths=(8, 32)):
    """The 1,000,000 x 20,000 count matrix (~200M entries, values up to 255):
    the VCSR from the generator, the VCSC regrouped on the device by the
    library; widths 8 and 32, the four directions each the headline's way
    (deterministic through a schedule where the direction has one, else the
    plain walk) plus atomic mode for the misaligned two. One copy: the matrix
    (0.9 GB) is several times the 256 MB Infinity Cache. Device footprint
    against the expanded CSR, and each schedule's resident bytes."""
    import torch

    import sparse_dense_matmul_amd as sdm
    import workloads as W

    workers = max(1, min(16, cpu_threads()))
    t0 = time.perf_counter()
    L = W.config5_vcsr(workers=workers)
    log(f"1M x 20k VCSR generated in {time.perf_counter() - t0:.1f} s ({L.nnz} entries)")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    A = {"vcsr": sdm.VcsMatrix.from_arrays("vcsr", L.shape, up(L.major_ptr), up(L.values),
                                           up(L.value_ptr), up(L.indices))}
    A["vcsc"] = A["vcsr"].regroup()
    torch.cuda.synchronize()
    m, n = L.shape
    nbytes = {lay: a.footprint()[0] for lay, a in A.items()}
    stream = torch.cuda.current_stream(dev)
    res = {"footprint_bytes": nbytes, "expanded_csr_bytes": A["vcsr"].footprint()[1],
           "footprint_ratio": {lay: round(b / A["vcsr"].footprint()[1], 3)
                               for lay, b in nbytes.items()}}
    for w in widths:
        rng = np.random.default_rng(w)
        B = {"AB": up(W.dense_normal(rng, n, w)), "BA": up(W.dense_normal(rng, m, w))}
        per, tot_us, tot_b = {}, 0.0, 0
        for name, lay, direction, walk in DIRECTIONS:
            h = A[lay]
            o = torch.empty((m if direction == "AB" else n, w), device=dev)
            has_sc = h.workspace_size(direction, "deterministic", w) > 0
            entry = {}
            if has_sc:
                t0 = time.perf_counter()
                sc = h.schedule(direction, w)
                entry["schedule_build_ms"] = round(1e3 * (time.perf_counter() - t0), 1)
                entry["schedule_bytes"] = sc.nbytes
                run = lambda k=0: sc.spmm(B[direction], out=o)
            else:
                sc = None
                run = lambda k=0: h.spmm(B[direction], direction, out=o)
            us = time_launches(run, steps, stream)
            other = "vcsc" if lay == "vcsr" else "vcsr"
            walked = nbytes[lay] if walk == "aligned" else nbytes[other]
            nb = walked + dense_bytes(L.shape, direction, w)
            info = h.plan_info(w, direction, "deterministic" if has_sc else "atomic")
            entry.update(us=round(us, 1), GBps=round(nb / (us * 1e-6) / 1e9, 1),
                         frac=round(nb / (us * 1e-6) / 1e9 / PEAK_GBPS, 4),
                         kernel=info["kernel_name"] +
                         (f" (tiled, {info['tiles']} tiles) + k_tile_sum" if info["tiles"] else ""))
            if walk == "scatter":
                ua = time_launches(lambda k=0: h.spmm(B[direction], direction, out=o), steps,
                                   stream)
                ba = nbytes[lay] + dense_bytes(L.shape, direction, w)
                entry["atomic"] = {"us": round(ua, 1), "GBps": round(ba / (ua * 1e-6) / 1e9, 1)}
            per[name] = entry
            tot_us += us
            tot_b += nb
            del sc, o
            torch.cuda.empty_cache()
        res[f"w={w}"] = {"GBps": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
                         "frac": round(tot_b / (tot_us * 1e-6) / 1e9 / PEAK_GBPS, 4),
                         "directions": per}
        del B
    del A
    torch.cuda.empty_cache()
    return {"workload": f"VCS count matrix {m} x {n}, {L.nnz} entries, {L.n_groups} groups "
                        f"(VCSR), cold HBM", **res}


def other_widths(layouts, dev, widths, steps, copies=8):
    """The same four directions at other widths of the pages' workload (by
    default 1, 8, 32 and 64), beside the headline (not in it): each direction the way the
    headline runs it (deterministic, every workspace sized for the width),
    cold copies rotated. Returns per width the microseconds per direction and
    the aggregate GB/s over the same byte count as the headline."""
    import torch

    import sparse_dense_matmul_amd as sdm
    import workloads as W

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    res = {}
    stream = torch.cuda.current_stream(dev)
    m, n = layouts["vcsr"].shape
    hs = [{lay: sdm.VcsMatrix.from_arrays(lay, L.shape, *[up(a) for a in (L.major_ptr, L.values,
                                                                          L.value_ptr, L.indices)])
           for lay, L in layouts.items()} for _ in range(copies)]
    for w in widths:
        rng = np.random.default_rng(w)
        Bs = [{"AB": up(W.dense_normal(rng, n, w)), "BA": up(W.dense_normal(rng, m, w))}
              for _ in range(copies)]
        per, tot_us, tot_b = {}, 0.0, 0
        for name, lay, direction, walk in DIRECTIONS:
            L = layouts[lay]
            out = [torch.empty((m if direction == "AB" else n, w), device=dev) for _ in range(copies)]
            size = hs[0][lay].workspace_size(direction, "deterministic", w)
            mode = "deterministic" if size else "atomic"
            scs = [h[lay].schedule(direction, w) for h in hs] if size else None
            if scs:
                run = lambda k: scs[k % copies].spmm(Bs[k % copies][direction], out=out[k % copies])
            else:
                run = lambda k: hs[k % copies][lay].spmm(Bs[k % copies][direction], direction,
                                                         out=out[k % copies])
            for k in range(copies):
                run(k)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for k in range(steps):
                run(k)
            b.record(stream)
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / steps
            other = layouts["vcsc" if lay == "vcsr" else "vcsr"]
            nb = (L.nbytes() if walk == "aligned" else other.nbytes()) + dense_bytes(L.shape,
                                                                                   direction, w)
            info = hs[0][lay].plan_info(w, direction, mode)
            per[name] = {"us": round(us, 2), "kernel": info["kernel_name"] +
                         (f" (tiled, {info['tiles']} tiles) + k_tile_sum" if info["tiles"] else "")}
            if scs:
                per[name]["schedule_bytes"] = scs[0].nbytes
            tot_us += us
            tot_b += nb
            del scs, out
        res[f"w={w}"] = {"GBps": round(tot_b / (tot_us * 1e-6) / 1e9, 1), "directions": per}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--width", type=int, default=16)
    ap.add_argument("--copies", type=int, default=20, help="matrix copies rotated for cold HBM")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-atomic", action="store_true", help="skip the atomic-mode timings")
    ap.add_argument("--no-csr", action="store_true", help="skip the CSR operator timings")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--no-expand", action="store_true", help="skip the VCS expansion timings")
    ap.add_argument("--no-csr64", action="store_true",
                    help="skip the timings of the CSR past 2^31 entries")
    ap.add_argument("--other-widths", default="1,8,32,64",
                    help="widths also timed beside the headline (comma list, empty for none)")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the 1M x 20k matrix (widths 8 and 32, four directions)")
    ap.add_argument("--no-csr-small", action="store_true", help="skip the 2,000 x 500 CSR")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the secondary ceilings (LDS/L2 gathers, atomics, launches)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (a multi-GPU "
              "product would shard the matrix by major slices; only the one-GPU path exists)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.ceilings:
        print(json.dumps(ceilings()), flush=True)
        return

    import torch

    import sparse_dense_matmul_amd as sdm
    import workloads as W

    dev = torch.device("cuda:0")
    w = args.width
    log("generating the 60k x 2k count matrix")
    t = W.count_60k()
    layouts = {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}
    m, n = t.shape
    rng = np.random.default_rng(2)
    dense = {"AB": W.dense_normal(rng, n, w), "BA": W.dense_normal(rng, m, w)}

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base = {lay: [up(a) for a in (L.major_ptr, L.values, L.value_ptr, L.indices)]
            for lay, L in layouts.items()}
    dense_d = {d: up(x) for d, x in dense.items()}
    K = max(args.copies, 2)
    log(f"placing {K} copies of each operand set on the device")
    copies = []
    for _ in range(K):
        c = {"A": {}, "sc": {}}
        for lay, L in layouts.items():
            c["A"][lay] = sdm.VcsMatrix.from_arrays(lay, L.shape, *[a.clone() for a in base[lay]])
        c["B"] = {d: x.clone() for d, x in dense_d.items()}
        c["out"] = {(lay, d): torch.empty((m if d == "AB" else n, w), device=dev)
                    for lay in layouts for d in ("AB", "BA")}
        copies.append(c)
    torch.cuda.synchronize()

    def run(k, d, mode):
        name, lay, direction, _ = DIRECTIONS[d]
        c = copies[k % K]
        sc = c["sc"].get((lay, direction)) if mode == "deterministic" else None
        if sc is not None:
            sc.spmm(c["B"][direction], out=c["out"][(lay, direction)])
        else:
            c["A"][lay].spmm(c["B"][direction], direction, mode=mode,
                             out=c["out"][(lay, direction)])

    # one-time build of the deterministic schedules (vspmm_schedule_create):
    # the opposite layout of a misaligned direction, or the tiled copy of a
    # direction whose dense input does not fit in LDS, for this width
    build_ms, sched_bytes = {}, {}
    stream = torch.cuda.current_stream(dev)
    for d, (name, lay, direction, walk) in enumerate(DIRECTIONS):
        if copies[0]["A"][lay].workspace_size(direction, "deterministic", w) == 0:
            continue
        times = []
        for k in range(K):
            c = copies[k]
            scratch = c["A"][lay].workspace(direction, "deterministic", w)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            c["sc"][(lay, direction)] = c["A"][lay].schedule(direction, w, workspace=scratch)
            times.append(1e3 * (time.perf_counter() - t0))  # (the build waits for its stream)
            del scratch
        build_ms[name] = round(float(np.median(times)), 3)
        sched_bytes[name] = copies[0]["sc"][(lay, direction)].nbytes
    torch.cuda.empty_cache()
    log(f"deterministic schedules built: {build_ms} ms, resident bytes {sched_bytes}")

    def time_direction(d, mode):
        for k in range(args.warmup):
            run(k, d, mode)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k in range(args.steps):
            run(args.warmup + k, d, mode)
        b.record(stream)
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / args.steps  # us per launch

    wall0 = time.perf_counter()
    per_dir = {}
    for d, (name, lay, direction, walk) in enumerate(DIRECTIONS):
        L = layouts[lay]
        entry = {"walk": walk}
        A0 = copies[0]["A"][lay]
        has_ws = (lay, direction) in copies[0]["sc"]
        info = A0.plan_info(w, direction, "deterministic" if has_ws else "atomic")
        kernel = info["kernel_name"] + (" (tiled) + k_tile_sum" if info["tiles"] else "")
        tiled = f", tiled schedule ({info['tiles']} tiles of B)" if info["tiles"] else ""
        if walk == "aligned":
            us = time_direction(d, "deterministic" if has_ws else "atomic")
            b = L.nbytes() + dense_bytes(L.shape, direction, w)
            entry.update(us=round(us, 2), min_bytes=b, mode="aligned" + tiled, kernel=kernel)
        else:
            us = time_direction(d, "deterministic")
            # credited bytes: the matrix in the layout that runs along the
            # output (what a walk must read at least), never a schedule's extras
            other = layouts["vcsc" if lay == "vcsr" else "vcsr"]
            b = other.nbytes() + dense_bytes(L.shape, direction, w)
            entry.update(us=round(us, 2), min_bytes=b,
                         mode="deterministic (pass 2)" + tiled, kernel=kernel)
            if not args.no_atomic:
                ua = time_direction(d, "atomic")
                ba = L.nbytes() + dense_bytes(L.shape, direction, w)
                entry["atomic"] = {"us": round(ua, 2), "min_bytes": ba,
                                   "GBps": round(ba / (ua * 1e-6) / 1e9, 1),
                                   "kernels": "k_zero + k_scatter"}
        entry["GBps"] = round(entry["min_bytes"] / (entry["us"] * 1e-6) / 1e9, 1)
        entry["frac"] = round(entry["GBps"] / PEAK_GBPS, 4)
        per_dir[name] = entry
    wall = time.perf_counter() - wall0

    step_us = sum(e["us"] for e in per_dir.values())
    step_bytes = sum(e["min_bytes"] for e in per_dir.values())
    value = step_bytes / (step_us * 1e-6) / 1e9
    dom = max(per_dir, key=lambda k: per_dir[k]["us"])

    # the same steps replayed from a HIP graph (beside the headline): one
    # graph holds a step on every copy, each direction in its headline mode
    graph = None
    if not args.no_graph:
        modes = ["deterministic" if (lay, direction) in copies[0]["sc"] else "atomic"
                 for _, lay, direction, _ in DIRECTIONS]
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for k in range(K):
                    for d in range(len(DIRECTIONS)):
                        run(k, d, modes[d])
        torch.cuda.synchronize()
        reps = max(2, -(-args.steps // K))
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        g_step_us = 1e3 * a.elapsed_time(b) / (reps * K)
        graph = {"ms_per_step": round(g_step_us / 1e3, 5),
                 "GBps": round(step_bytes / (g_step_us * 1e-6) / 1e9, 1),
                 "steps": reps * K,
                 "how": f"a HIP graph of {K} steps (one per operand copy, the four directions each in "
                        "its headline mode), replayed; the same kernels and bytes as the headline"}
        del g

    # guard: aligned and deterministic outputs repeat bit for bit
    c0 = copies[0]
    r1 = c0["A"]["vcsr"].spmm(c0["B"]["AB"], "AB").clone()
    r2 = c0["A"]["vcsr"].spmm(c0["B"]["AB"], "AB")
    sc = c0["sc"][("vcsc", "AB")]
    r3 = sc.spmm(c0["B"]["AB"]).clone()
    r4 = sc.spmm(c0["B"]["AB"])
    repeat_ok = bool(torch.equal(r1, r2) and torch.equal(r3, r4))

    traffic, traffic_src = traffic_record(per_dir[dom]["kernel"], dom, w)
    # atomic mode against the measured float-atomic ceiling (a width-16 scatter's
    # adds at the probe's rate; the probe adds 16 columns per entry)
    probe = probe_record()
    if probe and not args.no_atomic and w == 16:
        rate = probe["atomic_w16_G_entries_per_s"] * 1e9
        for name, e in per_dir.items():
            if "atomic" in e:
                e["atomic"]["frac_of_atomic_ceiling"] = round(t.nnz / rate * 1e6 / e["atomic"]["us"], 3)
    atomic_us = sum(e["atomic"]["us"] if "atomic" in e else e["us"] for e in per_dir.values())
    atomic_bytes = sum(e["atomic"]["min_bytes"] if "atomic" in e else e["min_bytes"]
                       for e in per_dir.values())
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"VCS count matrix {m} x {n}, {t.nnz} nnz, width {w}, 4 directions "
                               "(VCSR@B, B@VCSR, VCSC@B, B@VCSC); misaligned directions in "
                               "deterministic two-pass mode with the schedule built, "
                               "B@VCSC on its tiled schedule; cold HBM",
                   "width": w, "parallelism": "none (1 GPU)"},
        "frac_of_peak": round(value / PEAK_GBPS, 4),
        "gflops": round(4 * 2 * t.nnz * w / (step_us * 1e-6) / 1e9, 1),
        "directions": per_dir,
        "atomic_mode": {"value": round(atomic_bytes / (atomic_us * 1e-6) / 1e9, 2) if not
                        args.no_atomic else None, "unit": "GB/s",
                        "ms_per_step": round(atomic_us / 1e3, 5) if not args.no_atomic else None},
        "det_schedule_build_ms": build_ms,
        "det_schedule_bytes": sched_bytes,
        "footprint_bytes": {lay: copies[0]["A"][lay].footprint()[0] for lay in layouts},
        "graph_replay": graph,
        "roofline": {"bound": "hbm", "kernel": f"{per_dir[dom]['kernel']} ({dom})",
                     "achieved": per_dir[dom]["GBps"], "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": per_dir[dom]["frac"], "traffic": traffic,
                     "traffic_source": traffic_src,
                     "algorithmic_bytes": per_dir[dom]["min_bytes"],
                     "launch_us": per_dir[dom]["us"],
                     # what bounds the walk below the HBM roofline (SQ counters)
                     # what bounds the walk below the HBM roofline: its SQ counters,
                     # and the measured ceilings of the other resources it uses
                     "secondary": {"counters": ceiling_record(per_dir[dom]["kernel"].split()[0]),
                                   "ceilings": probe}},
        "repeat_bitwise": repeat_ok,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_expand:
        log("timing the expansions (reported beside the headline)")
        result["expand"] = expansions(layouts, dev, args.steps)
    if args.other_widths:
        log("timing the other widths (reported beside the headline)")
        result["other_widths"] = other_widths(
            layouts, dev, [int(x) for x in args.other_widths.split(",")], args.steps)
    if not args.no_csr_small:
        log("timing the 2,000 x 500 CSR (reported beside the headline)")
        result["csr_small"] = csr_small_products(dev, args.steps)
    if not args.no_large:
        log("timing the 1M x 20k matrix (reported beside the headline)")
        result["large"] = large_vcs_products(dev, max(3, min(args.steps, 10)))
    if not args.no_csr:
        log("timing the CSR operator (reported beside the headline)")
        result["csr"] = csr_products(dev, args.steps)
    if not args.no_csr64:
        log("timing the CSR past 2^31 entries (reported beside the headline)")
        result["csr64"] = csr64_products(dev, args.steps)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        result["cpu_baseline"] = cpu_baseline(layouts, w, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
