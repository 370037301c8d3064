"""Benchmark of the FlashIPA forward (lift + fused attention + epilogue) on one
MI355X.

Prints ONE JSON line.  A step is one forward of the whole path over one batch
of synthetic, seeded inputs already resident in HBM.  The headline workload is
the long-sequence case B=1, N=16384, H=8, D=Dv=16, P=4, Q=8, Cz=64, R=2,
Cout=128, bf16 inputs (random-walk frames, 3.8 angstrom steps, all masks
valid); the other sequence lengths of the sweep (and the short-chain batch at
N=512) are reported under "sweep".

value = effective TFLOP/s = 2 H (d_qk + d_v) sum_b L_b^2 / time per forward,
with d_qk = D + 3P + 2 + R Cz and d_v = Dv + 3Q + R Cz (the lifted inner
product and value widths of the method; padding and split columns are not
counted).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "IPA fwd ms/call + effective TFLOP/s (% MFMA peak) at N=512..16384; peak mem"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "flash_mfma_traffic.json")
KERNEL_SOURCES = ("flash_mfma.hip", "mfma_tile.h", "common.h")


def host_cores() -> dict:
    """Host CPU the oracle baselines run on: the cores this process may use
    (at most 16, one GPU's share of a box), nproc and the CPU model."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cores": max(1, min(usable, 16)), "nproc": os.cpu_count(), "cpu_model": model}


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rna_structure_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def eff_flops(shape, mask) -> float:
    L = mask.sum(axis=1).astype(float)
    return 2.0 * shape.H * (shape.d_qk + shape.d_v) * float((L ** 2).sum())


def _mfma_dims(shape):
    """(NQS, NVB, GS) of the compiled matrix-core instance used for a shape."""
    rcz = shape.R * shape.Cz
    for nqs, nvb in ((3, 2), (5, 3), (9, 5), (13, 7)):
        if shape.D + rcz <= 16 * nqs and shape.Dv + rcz + 1 <= 32 * nvb:
            return nqs, nvb, (3 if shape.P <= 4 else 4)
    raise ValueError("no matrix-core instance for this shape")


def lift_bytes(shape, with_pm: bool) -> float:
    """Algorithmic HBM bytes of the lift kernel: every input read once, every
    lifted row written once (per residue: q, k, v, the points, frames, zl, zr,
    mask; per head key rows, transposed value rows, the 16 scalar query
    columns, query points; once the pair-factor key and value rows and the
    query pair-factor row that the heads share)."""
    nqs, nvb, gs = _mfma_dims(shape)
    H, R, Cz = shape.H, shape.R, shape.Cz
    rd = 2 * H * (2 * shape.D + shape.Dv) + 2 * 3 * H * (2 * shape.P + shape.Q) + 2 * 12 + 2 * 2 * R * Cz + 1
    kt = H * (16 + 16 * gs + 8) * 2 + (16 * (nqs - 1) + 8) * 2  # head key rows + shared pair-factor rows
    vz = (32 * (nvb - 1) * 72 * 2 + 1023) // 1024 * 1024
    vt = H * 64 * 72 * 2 / 64 + vz / 64                      # head value rows + shared pair-factor rows
    wr = kt + vt + H * 16 * 2 + 16 * (nqs - 1) * 2 + H * 16 * 4
    per_res = rd + wr
    extra = shape.B * shape.N * shape.N if with_pm else 0
    return shape.B * shape.N * per_res + extra


def lift_method_bytes(shape, with_pm: bool) -> float:
    """HBM bytes of the lift as the method lays its rows out (Flash IPA page,
    the factorised logit): the same inputs read once, and per head a query
    row and a key row of d_qk = D + 3P + 2 + R Cz columns and a value row of
    d_v = Dv + 3Q + R Cz columns written in 16-bit, the pair factors inside
    every head's rows.  The lift here shares the pair-factor rows among the
    heads and moves fewer bytes (lift_bytes); this count is the work of the
    method, as flops count the method's products."""
    H, R, Cz = shape.H, shape.R, shape.Cz
    rd = 2 * H * (2 * shape.D + shape.Dv) + 2 * 3 * H * (2 * shape.P + shape.Q) + 2 * 12 + 2 * 2 * R * Cz + 1
    d_qk = shape.D + 3 * shape.P + 2 + R * Cz
    d_v = shape.Dv + 3 * shape.Q + R * Cz
    wr = H * (2 * d_qk + d_v) * 2
    extra = shape.B * shape.N * shape.N if with_pm else 0
    return shape.B * shape.N * (rd + wr) + extra


def epilogue_bytes(shape) -> float:
    """Algorithmic HBM bytes of the epilogue: O, lse, zl and frames read, the
    update and local points written, per residue (w_out once)."""
    H = shape.H
    do = shape.Dv + shape.R * shape.Cz + 3 * shape.Q
    rd = H * do * 4 + H * 4 + 2 * shape.R * shape.Cz + 2 * 12
    wr = shape.Cout * 4 + H * shape.Q * 3 * 4
    return shape.B * shape.N * (rd + wr) + 2 * shape.F * shape.Cout


def make_workload(name):
    from rna_structure_amd.synth import make_config
    return make_config(name)


def time_forward(inp, steps, warmup, per_kernel=True, min_warm_ms=40.0, stacked=False):
    """Forward time with inputs resident: `warmup` untimed forwards, continued
    until at least min_warm_ms of GPU time has passed (the clock ramps up over
    the first tens of milliseconds of load), then `steps` timed forwards.
    stacked=True times the pages' stacked point layout (comparison calls)."""
    import torch
    from rna_structure_amd import _lib
    shape = inp["shape"]
    t = _lib.device_inputs(inp, "cuda")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_mem = torch.cuda.memory_allocated()
    f = _lib.FlashIPA(shape, eps=inp["eps"], with_pair_mask=t["pair_mask"] is not None, stacked=stacked)
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record()
    for _ in range(warmup):
        f.forward(t)
    w1.record()
    torch.cuda.synchronize()
    warm = w0.elapsed_time(w1)
    while warm < min_warm_ms:
        w0.record()
        for _ in range(max(1, warmup)):
            f.forward(t)
        w1.record()
        torch.cuda.synchronize()
        warm += w0.elapsed_time(w1)
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        f.forward(t)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    res = dict(ms=ms, peak_mem_mb=torch.cuda.max_memory_allocated() / 2**20,
               work_mem_mb=(torch.cuda.max_memory_allocated() - base_mem) / 2**20)
    if per_kernel:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for k in range(steps):
            ev[k][0].record(st)
            f.lift(t)
            ev[k][1].record(st)
            f.attend()
            ev[k][2].record(st)
            f.epilogue(t)
            ev[k][3].record(st)
        torch.cuda.synchronize()
        res["lift_ms"] = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
        res["flash_ms"] = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
        res["epilogue_ms"] = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    del f, t
    torch.cuda.empty_cache()
    return res


# kNN distogram (pair-feature preprocessing): 8 fp32 operations per ordered
# pair (3 differences, 3 squares, 2 sums) against the rate of unfused,
# unpacked fp32 vector operations: 256 CUs x 64 lanes x 2.4 GHz.
KNN_FLOPS_PER_PAIR = 8
PEAK_VALU_TOPS = 256 * 64 * 2.4e9 / 1e12
KNN_WORKLOADS = (
    ("knn_16384", 1, 16384, dict(frames="walk", step=3.8)),
    ("knn_rna_2048", 1, 2048, dict(frames="walk", step=6.0)),
    ("knn_short_batch", 39, 512, dict(frames="walk", step=3.8)),
    ("knn_gauss_8192", 1, 8192, dict(frames="gauss", trans_sigma=30.0)),
)


def time_knn(name, B, N, kw, steps, k=20, nbins=20, dmax=20.0, min_warm_ms=40.0):
    """Time ipa_knn_distogram on resident positions: warm-up of at least
    min_warm_ms of GPU time, then `steps` timed calls."""
    import numpy as np
    import torch
    from rna_structure_amd import _lib
    from rna_structure_amd.synth import make_positions
    pos = make_positions(B, N, 7000 + N, **kw)
    t = torch.from_numpy(np.ascontiguousarray(pos["translation"])).cuda()
    m = torch.from_numpy(pos["mask"].astype(np.uint8)).cuda()
    kd = _lib.KnnDistogram(B, N, k, nbins, dmax)
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    warm = 0.0
    while warm < min_warm_ms:
        e0.record(st)
        for _ in range(5):
            kd(t, m)
        e1.record(st)
        torch.cuda.synchronize()
        warm += e0.elapsed_time(e1)
    e0.record(st)
    for _ in range(steps):
        kd(t, m)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = B * N * N
    tops = KNN_FLOPS_PER_PAIR * pairs / (ms * 1e-3) / 1e12
    out_bytes = B * N * k * (4 + 4 + 4 * nbins)
    return {"workload": name, "B": B, "N": N, "k": k, "nbins": nbins, "frames": kw["frames"], "ms": round(ms, 4),
            "gpairs_per_s": round(pairs / (ms * 1e-3) / 1e9, 1), "alu_tflops": round(tops, 2),
            "alu_frac": round(tops / PEAK_VALU_TOPS, 4), "out_bytes": out_bytes,
            "out_GBs": round(out_bytes / (ms * 1e-3) / 1e9, 1)}


# Backward (fp32 arithmetic): algorithmic flops per (query, key, head) of the
# attention core without recomputation -- logit 2 d_k + 9P, output 2 d_v,
# dP 2 d_v, dQ and dK 2 d_k each, dV 2 d_v, point gradients 12P -- against the
# unpacked fp32 FMA rate 256 CUs x 64 lanes x 2 x 2.4 GHz = 78.6 TFLOP/s.
PEAK_FP32_FMA_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12
# The pair passes of the standard widths run on fp32 matrix cores (dense fp32
# MFMA 157.3 TFLOP/s); the same algorithmic flops are reported against both.
PEAK_FP32_MFMA_TFLOPS = 157.3
BACKWARD_WORKLOADS = (
    ("backward_rna_2048", 1, 2048, dict(frames="walk", step=6.0), 10),
    ("backward_4096", 1, 4096, dict(frames="walk", step=3.8), 5),
    ("backward_16384", 1, 16384, dict(frames="walk", step=3.8), 2),
)


def backward_flops(shape, mask) -> float:
    import numpy as np
    dk = shape.D + shape.R * shape.Cz
    dv = shape.Dv + shape.R * shape.Cz + 3 * shape.Q
    per_pair = 6 * dk + 6 * dv + 21 * shape.P
    L = np.asarray(mask).sum(axis=1).astype(np.float64)
    return float(shape.H * per_pair * np.sum(L * L))


def time_backward(name, B, N, kw, steps, min_warm_ms=40.0):
    import numpy as np
    import torch
    from rna_structure_amd import _lib
    from rna_structure_amd.synth import IPAShape, make_inputs
    shape = IPAShape(B=B, N=N, H=8, dtype="f32")
    inp = make_inputs(shape, 8000 + N, **kw)
    t = _lib.device_inputs(inp, "cuda")
    rng = np.random.default_rng(N)
    du = torch.from_numpy(rng.standard_normal((B, N, shape.Cout)).astype(np.float32)).cuda()
    dl = torch.from_numpy(rng.standard_normal((B, N, shape.H, shape.Q, 3)).astype(np.float32)).cuda()
    bw = _lib.IPABackward(shape, eps=inp["eps"])
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    warm = 0.0
    while warm < min_warm_ms:
        e0.record(st)
        bw(t, du, dl)
        e1.record(st)
        torch.cuda.synchronize()
        warm += e0.elapsed_time(e1)
    e0.record(st)
    for _ in range(steps):
        bw(t, du, dl)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = backward_flops(shape, inp["mask"])
    tf = fl / (ms * 1e-3) / 1e12
    ws_mb = bw.ws.numel() / 2**20
    del bw, t
    torch.cuda.empty_cache()
    return {"workload": name, "B": B, "N": N, "H": shape.H, "ms": round(ms, 3), "tflops": round(tf, 2),
            "frac_fp32_mfma": round(tf / PEAK_FP32_MFMA_TFLOPS, 4), "frac_fp32_fma": round(tf / PEAK_FP32_FMA_TFLOPS, 4),
            "workspace_mb": round(ws_mb, 1)}


def backward_cpu_baseline(N=2048):
    """The float64 autograd oracle for a whole backward at a bounded length
    (same widths, B=1, H=8) on the host's cores: the upstream rows split into
    one block per process (the gradients of the blocks add up to the whole),
    as algorithmic TFLOP/s (the flops of backward_flops)."""
    from rna_structure_amd.synth import IPAShape, make_inputs
    sh = IPAShape(B=1, N=N, H=8, dtype="f32")
    inp = make_inputs(sh, 9000 + N, frames="walk", step=3.8)
    # The backward oracle's workers import torch, and a process that has
    # loaded torch counts as one that holds the GPU: keep those workers, this
    # process and the child within the 16 processes one GPU may have.
    r = _run_cpu_oracle("backward", str(N), 0.0, max_workers=12)
    flops = backward_flops(sh, inp["mask"])
    return dict(value=round(flops / r["seconds_per_call"] / 1e12, 6), unit="TFLOP/s", cores=r["workers"],
                kind="oracle", nproc=r["nproc"], cpu_model=r["cpu_model"],
                sample=f"whole backward at N={N} (B1 H8, standard widths), float64 autograd oracle, upstream rows "
                       f"in {r['workers']} blocks on as many processes, {r['wall_s']:.1f} s wall")


def backward_section(args):
    res = []
    for name, B, N, kw, steps in BACKWARD_WORKLOADS:
        res.append(time_backward(name, B, N, kw, steps))
        print(f"# backward {res[-1]}", file=sys.stderr, flush=True)
    sec = {"peak_fp32_mfma_tflops": PEAK_FP32_MFMA_TFLOPS, "peak_fp32_fma_tflops": round(PEAK_FP32_FMA_TFLOPS, 1),
           "inputs": "fp32", "runs": res}
    if not args.no_cpu_baseline:
        sec["cpu_baseline"] = backward_cpu_baseline()
    return sec


def knn_cpu_baseline(N=16384, budget_s=3.0):
    """The kNN oracle on a sample of rows of the N-residue walk on the host's
    cores (rows split over one process per core), scaled to all rows."""
    r = _run_cpu_oracle("knn", str(N), budget_s)
    return {"workload": f"knn_{N}", "ms_per_call": round(r["seconds_per_call"] * 1e3, 1), "cores": r["workers"],
            "nproc": r["nproc"], "cpu_model": r["cpu_model"], "kind": "oracle",
            "sample": f"{r['rows']} of {N} rows, fp32 NumPy oracle in {r['workers']} processes, "
                      f"{r['wall_s']:.1f} s wall, scaled by N/rows"}


# ---------------------------------------------------------------- CPU oracle baselines
# The oracles are plain NumPy / PyTorch code whose einsums run on one core.
# To time them on the host's cores, a child process (started with
# --cpu-oracle, never touching the GPU) splits independent query rows over
# worker processes, one BLAS thread each: forward rows are independent, and
# the backward's gradient is a sum over upstream rows, so row blocks of the
# row-restricted gradient oracle add up to the whole backward.
_ORACLE = {}


def _oracle_job(rows):
    import numpy as np
    from threadpoolctl import threadpool_limits
    kind = _ORACLE["kind"]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if kind == "forward":
            from oracle import ipa_factored
            ipa_factored(_ORACLE["inp"], rows=rows, keep=("update", "local_points"))
        elif kind == "backward":
            import torch
            torch.set_num_threads(1)
            from oracle.ipa_backward import ipa_gradients
            du, dl = _ORACLE["du"], _ORACLE["dl"]
            ipa_gradients(_ORACLE["inp"], du[:, rows], dl[:, rows], rows=list(rows))
        elif kind == "knn":
            from oracle import knn_distogram
            pos = _ORACLE["inp"]
            knn_distogram(pos["translation"], pos["mask"], k=20, rows=np.asarray(rows))
        else:
            from oracle import flashbias_rows
            inp = _ORACLE["inp"]
            flashbias_rows(inp["q"], inp["k"], inp["v"], inp["phi_q"], inp["phi_k"], _ORACLE["scale"],
                           np.asarray(rows))
        return time.perf_counter() - t0


def cpu_oracle_main(kind: str, arg: str, budget_s: float, workers: int) -> None:
    """Child process: time an oracle on `workers` processes (one BLAS thread
    each) over a bounded sample of rows; print one JSON line."""
    import concurrent.futures
    import multiprocessing
    import numpy as np
    _ORACLE["kind"] = kind
    if kind == "forward":
        inp = make_workload(arg)
        N, nb = inp["shape"].N, inp["shape"].B
    elif kind == "backward":
        from rna_structure_amd.synth import IPAShape, make_inputs
        N = int(arg)
        sh = IPAShape(B=1, N=N, H=8, dtype="f32")
        inp = make_inputs(sh, 9000 + N, frames="walk", step=3.8)
        rng = np.random.default_rng(1)
        _ORACLE["du"] = rng.standard_normal((1, N, sh.Cout))
        _ORACLE["dl"] = rng.standard_normal((1, N, sh.H, sh.Q, 3))
    elif kind == "knn":
        from rna_structure_amd.synth import make_positions
        N = int(arg)
        inp = make_positions(1, N, 7000 + N, frames="walk", step=3.8)
    else:
        from rna_structure_amd.synth import make_bias_inputs
        name, dims, bkind, causal, _ = FLASHBIAS_WORKLOADS[1]
        inp = make_bias_inputs(**dims, seed=8000 + dims["N"], kind=bkind)
        _ORACLE["scale"] = 1.0 / math.sqrt(dims["D"])
        N = dims["N"]
    _ORACLE["inp"] = inp
    rng = np.random.default_rng(0)
    if kind == "backward":
        n = N  # the whole backward, split into row blocks
    else:
        probe = np.sort(rng.choice(N, size=min(N, 16), replace=False))
        per_row = _oracle_job(probe) / len(probe)
        n = int(max(workers, min(N, budget_s * workers / max(per_row, 1e-9))))
    rows = np.sort(rng.choice(N, size=n, replace=False))
    chunks = [c for c in np.array_split(rows, workers) if len(c)]
    ctx = multiprocessing.get_context("fork")
    with concurrent.futures.ProcessPoolExecutor(max_workers=len(chunks), mp_context=ctx) as ex:
        list(ex.map(_oracle_job, [chunks[0][:1]] * len(chunks)))  # start the workers
        t0 = time.perf_counter()
        list(ex.map(_oracle_job, chunks))
        wall = time.perf_counter() - t0
    print(json.dumps({"seconds_per_call": wall * N / n, "rows": n, "N": N, "wall_s": wall,
                      "workers": len(chunks)}), flush=True)


def _run_cpu_oracle(kind: str, arg: str, budget_s: float, max_workers: int = 16) -> dict:
    """Run cpu_oracle_main in a child process (which never touches the GPU)."""
    import subprocess
    host = host_cores()
    workers = min(host["cores"], max_workers)
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-oracle", kind, arg, str(budget_s), str(workers)]
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, env=env)
    if r.returncode != 0:
        raise RuntimeError(f"cpu oracle child failed: {r.stderr[-2000:]}")
    out = json.loads(r.stdout.strip().splitlines()[-1])
    out.update(host)
    return out


def _oracle_rate(inp, threads, budget_s):
    """Seconds per whole forward of the float64 oracle with `threads` BLAS
    threads, from a bounded sample of query rows scaled by N/rows (the per-row
    cost is the same for every row at fixed N); also the sample size."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import ipa_factored
    shape = inp["shape"]
    N = shape.N
    rng = np.random.default_rng(0)
    with threadpool_limits(limits=threads):
        rows = np.sort(rng.choice(N, size=min(N, 16), replace=False))
        t0 = time.perf_counter()
        ipa_factored(inp, rows=rows, keep=("update", "local_points"))
        per_row = (time.perf_counter() - t0) / len(rows)
        n = int(max(16, min(N, budget_s / max(per_row, 1e-9))))
        rows = np.sort(rng.choice(N, size=n, replace=False))
        t0 = time.perf_counter()
        ipa_factored(inp, rows=rows, keep=("update", "local_points"))
        el = time.perf_counter() - t0
    return el * N / n, n, el


def cpu_baseline(workload, inp, flops, budget_s=12.0):
    """The float64 oracle on the host's cores (query rows split over one
    process per core), timed on a bounded sample of query rows and scaled to
    the whole forward; the one-thread rate beside it."""
    shape = inp["shape"]
    r = _run_cpu_oracle("forward", workload, budget_s)
    one_s, n1, el1 = _oracle_rate(inp, 1, budget_s / 4)
    return dict(value=flops / r["seconds_per_call"] / 1e12, unit="TFLOP/s", cores=r["workers"], kind="oracle",
                sample=f"{r['rows']} of {shape.N} query rows x all {shape.B} samples, float64 NumPy oracle in "
                       f"{r['workers']} processes (one BLAS thread each), {r['wall_s']:.1f} s wall, scaled by "
                       f"N/rows to {r['seconds_per_call']:.1f} s per forward",
                seconds_per_call=r["seconds_per_call"], nproc=r["nproc"], cpu_model=r["cpu_model"],
                one_thread={"value": flops / one_s / 1e12, "seconds_per_call": one_s,
                            "sample": f"{n1} rows on one thread, {el1:.1f} s measured"})


def copy_calibration(mib: int, reps: int = 3) -> None:
    """Plain device-to-device copies of a known size: the HBM counters
    (FETCH_SIZE, WRITE_SIZE) read for this kernel calibrate those read for
    the FlashIPA kernels in the same profiling pass."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "reps": reps}), flush=True)


def hbm_calibration(mib: int = 2048, reps: int = 10) -> dict:
    """Achievable HBM rates of plain device kernels: a fill (writes only), a
    copy (read + write) and a sum (reads only) over MIB MiB, event-timed."""
    import torch
    n = mib * 2**20 // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    res = {}
    for name, fn, nbytes in (("fill", lambda: y.fill_(1.0), 4 * n),
                             ("copy", lambda: y.copy_(x), 8 * n),
                             ("sum", lambda: x.sum(), 4 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 4)}
    del x, y
    torch.cuda.empty_cache()
    return res


# Attention with a low-rank bias (bf16 matrix cores): algorithmic flops per
# (query, permitted key, head) 2 (D + R) for the logit with its bias and 2 Dv
# for the output, against the dense bf16 MFMA peak.  Workloads named after the
# FlashBias page's settings: a GPT-2-style causal ALiBi layer at N = 2048 (25
# heads of 64, the 1.5B model's), and a squared-distance bias over the 32186
# points of the PDE case (8 heads of 32, points in the unit cube).
FLASHBIAS_WORKLOADS = (
    ("alibi_gpt2_2048", dict(B=8, N=2048, M=2048, H=25, D=64, Dv=64, R=2), "alibi", True, 10),
    ("sqdist_pde_32186", dict(B=1, N=32186, M=32186, H=8, D=32, Dv=32, R=5), "sqdist", False, 5),
)


def time_flashbias(name, dims, kind, causal, steps, min_warm_ms=40.0):
    import numpy as np
    import torch
    from rna_structure_amd import _lib
    from rna_structure_amd.synth import make_bias_inputs
    inp = make_bias_inputs(**dims, seed=8000 + dims["N"], kind=kind)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dt).contiguous()
    q, k, v = (dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    pq, pk = (dev(inp[n], torch.float32) for n in ("phi_q", "phi_k"))
    km = torch.from_numpy(inp["key_mask"].astype(np.uint8)).cuda()
    f = _lib.BiasAttention(dims["B"], dims["N"], dims["M"], dims["H"], dims["D"], dims["Dv"], dims["R"],
                           1.0 / math.sqrt(dims["D"]), causal, "bf16", "f32")
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    warm = 0.0
    while warm < min_warm_ms:
        e0.record(st)
        for _ in range(3):
            f(q, k, v, pq, pk, km, stream=st)
        e1.record(st)
        torch.cuda.synchronize()
        warm += e0.elapsed_time(e1)
    e0.record(st)
    for _ in range(steps):
        f(q, k, v, pq, pk, km, stream=st)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    B, N, M, H = dims["B"], dims["N"], dims["M"], dims["H"]
    pairs = B * H * (N * (N + 1) // 2 if causal else N * M)
    flops = pairs * (2 * (dims["D"] + dims["R"]) + 2 * dims["Dv"])
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": name, **dims, "kind": kind, "causal": causal, "inputs": "bf16 q/k/v, fp32 factors",
            "ms": round(ms, 4), "pair_heads": pairs, "flops_per_pair_head": 2 * (dims["D"] + dims["R"]) + 2 * dims["Dv"],
            "tflops": round(tf, 2), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def flashbias_cpu_baseline(budget_s=10.0):
    """The float64 oracle on a sample of query rows of the squared-distance
    workload on the host's cores (rows split over one process per core),
    scaled by N/rows to a whole call (algorithmic TFLOP/s)."""
    name, dims, kind, causal, _ = FLASHBIAS_WORKLOADS[1]
    r = _run_cpu_oracle("flashbias", name, budget_s)
    N = dims["N"]
    flops = dims["B"] * dims["H"] * N * dims["M"] * (2 * (dims["D"] + dims["R"]) + 2 * dims["Dv"])
    return dict(value=round(flops / r["seconds_per_call"] / 1e12, 6), unit="TFLOP/s", cores=r["workers"],
                kind="oracle", nproc=r["nproc"], cpu_model=r["cpu_model"],
                sample=f"{r['rows']} of {N} query rows of {name}, float64 NumPy oracle in {r['workers']} processes, "
                       f"{r['wall_s']:.1f} s wall, scaled by N/rows to {r['seconds_per_call']:.0f} s per call")


def flashbias_section(args):
    res = []
    for name, dims, kind, causal, steps in FLASHBIAS_WORKLOADS:
        res.append(time_flashbias(name, dims, kind, causal, max(steps, args.steps // 2)))
        print(f"# flashbias {res[-1]}", file=sys.stderr, flush=True)
    sec = {"peak_bf16_tflops": PEAK_BF16_TFLOPS, "runs": res}
    if not args.no_cpu_baseline:
        sec["cpu_baseline"] = flashbias_cpu_baseline()
    return sec


def knn_section(args):
    res = []
    for name, B, N, kw in KNN_WORKLOADS:
        res.append(time_knn(name, B, N, kw, max(5, args.steps)))
        print(f"# knn {res[-1]}", file=sys.stderr, flush=True)
    sec = {"peak_alu_tflops": round(PEAK_VALU_TOPS, 2), "flops_per_pair": KNN_FLOPS_PER_PAIR, "runs": res}
    if not args.no_cpu_baseline:
        sec["cpu_baseline"] = knn_cpu_baseline()
    return sec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="sweep_16384")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-knn", action="store_true", help="skip the kNN distogram section")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward section")
    ap.add_argument("--backward-only", action="store_true",
                    help="run only the backward section and print it as the JSON line")
    ap.add_argument("--no-flashbias", action="store_true", help="skip the low-rank-bias attention section")
    ap.add_argument("--flashbias-only", action="store_true",
                    help="run only the low-rank-bias attention section and print it as the JSON line")
    ap.add_argument("--knn-only", action="store_true",
                    help="run only the kNN distogram section and print it as the JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run only plain copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--hbm-calibration", action="store_true",
                    help="print the fill / copy / sum rates of plain device kernels and exit")
    ap.add_argument("--stacked-layout", action="store_true",
                    help="time the headline workload with the pages' stacked point layout (comparison calls "
                         "ipa_lift_stacked / ipa_flash_fwd_stacked) instead of the centred split")
    ap.add_argument("--cpu-oracle", nargs=4, metavar=("KIND", "ARG", "BUDGET_S", "WORKERS"),
                    help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_oracle:
        kind, arg, budget, workers = args.cpu_oracle
        cpu_oracle_main(kind, arg, float(budget), int(workers))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.hbm_calibration:
        print(json.dumps({"hbm_calibration": hbm_calibration()}), flush=True)
        return
    if args.knn_only:
        print(json.dumps({"knn_distogram": knn_section(args)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": backward_section(args)}), flush=True)
        return
    if args.flashbias_only:
        print(json.dumps({"flashbias": flashbias_section(args)}), flush=True)
        return
    inp = make_workload(args.workload)
    shape = inp["shape"]
    flops = eff_flops(shape, inp["mask"])
    print(f"# workload {args.workload} {shape}", file=sys.stderr, flush=True)
    r = time_forward(inp, args.steps, args.warmup, min_warm_ms=0.0, stacked=args.stacked_layout)
    value = flops / (r["ms"] * 1e-3) / 1e12
    achieved = flops / (r["flash_ms"] * 1e-3) / 1e12
    traffic = None
    try:
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        if tr.get("kernel_hash") == kernel_hash() and tr.get("workload") == args.workload and not args.stacked_layout:
            traffic = tr["fetch_bytes"] + tr["write_bytes"]
    except (OSError, ValueError, KeyError):
        traffic = None
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"long-sequence IPA forward {args.workload}", "B": shape.B, "N": shape.N,
                   "H": shape.H, "D": shape.D, "Dv": shape.Dv, "P": shape.P, "Q": shape.Q, "Cz": shape.Cz,
                   "R": shape.R, "Cout": shape.Cout, "inputs": "bf16", "accumulate": "fp32",
                   **({"layout": "stacked bf16 point columns (comparison)"} if args.stacked_layout else {})},
        "kernels_ms": {"lift": round(r["lift_ms"], 4), "flash": round(r["flash_ms"], 4),
                       "epilogue": round(r["epilogue_ms"], 4)},
        "peak_mem_mb": round(r["peak_mem_mb"], 1),
        "hbm_kernels": {
            name: {"bytes": round(nb), "achieved_GBs": round(nb / (ms * 1e-3) / 1e9, 1),
                   "frac": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            for name, nb, ms in (("lift", lift_bytes(shape, inp["pair_mask"] is not None), r["lift_ms"]),
                                 ("epilogue", epilogue_bytes(shape), r["epilogue_ms"]))},
        "lift_method_layout": {
            "bytes": round(lift_method_bytes(shape, inp["pair_mask"] is not None)),
            "achieved_GBs": round(lift_method_bytes(shape, inp["pair_mask"] is not None) / (r["lift_ms"] * 1e-3) / 1e9, 1),
            "frac": round(lift_method_bytes(shape, inp["pair_mask"] is not None) / (r["lift_ms"] * 1e-3) / 1e9
                          / PEAK_HBM_GBS, 4)},
        "roofline": {"bound": "mfma", "kernel": "flash_mfma_kernel", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    print(json.dumps({"partial": out}), file=sys.stderr, flush=True)
    if not args.no_sweep:
        sweep = []
        for name in ("tiny", "protein", "rna", "short_batch", "sweep_4096", "sweep_8192", "sweep_16384",
                     "sweep_32768"):
            if name == args.workload:
                rr, sh, fl = r, shape, flops
            else:
                w = make_workload(name)
                sh = w["shape"]
                fl = eff_flops(sh, w["mask"])
                rr = time_forward(w, max(3, args.steps // 4), 2)
            sweep.append({"workload": name, "B": sh.B, "N": sh.N, "H": sh.H, "dtype": sh.dtype, "ms": round(rr["ms"], 4),
                          "eff_tflops": round(fl / (rr["ms"] * 1e-3) / 1e12, 2),
                          "flash_ms": round(rr["flash_ms"], 4),
                          "flash_frac_mfma": round(fl / (rr["flash_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "lift_ms": round(rr["lift_ms"], 4), "epilogue_ms": round(rr["epilogue_ms"], 4),
                          "peak_mem_mb": round(rr["peak_mem_mb"], 1), "work_mem_mb": round(rr["work_mem_mb"], 1)})
            print(f"# sweep {sweep[-1]}", file=sys.stderr, flush=True)
        pts = [s for s in sweep if s["workload"].startswith("sweep_")]
        if len(pts) >= 2:
            import numpy as np
            x = np.log([p["N"] for p in pts])
            for key, name in (("ms", "time_exponent"), ("work_mem_mb", "mem_exponent")):
                y = np.log([max(p[key], 1e-9) for p in pts])
                out[name] = round(float(np.polyfit(x, y, 1)[0]), 3)
        out["sweep"] = sweep
        # rank sweep of the pair factors (R = 1, 2, 3) at N = 8192: R = 3 runs
        # on the widest matrix-core instance
        from rna_structure_amd.synth import IPAShape, make_inputs
        ranks = []
        for R in (1, 2, 3):
            sh = IPAShape(B=1, N=8192, H=8, R=R)
            w = make_inputs(sh, 6000 + R, frames="walk", step=3.8)
            fl = eff_flops(sh, w["mask"])
            rr = time_forward(w, max(3, args.steps // 4), 2)
            ranks.append({"R": R, "N": sh.N, "H": sh.H, "ms": round(rr["ms"], 4),
                          "eff_tflops": round(fl / (rr["ms"] * 1e-3) / 1e12, 2),
                          "flash_ms": round(rr["flash_ms"], 4),
                          "flash_frac_mfma": round(fl / (rr["flash_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "lift_ms": round(rr["lift_ms"], 4), "epilogue_ms": round(rr["epilogue_ms"], 4)})
            print(f"# rank sweep {ranks[-1]}", file=sys.stderr, flush=True)
        out["rank_sweep"] = ranks
        # the pages' stacked point layout (five bf16 columns per point, global
        # coordinates, two geometric K-steps) against the centred fp16 hi/lo
        # split (three), same inputs; the flops counted are the algorithmic
        # ones of both (their accuracy is compared in the GPU tests)
        layouts = []
        for N in (8192, 16384):
            sh = IPAShape(B=1, N=N, H=8)
            w = make_inputs(sh, 7000 + N, frames="walk", step=3.8)
            fl = eff_flops(sh, w["mask"])
            for stk in (False, True):
                rr = time_forward(w, max(3, args.steps // 4), 2, stacked=stk)
                layouts.append({"layout": "stacked bf16 (pages)" if stk else "centred fp16 hi/lo", "N": N,
                                "geometric_ksteps": 2 if stk else 3, "ms": round(rr["ms"], 4),
                                "flash_ms": round(rr["flash_ms"], 4),
                                "flash_frac_mfma": round(fl / (rr["flash_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                "lift_ms": round(rr["lift_ms"], 4)})
                print(f"# layout comparison {layouts[-1]}", file=sys.stderr, flush=True)
        out["layout_comparison"] = layouts
    if not args.no_sweep and not args.no_knn:
        out["knn_distogram"] = knn_section(args)
    if not args.no_sweep and not args.no_backward:
        out["backward"] = backward_section(args)
    if not args.no_sweep and not args.no_flashbias:
        out["flashbias"] = flashbias_section(args)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.workload, inp, flops)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
