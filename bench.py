"""Throughput of the quantized attention hot path on one MI355X.

A step is one sage_attn_fwd call (quantisation pass + fused attention) over the
seeded synthetic Flux-like workload (B=1, H=24, N=4608, d=128) with inputs resident in
HBM.  Prints one JSON line: whole-step TOPS (4*B*H*N^2*d per step), the attention
kernel's matrix-core roofline fraction, the quantisation pass's HBM rate, the same
figures at N=8192, 16384, 32760 (40 heads) and 65536, and the CPU oracle timed on the
whole Flux-like workload.

Before the W warm-up steps of a timed window the step runs untimed for --warm-seconds
(default 0.5 s): the GPU's clocks ramp up over tens of milliseconds after an idle gap
(the host-side set-up between measurements), and a short window right after one reads
low.  The time spent is reported as "warm_s".

python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-seconds S] [--workload NAME]
                [--no-sweep] [--no-cpu-baseline] [--pmc-run] [--sparse-run WORKLOADS]
                [--modes-run WORKLOADS]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TOPS = 5000.0        # MI355X dense INT8 (POP/s) = dense FP8 (PFLOP/s), x1000
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
SWEEP = ["sweep8k", "sweep16k", "video", "stress"]
MODE_SWEEP = ["sweep16k", "stress"]   # sweep workloads the optional modes are also timed on
SWEEP_STEPS = 20          # timed steps per sweep workload
COPY_BYTES = 1 << 30      # calibration copy of the counter runs
ATTN_SOURCES = ["quantized_attention_diffusion_amd/csrc/sage_attn.hip",
                "quantized_attention_diffusion_amd/csrc/sage_device.h",
                "quantized_attention_diffusion_amd/csrc/sage_internal.h",
                "quantized_attention_diffusion_amd/csrc/sage_tiles.h",
                "quantized_attention_diffusion_amd/build.py"]          # its compiler flags


def attn_kernel_name(w, info):
    """The attention kernel the library launches for workload w (FP8 P.V, 64-token
    scales): the 32x32 body for d = 128, the 16x16 one for d = 64; the workgroup-pair
    priority instance when the grid is at most two rounds of two workgroups per compute
    unit, the plain one otherwise."""
    import torch
    grid = -(-w.N // info["block_m"]) * w.B * w.H
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    pair = "true" if grid <= 4 * cus else "false"
    return f"k_attn32<{pair}>" if w.d == 128 else f"k_attn<{w.d}, 0, false, false, {pair}>"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="untimed steps for this long before the warm-up steps of each timed window")
    ap.add_argument("--workload", default="flux_like")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-run", action="store_true",
                    help="only run the short program that the rocprofv3 counter runs profile")
    ap.add_argument("--sparse-run", metavar="WORKLOADS", default=None,
                    help="only run the block-sparse step a few times at each bench density on "
                         "the comma-separated workloads (the program a rocprofv3 kernel trace "
                         "of the tile selection profiles)")
    ap.add_argument("--modes-run", metavar="WORKLOADS", default=None,
                    help="only run each optional mode's step a few times on the comma-separated "
                         "workloads (the program a rocprofv3 kernel trace of the mode kernels profiles)")
    return ap.parse_args()


def quant_bytes(w) -> float:
    """Algorithmic bytes of the quantisation pass: read Q, K, V once (bf16), write the
    INT8 Q/K and FP8 V codes once; scales and means are < 0.1% and not counted."""
    E = w.B * w.H * w.N * w.d
    return 9.0 * E


# the optional modes of sage_attn_fwd_ex that the bench times (whole step)
MODES = {"bf16_pv": dict(pv="bf16"),
         "bf16_pv_per_token": dict(pv="bf16", per_token=True),
         "fp8_pv_block_mean_k": dict(pv="fp8", k_block_mean=True)}


def warm(fn, seconds: float) -> float:
    """Runs fn untimed until `seconds` have passed (synchronising every 20 calls);
    returns the time spent."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


WARM_S = 0.5              # set from --warm-seconds
EVICT_BYTES = 512 << 20   # read before each cold-cache quantisation call
COLD_REPS = 9
CPU_SHARE = 16            # worker processes at most: the host-core share of one GPU


def measure_mode(w, steps, warmup, **opts):
    """Whole-step time of sage_attn_fwd_ex with options ``opts`` on workload w."""
    import torch
    import workloads
    import quantized_attention_diffusion_amd as sage

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workloads.make_qkv(w))
    out = torch.empty_like(q)
    mode = sage.mode_bits(**opts)
    ws = torch.empty(sage.sage_workspace_bytes_ex(w.B, w.H, w.N, w.d, mode), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    warm(lambda: sage.sage_attn_fwd_ex(q, k, v, out=out, workspace=ws, **opts), WARM_S)
    for _ in range(warmup):
        sage.sage_attn_fwd_ex(q, k, v, out=out, workspace=ws, **opts)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        sage.sage_attn_fwd_ex(q, k, v, out=out, workspace=ws, **opts)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return {"N": w.N, "ms_per_step": round(ms, 4), "tops": round(w.ops / (ms * 1e-3) / 1e12, 2)}


# densities of the block-sparse path that the bench times (whole step)
SPARSE_DENSITIES = (0.5, 0.25)


def measure_sparse(w, steps, warmup, density):
    """Whole-step time of sage_attn_fwd_sparse at ``density`` on workload w.  ``tops`` is
    dense-equivalent (4*B*H*N^2*d over the step time); ``kept`` is the fraction of key
    tiles each query block visits and ``tops_executed`` counts only those."""
    import math
    import torch
    import workloads
    import quantized_attention_diffusion_amd as sage

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workloads.make_qkv(w))
    out = torch.empty_like(q)
    ws = torch.empty(sage.sage_workspace_bytes_sparse(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    warm(lambda: sage.sage_attn_fwd_sparse(q, k, v, density, out=out, workspace=ws), WARM_S)
    for _ in range(warmup):
        sage.sage_attn_fwd_sparse(q, k, v, density, out=out, workspace=ws)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        sage.sage_attn_fwd_sparse(q, k, v, density, out=out, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    nt = sage.sage_padded_tokens(w.N) // sage.sage_kernel_info()["kv_tile"]
    kept = max(1, min(nt, math.ceil(density * nt))) / nt
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return {"N": w.N, "density": density, "kept": round(kept, 4), "ms_per_step": round(ms, 4),
            "tops": round(w.ops / (ms * 1e-3) / 1e12, 2),
            "tops_executed": round(kept * w.ops / (ms * 1e-3) / 1e12, 2)}


def measure(w, steps, warmup):
    import torch
    import workloads
    import quantized_attention_diffusion_amd as sage

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workloads.make_qkv(w))
    out = torch.empty_like(q)
    ws = torch.empty(sage.sage_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # whole step
    warm_s = warm(lambda: sage.sage_attn_fwd(q, k, v, out=out, workspace=ws), WARM_S)
    for _ in range(warmup):
        sage.sage_attn_fwd(q, k, v, out=out, workspace=ws)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(steps):
        sage.sage_attn_fwd(q, k, v, out=out, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / steps

    # the two passes alone, each timed with events on the stream the library uses
    quant = sage.sage_quant_qk(q, k, v)
    warm(lambda: (sage.sage_quant_qk(q, k, v, out=quant), sage.sage_attn_fwd_prequant(quant, out=out)), WARM_S)
    for _ in range(warmup):
        sage.sage_quant_qk(q, k, v, out=quant)
        sage.sage_attn_fwd_prequant(quant, out=out)
    torch.cuda.synchronize(dev)
    e0, e1, e2, e3 = ev(), ev(), ev(), ev()
    e0.record(stream)
    for _ in range(steps):
        sage.sage_quant_qk(q, k, v, out=quant)
    e1.record(stream)
    e2.record(stream)
    for _ in range(steps):
        sage.sage_attn_fwd_prequant(quant, out=out)
    e3.record(stream)
    torch.cuda.synchronize(dev)
    quant_ms = e0.elapsed_time(e1) / steps
    attn_ms = e2.elapsed_time(e3) / steps
    # the quantisation pass with a cold memory-side cache: 512 MiB (twice the chip's
    # 256 MiB cache) read before each timed call (read, not written, so that the cache
    # then holds clean lines and the timed call pays no write-backs of other data);
    # median over COLD_REPS calls
    evict = torch.ones(EVICT_BYTES // 4, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(COLD_REPS):
        evict.sum()
        e0.record(stream)
        sage.sage_quant_qk(q, k, v, out=quant)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        cold.append(e0.elapsed_time(e1))
    quant_cold_ms = sorted(cold)[len(cold) // 2]
    del q, k, v, out, ws, quant, evict
    torch.cuda.empty_cache()
    return dict(step_ms=step_ms, wall_s=wall, quant_ms=quant_ms, attn_ms=attn_ms, warm_s=warm_s,
                quant_cold_ms=quant_cold_ms, quant_cold_gbs=quant_bytes(w) / (quant_cold_ms * 1e-3) / 1e9,
                tops=w.ops / (step_ms * 1e-3) / 1e12,
                attn_tops=w.ops / (attn_ms * 1e-3) / 1e12,
                quant_gbs=quant_bytes(w) / (quant_ms * 1e-3) / 1e9)


def _oracle_rows_worker(args):
    """One worker of the CPU baseline: rebuilds the seeded inputs and their oracle
    quantisation (untimed set-up), then times the oracle's quantised attention of its
    share of the sampled query rows in every head."""
    name, rows = args
    import numpy as np
    import oracle
    import workloads
    from threadpoolctl import threadpool_limits

    w = workloads.get(name)
    with threadpool_limits(limits=1):
        q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
        quant = oracle.quantize(q, k, v)
        t0 = time.perf_counter()
        oracle.attention_pipeline(q, k, v, kv_tile=128, rows=np.asarray(rows), quant=quant)
        return time.perf_counter() - t0


def cpu_baseline(w, rows_total: int | None = None):
    """The CPU oracle (numpy) on the workload: the full quantisation of Q, K and V on
    one core, then the quantised attention of ``rows_total`` query rows (default: all
    of them) in every head, split over one worker process per host core, each with one
    BLAS thread.  With a sample of rows the time is scaled to the whole workload
    linearly in rows (rows are independent given the quantised K and V)."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np
    import oracle
    import workloads
    from threadpoolctl import threadpool_limits

    cores = max(1, min(CPU_SHARE, len(os.sched_getaffinity(0))))
    q, k, v = (t.float().numpy() for t in workloads.make_qkv(w))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.quantize(q, k, v)
        t_quant = time.perf_counter() - t0
    del q, k, v
    rows_total = w.N if rows_total is None else min(rows_total, w.N)
    rows = np.linspace(0, w.N - 1, rows_total).astype(np.int64)
    shares = [rows[i::cores].tolist() for i in range(cores)]
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        times = list(ex.map(_oracle_rows_worker, [(w.name, s) for s in shares]))
    t_rows = max(times)                      # the workers run concurrently
    est = t_quant + t_rows * w.N / rows_total
    return {"value": round(w.ops / est / 1e12, 8), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": (f"{w.name}: full quantisation on 1 core ({t_quant:.1f} s), then attention of "
                       f"{rows_total} of {w.N} query rows in all {w.H} heads split over {cores} "
                       f"processes ({t_rows:.1f} s wall, {sum(times):.1f} s CPU)"
                       + (f"; scaled by rows to {est:.0f} s per step" if rows_total < w.N else
                          f": {est:.1f} s per step") + "; numpy, 1 BLAS thread per process")}


def _code_tokens(text: str) -> str:
    """The text with C/C++ and Python comments removed and whitespace collapsed, so that
    an edit of a comment does not count as a change of the kernel."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)         # block comments
    text = re.sub(r"//[^\n]*", " ", text)                      # line comments
    text = re.sub(r"(?m)^\s*#(?!\s*(include|define|pragma|if|else|elif|endif|ifdef|ifndef|undef)\b)[^\n]*", " ",
                  text)                                         # Python comment lines
    text = re.sub(r'"""(.*?)"""', " ", text, flags=re.S)        # Python docstrings
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the sources and build flags that define the attention kernel (their code
    without comments); a recorded traffic figure is used only while it matches."""
    import hashlib

    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a device
    copy of known size), or None when there is none for this workload or the kernel
    source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"attn_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-record:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("source_hash") == kernel_source_hash():
                    return rec
    return None


def pmc_run(w, reps: int = 3):
    """Short program for rocprofv3 counter runs: a 1 GiB elementwise copy kernel
    (calibrates the byte counters against a known size), then ``reps`` quantisation
    passes and ``reps`` attention launches on the workload."""
    import torch
    import workloads
    import quantized_attention_diffusion_amd as sage

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)        # an elementwise kernel: reads and writes COPY_BYTES
    torch.cuda.synchronize(dev)
    q, k, v = (t.to(dev) for t in workloads.make_qkv(w))
    quant = sage.sage_quant_qk(q, k, v)
    out = torch.empty_like(q)
    for _ in range(reps):
        sage.sage_quant_qk(q, k, v, out=quant)
    torch.cuda.synchronize(dev)
    for _ in range(reps):
        sage.sage_attn_fwd_prequant(quant, out=out)
    torch.cuda.synchronize(dev)
    print(f"[bench] pmc run done: copy {COPY_BYTES} B x{reps}, quant x{reps}, attention x{reps}",
          file=sys.stderr, flush=True)


def sparse_run(names: str):
    """Block-sparse steps for a kernel trace: per workload and density of
    SPARSE_DENSITIES, 5 steps (3 at 64K tokens and more) into a preallocated workspace."""
    import torch
    import workloads
    import quantized_attention_diffusion_amd as sage

    for name in names.split(","):
        w = workloads.get(name)
        q, k, v = (t.cuda() for t in workloads.make_qkv(w))
        out = torch.empty_like(q)
        ws = torch.empty(sage.sage_workspace_bytes_sparse(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
        for dens in SPARSE_DENSITIES:
            for _ in range(5 if w.N < 60000 else 3):
                sage.sage_attn_fwd_sparse(q, k, v, dens, out=out, workspace=ws)
            torch.cuda.synchronize()
            print(f"[bench] sparse run {name} density {dens} done", file=sys.stderr, flush=True)
        del q, k, v, out, ws
        torch.cuda.empty_cache()


def modes_run(names: str):
    """Steps of each optional mode (MODES, then FP8 P.V with per-token scales) for a
    kernel trace: per workload and mode, untimed steps for 0.3 s (clocks up), then 5
    steps (3 at 64K tokens and more) into a preallocated workspace."""
    import torch
    import workloads
    import quantized_attention_diffusion_amd as sage

    modes = dict(MODES, fp8_pv_per_token=dict(pv="fp8", per_token=True))
    for name in names.split(","):
        w = workloads.get(name)
        q, k, v = (t.cuda() for t in workloads.make_qkv(w))
        out = torch.empty_like(q)
        for mname, opts in modes.items():
            mode = sage.mode_bits(opts.get("pv", "fp8"), opts.get("per_token", False), opts.get("k_block_mean", False))
            ws = torch.empty(sage.sage_workspace_bytes_ex(w.B, w.H, w.N, w.d, mode), dtype=torch.uint8, device="cuda")
            warm(lambda: sage.sage_attn_fwd_ex(q, k, v, out=out, workspace=ws, **opts), 0.3)
            for _ in range(5 if w.N < 60000 else 3):
                sage.sage_attn_fwd_ex(q, k, v, out=out, workspace=ws, **opts)
            torch.cuda.synchronize()
            print(f"[bench] modes run {name} {mname} done", file=sys.stderr, flush=True)
            del ws
        del q, k, v, out
        torch.cuda.empty_cache()


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); across GPUs the "
              "heads would be sharded, each GPU running this step on its share with no "
              "communication.", file=sys.stderr)
        sys.exit(2)
    import workloads

    global WARM_S
    WARM_S = max(0.0, args.warm_seconds)
    w = workloads.get(args.workload)
    # The CPU baseline runs first, in worker processes started before this process
    # touches the GPU.
    cpu = None
    if not args.no_cpu_baseline and not args.pmc_run and not args.sparse_run and not args.modes_run:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)
        print(f"[bench] cpu baseline done: {cpu['sample']}", file=sys.stderr, flush=True)

    import torch
    import quantized_attention_diffusion_amd as sage

    sage.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.pmc_run:
        pmc_run(w)
        return
    if args.sparse_run:
        sparse_run(args.sparse_run)
        return
    if args.modes_run:
        modes_run(args.modes_run)
        return
    # The longer sequences run first (they also bring the GPU to its working clocks);
    # the headline workload is timed last.
    sweep, quality = {}, {}
    if not args.no_sweep:
        for name in SWEEP:
            ws = workloads.get(name)
            print(f"[bench] sweep {name} N={ws.N}", file=sys.stderr, flush=True)
            rs = measure(ws, SWEEP_STEPS, 2)
            sweep[name] = {"N": ws.N, "H": ws.H, "ms_per_step": round(rs["step_ms"], 4),
                           "tops": round(rs["tops"], 2), "attn_ms": round(rs["attn_ms"], 4),
                           "attn_tops": round(rs["attn_tops"], 2),
                           "mfma_util": round(rs["attn_tops"] / PEAK_TOPS, 4),
                           "quant_ms": round(rs["quant_ms"], 4),
                           "quant_gbs": round(rs["quant_gbs"], 1),
                           "quant_cold_ms": round(rs["quant_cold_ms"], 4),
                           "quant_cold_gbs": round(rs["quant_cold_gbs"], 1)}
        for name in MODE_SWEEP + [w.name]:
            wq = workloads.get(name)
            print(f"[bench] optional modes {name} N={wq.N}", file=sys.stderr, flush=True)
            st, wu = (args.steps, args.warmup) if name == w.name else (SWEEP_STEPS, 2)
            quality[name] = {mname: measure_mode(wq, st, wu, **opts) for mname, opts in MODES.items()}
            for dens in SPARSE_DENSITIES:
                quality[name][f"sparse_{dens}"] = measure_sparse(wq, st, wu, dens)
    print(f"[bench] {w.name} B={w.B} H={w.H} N={w.N} d={w.d}: {args.warmup} warmup + {args.steps} steps",
          file=sys.stderr, flush=True)
    r = measure(w, args.steps, args.warmup)
    info = sage.sage_kernel_info()
    traffic = recorded_traffic(w.name)
    line = {
        "metric": "quantized-attention TOPS (4*B*H*N^2*d per step: quantisation + attention)",
        "value": round(r["tops"], 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_s": round(r["warm_s"], 3),
        "ms_per_step": round(r["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 QK^T + fp8 PV (fp32 softmax, bf16 io)",
        "data": "synthetic (seeded N(0,1) Q/V, K with N(0,9) channel bias)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "kv_tile": info["kv_tile"], "block_m": info["block_m"]},
        "attn_only": {"ms": round(r["attn_ms"], 5), "tops": round(r["attn_tops"], 2),
                      "mfma_util": round(r["attn_tops"] / PEAK_TOPS, 4)},
        "quant_only": {"ms": round(r["quant_ms"], 5), "gbs": round(r["quant_gbs"], 1),
                       "hbm_frac": round(r["quant_gbs"] / PEAK_HBM_GBS, 4),
                       "cold_ms": round(r["quant_cold_ms"], 5), "cold_gbs": round(r["quant_cold_gbs"], 1),
                       "cold_hbm_frac": round(r["quant_cold_gbs"] / PEAK_HBM_GBS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(r["attn_tops"], 2), "peak": PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": round(r["attn_tops"] / PEAK_TOPS, 4),
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "kernel": attn_kernel_name(w, info),
                     "algorithmic_bytes": 5 * w.B * w.H * w.N * w.d},
        "sweep": sweep,
        "modes": quality,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
