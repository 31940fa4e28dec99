"""Benchmark: C = A*A for R-MAT scale 18, edge factor 16 (262,144 x 262,144),
with R-MAT scale 20, edge factor 8 (1,048,576 x 1,048,576) as a second full
record in the same line.

One step is the whole hot path: spgemm_symbolic + spgemm_numeric (setup,
InterOffsets, binning, the heavy rows' chunk counts and split, light rows,
accumulation of every (heavy row, chunk), prefix sums), on inputs already
resident in HBM, with the library's default options. Protocol after the
gMAGNUS page (Section IV-A): warmup runs, then timed runs, mean reported.
Prints one JSON line.

paths = the same product with the page's own numeric dataflows (outer
        product into C-hat then multisplit; the first multisplit level
        formed in its tiles), a few steps each, with each phase's
        algorithmic GB/s and fraction of the HBM peak

value  = intermediate products per second (sum of u(i) over all rows / step time)
roofline = the dominant kernel's algorithmic bytes per launch / its mean
           launch time (HIP events recorded by the library on the stream the
           kernel runs on), against MI355X's 8 TB/s HBM peak
cpu_baseline = the CPU oracle on a bounded row sample of the same product,
           plus one-thread oracle rates on the two small workloads
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="rmat18_ef16")
    ap.add_argument("--also", default="rmat20_ef8",
                    help="comma-separated workloads timed after the headline one, each a full "
                         "record under 'workloads' ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paths", action="store_true",
                    help="skip timing the other numeric paths (separate C-hat, fused first level)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--tau", type=int, default=0)
    ap.add_argument("--width", type=int, default=0)
    ap.add_argument("--cap", type=int, default=0)
    ap.add_argument("--max-batch-products", type=int, default=0,
                    help="heavy products per row batch of the C-hat dataflows (0: one batch)")
    ap.add_argument("--numeric-mode", type=int, default=0, choices=(0, 1, 2, 3),
                    help="heavy numeric dataflow of the timed steps: 0 the library's choice "
                         "(direct), 1 fused first level, 2 separate C-hat (the page's), 3 direct")
    ap.add_argument("--pairs", action="store_true",
                    help="time the gMAGNUS page's RMat set instead (Table III: independent A, B "
                         "of scales 15-20, A.nnz/A.n 4..32, B.nnz/B.n 8); one line with every pair")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    return ap.parse_args()


def copy_rate_GBps(mib: int = 2048) -> float:
    """Read + write bytes per second of a plain streaming elementwise kernel
    over mib MiB: the measured speed of light that the gMAGNUS page reports
    its kernels against (Section IV-C), next to the nominal HBM peak."""
    import torch
    n = mib * (1 << 20) // 8
    src = torch.empty(n, dtype=torch.float64, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        torch.add(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 8 / (ms * 1e-3) / 1e9


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(mib: int):
    """A plain device copy of known size.

    HBM counters read on it scale the counters of the other kernels, and its
    rate is the measured speed of light (read + write bytes per second) that
    the gMAGNUS page uses as the kernels' peak (Section IV-C).
    """
    import torch
    n = mib * (1 << 20) // 8
    src = torch.empty(n, dtype=torch.float64, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    # a plain streaming elementwise kernel: reads n*8 bytes, writes n*8 bytes
    torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record()
    for _ in range(reps):
        torch.add(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_calibration_bytes_each_way": n * 8, "launches": reps + 1,
                      "copy_ms": ms, "copy_GBps_read_plus_write": 2 * n * 8 / (ms * 1e-3) / 1e9}))
    # the same streaming add on 2-byte elements (the split B's columns are 2 bytes)
    s16 = src.view(torch.int16)
    d16 = dst.view(torch.int16)
    torch.add(s16, 1, out=d16)
    torch.cuda.synchronize()
    # isolated gathers: one element from each of ng distinct random 256-byte
    # blocks of the 2 GiB buffer (far larger than the caches), from 8-byte and
    # from 2-byte data; the indices themselves are read in a stream (8 B each)
    blocks = (n * 8) // 256
    ng = min(1 << 22, blocks // 2)
    g = torch.Generator(device="cpu").manual_seed(7)
    sel = torch.randperm(blocks, generator=g)[:ng].sort().values
    idx64 = (sel * 32).to("cuda")   # float64 element at the start of the block
    idx16 = (sel * 128).to("cuda")  # int16 element at the start of the block
    torch.cuda.synchronize()
    out64 = torch.take(src, idx64)
    out16 = torch.take(s16, idx16)
    torch.cuda.synchronize()
    print(json.dumps({"int16_add_bytes_each_way": n * 8,
                      "gather_elements": ng, "gather_index_bytes": ng * 8,
                      "gather_f64_useful_bytes": ng * 8, "gather_i16_useful_bytes": ng * 2,
                      "dispatch_order": ["fill", "add f64 x4", "add i16", "take f64", "take i16"],
                      "check": float(out64.sum().item()) + float(out16.sum().item())}))


# kernels behind each timed phase, for the HBM traffic the counters measured
PHASE_KERNELS = {
    "numeric:multisplit": ["k_multisplit<true,"],
    "numeric:outer_prod": ["k_expand<true>"],
    "numeric:heavy_accum": ["k_chunk_window<true", "k_acc_rank<true,", "k_acc_hash<1,true,"],
    "numeric:direct_dense": ["k_direct_window"],
    "numeric:direct_rank": ["k_direct_rank<", "k_gather_bval"],
}
HEAVY_PHASES = ("outer_prod", "multisplit", "heavy_accum", "histo", "direct_dense", "direct_rank")


def measured_traffic(workload: str, phase: str):
    """HBM bytes per launch of a phase's kernels from profiles/hbm_traffic_<workload>.txt.

    The file holds FETCH_SIZE and WRITE_SIZE per dispatch (already scaled by the
    plain-copy calibration) together with a hash of the kernel's source file;
    a kernel whose source changed since is not reported (None).
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    prefixes = PHASE_KERNELS.get(phase)
    if not prefixes or not os.path.exists(path):
        return None
    total, found = 0, False
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        name, wl, src, digest, fetch, write = line.split()
        if wl != workload or not any(name.startswith(p) for p in prefixes):
            continue
        src_path = os.path.join(ROOT, "spgemm_irregular_matrices_amd", "csrc", src)
        now = hashlib.sha256(open(src_path, "rb").read()).hexdigest()[:16]
        if now != digest:
            return None
        total += int(fetch) + int(write)
        found = True
    return total if found else None


def _phase_fracs(per_phase: dict, steps: int) -> dict:
    """ms per step, algorithmic GB/s and fraction of the HBM peak of every timed phase."""
    out = {}
    for k, v in per_phase.items():
        if not v["launches"]:
            continue
        rec = {"ms_per_step": v["ms"] / steps}
        if v["bytes"] > 0 and v["ms"] > 0:
            gbps = v["bytes"] / (v["ms"] * 1e-3) / 1e9
            rec["algorithmic_GBps"] = gbps
            rec["frac"] = gbps / HBM_PEAK_GBS
        out[f"{k[0]}:{k[1]}"] = rec
    return out


def _accumulate(per_phase: dict, st: dict):
    for pn in ("symbolic", "numeric"):
        for ph, rec in st[pn].items():
            d = per_phase.setdefault((pn, ph), {"ms": 0.0, "launches": 0, "bytes": 0.0})
            d["ms"] += rec["ms"]
            d["launches"] += rec["launches"]
            d["bytes"] += rec["bytes"]


def time_numeric_path(dA, dB, numeric_mode: int, steps: int, max_batch_products: int = 0) -> dict:
    """Mean step time of the same product with another heavy numeric path, and
    each phase's algorithmic GB/s (the page's kernels: outer product,
    histogram, multisplit, accumulation)."""
    import torch
    from spgemm_irregular_matrices_amd import binding
    with binding.Plan(timing=True, numeric_mode=numeric_mode,
                      max_batch_products=max_batch_products) as plan:
        def step():
            rp, nnz = plan.symbolic(dA, dB)
            col = torch.empty(nnz, dtype=torch.int32, device="cuda")
            val = torch.empty(nnz, dtype=torch.float64, device="cuda")
            plan.numeric(dA, dB, rp, col, val)
        step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        per_phase = {}
        for _ in range(steps):
            step()
            st = plan.stats()
            _accumulate(per_phase, st)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
    torch.cuda.empty_cache()
    heavy_bytes = sum(v["bytes"] for k, v in per_phase.items() if k[1] in HEAVY_PHASES)
    heavy_ms = sum(v["ms"] for k, v in per_phase.items() if k[1] in HEAVY_PHASES)
    return {"ms_per_step": ms, "numeric_path": st["numeric_path"], "row_batches": st["nbatches"],
            "vchunks": st["vchunks"],
            "heavy_path": {"ms_per_step": heavy_ms / steps,
                           "frac": (heavy_bytes / (heavy_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
                           if heavy_ms else 0},
            "phases": {k: v for k, v in _phase_fracs(per_phase, steps).items()
                       if v["ms_per_step"] >= 0.05}}


def host_threads():
    """(threads the oracle uses, cores this process may run on).

    A one-GPU machine gives the process a share of 16 host threads whatever the
    affinity mask shows, so the oracle uses at most 16."""
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:
        visible = os.cpu_count() or 1
    return max(1, min(visible, 16)), visible


def cpu_baseline(A, B, target_s: float):
    """Time the oracle on an evenly spaced row sample sized for ~target_s seconds."""
    import oracle

    oracle.build(force=False)
    cores, visible = host_threads()
    u = oracle.row_products(A, B)
    total = int(u.sum())
    frac = 1.0 / 4096
    while True:
        step = max(1, int(round(1.0 / frac)))
        rows = np.arange(0, A.nrows, step, dtype=np.int64)
        t0 = time.perf_counter()
        oracle.spgemm_rows(A, B, rows, nthreads=cores)
        dt = time.perf_counter() - t0
        prods = int(u[rows].sum())
        if dt >= target_s * 0.5 or step == 1:
            break
        frac = min(1.0, frac * max(2.0, min(16.0, target_s / max(dt, 1e-3))))
    return {"value": prods / dt, "unit": "products/s", "cores": cores, "cores_visible": visible,
            "kind": "oracle",
            "sample": f"one row of C in every {step} ({rows.size} rows, {prods} of {total} products)",
            "seconds": dt, "gflops": 2.0 * prods / dt / 1e9, "cpu_model": cpu_model()}


def oracle_one_thread():
    """The oracle on one thread for the two small workloads: every row of the
    1024^2 R-MAT square (best of 3), one row in 16 of the 2^20 banded square."""
    import oracle
    from spgemm_irregular_matrices_amd import synth

    out = {}
    for name, step, reps in (("rmat10_ef8", 1, 3), ("banded_n1M_17diag", 16, 1)):
        A, B = synth.workload(name)
        u = oracle.row_products(A, B)
        rows = np.arange(0, A.nrows, step, dtype=np.int64)
        best = None
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.spgemm_rows(A, B, rows, nthreads=1)
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        prods = int(u[rows].sum())
        out[name] = {"value": prods / best, "unit": "products/s", "seconds": best,
                     "sample": "every row, best of 3" if step == 1 else f"one row in {step}"}
    return out


def bench_workload(name: str, args, copy_gbps: float, with_paths: bool, with_cpu: bool) -> dict:
    """Time `args.steps` steps of one workload; returns its full record."""
    import torch

    from spgemm_irregular_matrices_amd import binding, synth

    A, B = synth.workload(name)
    dA = binding.DeviceCSR.from_host(A)
    dB = dA if B is A else binding.DeviceCSR.from_host(B)
    torch.cuda.synchronize()

    plan = binding.Plan(timing=True, tau_override=args.tau, chunk_width_override=args.width,
                        nchunks_cap=args.cap, numeric_mode=args.numeric_mode,
                        max_batch_products=args.max_batch_products)

    def step():
        rp, nnz = plan.symbolic(dA, dB)
        col = torch.empty(nnz, dtype=torch.int32, device="cuda")
        val = torch.empty(nnz, dtype=torch.float64, device="cuda")
        plan.numeric(dA, dB, rp, col, val)
        return rp, col, val

    for _ in range(args.warmup):
        out = step()
        del out
    torch.cuda.synchronize()

    per_phase = {}
    step_ms = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ts = time.perf_counter()
        out = step()
        st = plan.stats()   # waits for this step's events
        step_ms.append((time.perf_counter() - ts) * 1e3)
        _accumulate(per_phase, st)
        del out
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3

    products = st["sum_products"]
    value = products * args.steps / elapsed

    # dominant kernel by measured time: of the heavy path when there is one
    # (the numeric light rows run on a second stream beside it, so their
    # phase window spans heavy work too), else of the light rows
    cands = [k for k in per_phase if k[1] in HEAVY_PHASES and per_phase[k]["launches"]]
    if not cands:
        cands = [k for k in per_phase if k[1] == "light_accum"]
    dom = max(cands, key=lambda k: per_phase[k]["ms"])
    d = per_phase[dom]
    launch_ms = d["ms"] / max(d["launches"], 1)
    bytes_per_launch = d["bytes"] / max(d["launches"], 1)
    achieved = bytes_per_launch / (launch_ms * 1e-3) / 1e9 if launch_ms > 0 else 0.0
    traffic = measured_traffic(name, f"{dom[0]}:{dom[1]}")
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": f"{dom[0]}:{dom[1]}", "launch_ms": launch_ms,
                "bytes_per_launch": bytes_per_launch,
                "measured_copy_GBps": copy_gbps, "frac_of_measured_copy": achieved / copy_gbps}
    heavy_bytes = sum(v["bytes"] for k, v in per_phase.items() if k[1] in HEAVY_PHASES)
    heavy_ms = sum(v["ms"] for k, v in per_phase.items() if k[1] in HEAVY_PHASES)
    plan.close()

    paths = None
    if with_paths:
        # the page's dataflows on the same product: outer product into C-hat
        # then multisplit (in one batch, and in batches of at most 2^31 - 1
        # products where C-hat holds more), and the first level formed in the
        # multisplit tiles
        paths = {"separate_chat": time_numeric_path(dA, dB, 2, 3),
                 "fused_first_level": time_numeric_path(dA, dB, 1, 3)}
        if st["heavy_products"] > (1 << 31) - 1 and name == "rmat20_ef8":
            paths["separate_chat_batched"] = time_numeric_path(dA, dB, 2, 3, (1 << 31) - 1)
    del dA, dB
    torch.cuda.empty_cache()

    cpu = cpu_baseline(A, B, args.cpu_seconds) if with_cpu else None
    phases = _phase_fracs(per_phase, args.steps)
    return {
        "value": value, "unit": "products/s", "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms,
        "config": {"workload": name, "description": synth.describe(name),
                   "nrows": A.nrows, "nnz_A": A.nnz, "sum_products": products,
                   "nnz_C": st["nnz_c"], "heavy_rows": st["heavy_rows"],
                   "heavy_products": st["heavy_products"], "tau": st["tau"],
                   "vchunks": st["vchunks"], "final_chunk_width": st["final_chunk_width"],
                   "row_batches": st["nbatches"],
                   "numeric_path": {0: "none", 1: "fused first level", 2: "separate C-hat",
                                    3: "direct"}[st["numeric_path"]]},
        "gflops": 2.0 * value / 1e9,
        "roofline": roofline,
        "heavy_path": {"ms_per_step": heavy_ms / args.steps,
                       "algorithmic_GBps": heavy_bytes / (heavy_ms * 1e-3) / 1e9 if heavy_ms else 0,
                       "frac": (heavy_bytes / (heavy_ms * 1e-3) / 1e9 / HBM_PEAK_GBS) if heavy_ms else 0},
        "phase_ms_per_step": {k: v["ms_per_step"] for k, v in phases.items()},
        # algorithmic bytes of a phase over its measured time (phases that count bytes)
        "phase_algorithmic_GBps": {k: v["algorithmic_GBps"] for k, v in phases.items()
                                   if "algorithmic_GBps" in v},
        "phase_frac": {k: v["frac"] for k, v in phases.items() if "frac" in v},
        "step_ms_min_max": [min(step_ms), max(step_ms)],
        "cpu_baseline": cpu,
        "paths": paths,
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library runs one product on one GPU", file=sys.stderr)
        sys.exit(2)
    import torch

    from spgemm_irregular_matrices_amd import binding

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load()
    copy_gbps = copy_rate_GBps()
    if args.pairs:
        from spgemm_irregular_matrices_amd import synth
        pairs = []
        for s, a in synth.TABLE3_CELLS:
            r = bench_workload(synth.pair_name(s, a), args, copy_gbps, False, False)
            c = r["config"]
            pairs.append({"scale": s, "a_density": a, "b_density": 8, "ms_per_step": r["ms_per_step"],
                          "products_per_s": r["value"], "gflops": r["gflops"],
                          "sum_products": c["sum_products"], "nnz_C": c["nnz_C"],
                          "C_per_row": c["nnz_C"] / c["nrows"],
                          "C_hat_per_row": c["sum_products"] / c["nrows"],
                          "heavy_rows": c["heavy_rows"], "numeric_path": c["numeric_path"],
                          "heavy_path_frac": r["heavy_path"]["frac"],
                          "dominant": r["roofline"]["kernel"], "dominant_frac": r["roofline"]["frac"]})
            print(json.dumps({"pair": pairs[-1]}), file=sys.stderr, flush=True)
        print(json.dumps({"metric": "SpGEMM intermediate products/s, R-MAT A*B pairs (Table III set)",
                          "unit": "products/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "dtype": "f64", "data": "synthetic",
                          "pairs": pairs}))
        return
    head = bench_workload(args.workload, args, copy_gbps, not args.no_paths,
                          not args.no_cpu_baseline)
    others = {}
    for name in [w for w in args.also.split(",") if w and w != args.workload]:
        others[name] = bench_workload(name, args, copy_gbps, not args.no_paths,
                                      not args.no_cpu_baseline)
    if head["cpu_baseline"] is not None:
        head["cpu_baseline"]["one_thread"] = oracle_one_thread()

    line = {
        "metric": "SpGEMM intermediate products/s (GFLOP/s) and HBM GB/s fraction, R-MAT A*A",
        "value": head["value"], "unit": "products/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
    }
    for k, v in head.items():
        if k not in line:
            line[k] = v
    if others:
        line["workloads"] = others
    print(json.dumps(line))


if __name__ == "__main__":
    main()
