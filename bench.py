"""Benchmark of the DSA forward hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
lightning-indexer scores -> per-query top-k -> sparse MLA (absorbed latent
form), enqueued through the C ABI on the current stream.  The default
workload is batch-32 decode at 131072-token context (one new query per
sequence, 128-head MLA over its 2048 selected latent rows).

Prints one JSON line: throughput in queries/s over the timed steps (inputs
resident in HBM), the roofline position of the dominant kernel measured with
HIP events on the launch stream, and the CPU oracle timed on a bounded sample
of the same workload.  Timed steps call the fused entry point where the
workload has one; every few steps (at least five per run) run the stages as separate calls with
events between them, which gives each kernel's duration inside the timed
region.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--fp8-indexer]
  python bench.py --calib-copy     (plain 1 GiB device copy, for counter scaling)
  python bench.py --next projections|paged|compressed
                                   (the calls built beside the path, timed with HIP events)
  python bench.py --record-traffic --workload NAME --pmc-fetch F.csv --pmc-write W.csv
                  --calib-fetch CF.csv --calib-write CW.csv --commands "..."
                                   (store the dominant kernel's HBM bytes per launch)
  python bench.py --record-mfma --workload NAME --kernel K --pmc-mfma M.csv --pmc-util U.csv
                  --ktrace T.csv --commands "..."
                                   (store a matrix-core kernel's MFMA counters per launch)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA fwd queries/s (indexer+top-k+sparse MLA) at 128K ctx; % MFMA / % HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
DEFAULT_WORKLOAD = "dsa_decode_b32_128k"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true",
                    help="capture the fused step once in a HIP graph and replay it (workloads with a fused call)")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch size")
    ap.add_argument("--staged", action="store_true",
                    help="run every timed step as separate stage calls with HIP events between them")
    ap.add_argument("--fp8-indexer", action="store_true",
                    help="decode workloads: the FP8 indexer (key cache held as E4M3 codes; each step quantises "
                         "its queries, then scores)")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--next", choices=["projections", "paged", "compressed"],
                    help="time the calls built beside the path (one JSON line; not the headline)")
    ap.add_argument("--record-traffic", action="store_true",
                    help="store the dominant kernel's HBM traffic from four rocprofv3 -f csv counter files")
    ap.add_argument("--pmc-fetch")
    ap.add_argument("--pmc-write")
    ap.add_argument("--calib-fetch")
    ap.add_argument("--calib-write")
    ap.add_argument("--commands", default="", help="the rocprofv3 command lines, recorded with the traffic")
    ap.add_argument("--record-mfma", action="store_true",
                    help="store one kernel's matrix-core counters (rocprofv3 -f csv counter and kernel-trace files)")
    ap.add_argument("--kernel", help="--record-mfma: the kernel (name prefix)")
    ap.add_argument("--pmc-mfma", help="--record-mfma: counter file with SQ_INSTS_VALU_MFMA_MOPS_BF16, "
                    "SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, GRBM_GUI_ACTIVE")
    ap.add_argument("--pmc-util", help="--record-mfma: counter file with the derived MfmaUtil and LdsBankConflict")
    ap.add_argument("--ktrace", help="--record-mfma: kernel-trace file of the same run as --pmc-mfma")
    return ap.parse_args()


# Source files each timed kernel is built from: stored counter readings stay
# valid until the code of one of them changes (comments and layout aside).
KERNEL_SOURCES = {
    "indexer_dma_bf16": ["indexer.hip", "device_common.h", "select_common.h", "launch.h"],
    "indexer_tiled_bf16": ["indexer.hip", "device_common.h", "select_common.h", "launch.h"],
    "indexer_dma_fp8": ["indexer.hip", "device_common.h", "select_common.h", "launch.h"],
    "sparse_mla_bf16_kernel": ["sparse_mla.hip", "device_common.h"],
}


def code_only(text: str) -> str:
    """A C++ source without its comments, whitespace runs collapsed to one
    space: what the compiler sees of it (string and character literals kept
    whole)."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif text[i] in "\"'":
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_sources_digest(kernel: str) -> str:
    """Digest of the code of one kernel's HIP sources (comments and layout
    aside) and of their per-file compile flags."""
    from long_context_sparse_14_amd import build as _build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_sparse_14_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update((name + "\n" + code_only(f.read())).encode())
        h.update(" ".join(_build.EXTRA_FLAGS.get(name, [])).encode())
    return h.hexdigest()[:16]


def traffic_path(workload: str, kernel: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the rocprofv3 counter passes kept under profiles/,
    if they were taken on the current sources of that kernel."""
    path = traffic_path(workload, kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_digest") != kernel_sources_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_rows(csv_path: str, counter: str):
    """(kernel name, value) per dispatch for one counter of a rocprofv3 -f csv
    counter_collection file."""
    import csv
    out = []
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                out.append((row.get("Kernel_Name", ""), float(row["Counter_Value"])))
    if not out:
        raise SystemExit(f"{csv_path}: no {counter} rows")
    return out


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def record_traffic(args):
    """Turn four counter passes (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, over
    this benchmark and over the plain-copy calibration) into the stored HBM
    traffic of the dominant kernel."""
    import synth
    wl = synth.WORKLOADS[args.workload]
    _, kname, _, work, wunit = dominant_stage(wl, args.fp8_indexer)
    calib_bytes = 1 << 30

    def per_dispatch(csv_path, counter, name_part):
        vals = [v * 1024.0 for k, v in _pmc_rows(csv_path, counter) if name_part in k]
        if not vals:
            raise SystemExit(f"{csv_path}: no dispatch of a kernel matching {name_part!r}")
        return _median(vals), len(vals)

    cf, _ = per_dispatch(args.calib_fetch, "FETCH_SIZE", "copy")
    cw, _ = per_dispatch(args.calib_write, "WRITE_SIZE", "copy")
    kf, nf = per_dispatch(args.pmc_fetch, "FETCH_SIZE", kname)
    kw, nw = per_dispatch(args.pmc_write, "WRITE_SIZE", kname)
    f_scale, w_scale = calib_bytes / cf, calib_bytes / cw
    rec = {
        "workload": wl.name,
        "kernel": kname,
        "kernel_sources_digest": kernel_sources_digest(kname),
        "fetch_bytes_per_launch_raw": kf,
        "write_bytes_per_launch_raw": kw,
        "calib_copy_bytes": calib_bytes,
        "calib_fetch_bytes_raw": cf,
        "calib_write_bytes_raw": cw,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_bytes_per_launch": round(kf * f_scale + kw * w_scale),
        "algorithmic_work_per_launch": int(work),
        "algorithmic_unit": wunit,
        "dispatches": {"fetch": nf, "write": nw},
        "commands": args.commands,
    }
    with open(traffic_path(wl.name, kname), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def mfma_path(workload: str, kernel: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_mfma.json")


def kernel_flops(wl, kernel: str) -> int:
    """Algorithmic matrix flops of one launch of a matrix-core kernel on the whole workload."""
    B, Tq, N, q0, K = wl.B, wl.Tq, wl.N, wl.q_pos0, wl.K
    vis = [min(N, q0 + t + 1) for t in range(Tq)]
    if kernel.startswith("indexer"):
        return 2 * wl.H_I * wl.D_I * B * sum(vis)
    if kernel.startswith("sparse_mla"):
        return 2 * wl.H * (wl.D + wl.DV) * B * sum(min(v, K) for v in vis)
    raise SystemExit(f"no flop count for {kernel}")


def record_mfma(args):
    """One kernel's matrix-core counters per launch, from a rocprofv3 --pmc run
    (with its kernel trace) and a second run of the derived utilisation metrics:
    bf16 MFMA flops counted by the hardware (MOPS x 512) against the algorithmic
    count, the counted and algorithmic rates against the dense bf16 peak, and
    the profiler's MfmaUtil (matrix-core busy cycles per SIMD and active cycle)."""
    import csv

    import synth
    wl = synth.WORKLOADS[args.workload]
    kname = args.kernel

    import re
    named = re.compile(r"(?<![A-Za-z0-9_])" + re.escape(kname) + r"(?![A-Za-z0-9_])")

    def per_dispatch(path, counter):
        vals = [v for k, v in _pmc_rows(path, counter) if named.search(k)]
        if not vals:
            raise SystemExit(f"{path}: no {counter} for a kernel named {kname!r}")
        return _median(vals), len(vals)

    raw = {}
    for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT",
              "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"):
        raw[c], n = per_dispatch(args.pmc_mfma, c)
    util = {c: per_dispatch(args.pmc_util, c)[0] for c in ("MfmaUtil", "LdsBankConflict")}
    durs = []
    with open(args.ktrace, newline="") as f:
        for row in csv.DictReader(f):
            if named.search(row.get("Kernel_Name", "")):
                durs.append((float(row["End_Timestamp"]) - float(row["Start_Timestamp"])) * 1e-9)
    if not durs:
        raise SystemExit(f"{args.ktrace}: no dispatch of {kname}")
    sec = _median(durs)
    counted = raw["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
    algo = kernel_flops(wl, kname)
    rec = {
        "workload": wl.name,
        "kernel": kname,
        "kernel_sources_digest": kernel_sources_digest(kname),
        "dispatches": n,
        "kernel_us_median": round(sec * 1e6, 2),
        "counters_per_launch": raw,
        "derived_per_launch": util,
        "mfma_flops_counted": counted,
        "mfma_flops_algorithmic": algo,
        "counted_over_algorithmic": round(counted / algo, 4),
        "counted_tflops": round(counted / sec / 1e12, 1),
        "algorithmic_tflops": round(algo / sec / 1e12, 1),
        "peak_tflops": BF16_PEAK_TFLOPS,
        "frac_counted": round(counted / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
        "frac_algorithmic": round(algo / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
        "mfma_util_pct": round(util["MfmaUtil"], 2),
        "lds_bank_conflict_pct": round(util["LdsBankConflict"], 2),
        "lds_conflicts_per_access": round(raw["SQ_LDS_BANK_CONFLICT"] /
                                          max(1.0, raw["SQ_LDS_IDX_ACTIVE"] - raw["SQ_LDS_BANK_CONFLICT"]), 4),
        "commands": args.commands,
    }
    with open(mfma_path(wl.name, kname), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def stored_mfma(workload: str, kernel: str):
    """The stored matrix-core counter record of a kernel, if taken on its current sources."""
    path = mfma_path(workload, kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_digest") != kernel_sources_digest(kernel):
        return None
    return {k: rec[k] for k in ("frac_counted", "counted_over_algorithmic", "mfma_util_pct", "kernel_us_median")}


def dominant_stage(wl, fp8=False):
    """Stage that bounds the workload, its roofline and its algorithmic work per launch."""
    B, Tq, N, q0, K = wl.B, wl.Tq, wl.N, wl.q_pos0, wl.K
    vis = [min(N, q0 + t + 1) for t in range(Tq)]
    keys = B * sum(vis)                                  # (query, visible key) pairs
    sel = B * sum(min(v, K) for v in vis)                # (query, selected key) pairs
    if fp8:
        # FP8 decode indexer: each key's 128 code bytes and 4-byte scale read once, its fp32 score
        # written once, plus the query codes, scales and head weights
        nbytes = B * N * (wl.D_I + 4) + keys * 4 + B * Tq * wl.H_I * (wl.D_I + 4 + 2)
        return "index", "indexer_dma_fp8", "hbm", nbytes, "B"
    if "mla" in wl.stages and Tq > 4:
        # prefill: the sparse MLA (K selected rows x 128 heads x 1088 MACs each) dominates
        flops = 2 * wl.H * (wl.D + wl.DV) * sel
        return "mla", "sparse_mla_bf16_kernel", "mfma", flops, "flop"
    if "index" in wl.stages and Tq <= 4:
        # decode indexer: each visible key row (256 B) read once, its fp32 score written once
        nbytes = B * N * wl.D_I * 2 + keys * 4 + B * Tq * wl.H_I * (wl.D_I + 1) * 2
        return "index", "indexer_dma_bf16", "hbm", nbytes, "B"
    if "index" in wl.stages:
        flops = 2 * wl.H_I * wl.D_I * keys
        return "index", "indexer_tiled_bf16", "mfma", flops, "flop"
    if Tq <= 4:
        nbytes = sel * wl.D * 2 + B * Tq * wl.H * (wl.D + wl.DV) * 2 + B * Tq * K * 4
        return "mla", "sparse_mla_bf16_kernel", "hbm", nbytes, "B"
    flops = 2 * wl.H * (wl.D + wl.DV) * sel
    return "mla", "sparse_mla_bf16_kernel", "mfma", flops, "flop"


def calib_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 5}), flush=True)


def measured_ceilings(bound: str):
    """What this GPU sustains, measured in the same process before the timed
    steps (HIP events): a plain streaming read and a streaming copy of a
    1 GiB device buffer with the library's calibration kernel (16-byte
    accesses, the same kind as the HBM-bound kernels), and, for
    matrix-core-bound workloads, the rate of the vendor library's bf16 GEMM
    (torch.matmul on 8192^3, N(0,1) operands: dense bf16 matrix work is
    power-limited on this part, so realistic data runs well below the
    nominal peak)."""
    import torch

    import long_context_sparse_14_amd as dsa
    out = {}

    def rate(fn, reps):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    s = rate(lambda: dsa.calib_stream(a), 10)
    out["read_GBps"] = round(n / s / 1e9, 1)
    s = rate(lambda: dsa.calib_stream(a, b), 10)
    out["copy_GBps"] = round(2 * n / s / 1e9, 1)
    out["kernel"] = "dsa_calib_stream (16-byte streaming loads/stores, 1 GiB)"
    del a, b
    if bound == "mfma":
        g = torch.Generator(device="cuda")
        g.manual_seed(0)
        m = 8192
        x = torch.randn(m, m, device="cuda", generator=g).to(torch.bfloat16)
        y = torch.randn(m, m, device="cuda", generator=g).to(torch.bfloat16)
        z = torch.empty(m, m, device="cuda", dtype=torch.bfloat16)
        s = rate(lambda: torch.matmul(x, y, out=z), 10)
        out["library_gemm_bf16_TFLOPs"] = round(2 * m ** 3 / s / 1e12, 1)
    torch.cuda.empty_cache()
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _host_cpus() -> int:
    return os.cpu_count() or 1


def cpu_baseline(wl, x, budget_s: float):
    """The C++ oracle, as it stands, on whole queries of the same workload.

    Queries are taken in seeded random order, cycling over the workload's
    queries, in calls of one query per oracle thread (the oracle splits a
    call's queries over its threads), until the budget is spent."""
    import numpy as np

    import oracle

    nthreads = oracle.threads()
    rows = [(b, t) for b in range(wl.B) for t in range(wl.Tq)]
    order = np.random.default_rng(0).permutation(len(rows))
    done, calls = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 <= budget_s:
        sel = [rows[order[(done + i) % len(rows)]] for i in range(nthreads)]
        if "index" in wl.stages:
            oracle.forward_batch(x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], sel, wl.q_pos0, wl.K, wl.scale,
                                 wl.DV, want_scores=False)
        else:
            oracle.sparse_mla_batch(x["q"], x["kv"], x["idx"], sel, wl.scale, wl.DV)
        done += len(sel)
        calls += 1
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "queries/s", "cores": int(nthreads), "kind": "oracle",
            "host_cpus": _host_cpus(), "cpu_model": _cpu_model(),
            "sample": f"{done} queries of {wl.name} (whole path per query: indexer, top-k, sparse MLA), in {calls} "
                      f"calls of {nthreads}, cycling in seeded random order over its {len(rows)}, {el:.1f} s; "
                      f"C++ oracle, double, {nthreads} threads"}


def cpu_baseline_fp8(wl, x, budget_s: float, max_seqs: int = 4):
    """The C++ oracle's FP8 path on whole decode queries: the key caches of a few sequences are
    quantised first (untimed: the cache is held as codes); each timed call quantises one query per
    oracle thread, scores, selects and attends."""
    import numpy as np

    import oracle

    nthreads = oracle.threads()
    seqs = np.sort(np.random.default_rng(0).permutation(wl.B)[:max_seqs])
    k8, ks = oracle.quantize_fp8_rows(x["k_idx"][seqs])                      # untimed
    q_idx, w, q = x["q_idx"][seqs], x["w"][seqs], x["q"][seqs]
    kv = x["kv"][seqs]
    rows = [(s, t) for s in range(len(seqs)) for t in range(wl.Tq)]
    done, timed = 0, 0.0
    N = wl.N
    while timed <= budget_s:
        sel = [rows[(done + i) % len(rows)] for i in range(nthreads)]
        t0 = time.perf_counter()
        q8, qs = oracle.quantize_fp8_rows(q_idx)
        sc = np.full((len(sel), N), -np.inf, dtype=np.float32)
        nvalid = []
        for i, (s, t) in enumerate(sel):
            r = oracle.index_scores_fp8_rows(q8[s], qs[s], k8[s], ks[s], w[s], [t], wl.q_pos0)[0]
            sc[i, :len(r)] = r
            nvalid.append(len(r))
        idx = oracle.topk_rows(sc, nvalid, wl.K)
        idx_full = np.full((len(seqs), wl.Tq, wl.K), -1, dtype=np.int32)
        for i, (s, t) in enumerate(sel):
            idx_full[s, t] = idx[i]
            oracle.sparse_mla_batch(q, kv, idx_full, [(s, t)], wl.scale, wl.DV)
        timed += time.perf_counter() - t0
        done += len(sel)
    return {"value": done / timed, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "host_cpus": _host_cpus(), "cpu_model": _cpu_model(),
            "sample": f"{done} queries of {wl.name} with the FP8 indexer (whole path per query), cycling over the "
                      f"queries of {len(seqs)} sequences whose key caches were quantised beforehand (untimed), "
                      f"{timed:.1f} s; C++ oracle, double, one query at a time"}


def bench_next(args):
    """Times the calls built beside the path, each with HIP events on the launch
    stream over back-to-back launches of prebuilt C-ABI argument lists."""
    import torch

    import long_context_sparse_14_amd as dsa

    lib = dsa.library()
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    bf = torch.bfloat16
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    reps = max(5, args.steps)

    def rnd(*shape, sc=1.0):
        return (torch.randn(*shape, device="cuda", generator=g) * sc).to(bf)

    def ints(lo, hi, *shape):
        return torch.randint(lo, hi + 1, shape, device="cuda", generator=g).to(bf)

    def timed(fn, a):
        def once():
            rc = fn(*a)
            if rc != 0:
                raise RuntimeError(lib.dsa_last_error().decode())
        for _ in range(3):
            once()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            once()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us per call

    P = lambda t: t.data_ptr() if t is not None else None
    rows = []
    if args.next == "projections":
        H = 128
        w_uk, w_uv = rnd(H, 128, 512, sc=1 / 16), rnd(H, 128, 512, sc=1 / 16)
        for M in (32, 16384):
            q, ol = rnd(M, H, 192), rnd(M, H, 512)
            ql = torch.empty(M, H, 576, dtype=bf, device="cuda")
            o = torch.empty(M, H, 128, dtype=bf, device="cuda")
            fl = 2.0 * M * H * 128 * 512
            us = timed(lib.dsa_mla_absorb_q, (P(q), P(w_uk), P(ql), M, H, 128, 64, 512, dsa.DSA_BF16, sp))
            nb = (w_uk.numel() + q.numel() + ql.numel()) * 2
            rows.append({"call": "dsa_mla_absorb_q", "M": M, "heads": H, "us": round(us, 2),
                         "GB_per_s": round(nb / us / 1e3, 1), "TFLOP_per_s": round(fl / us / 1e6, 1)})
            us = timed(lib.dsa_mla_out_proj, (P(ol), P(w_uv), P(o), M, H, 512, 128, dsa.DSA_BF16, sp))
            nb = (w_uv.numel() + ol.numel() + o.numel()) * 2
            rows.append({"call": "dsa_mla_out_proj", "M": M, "heads": H, "us": round(us, 2),
                         "GB_per_s": round(nb / us / 1e3, 1), "TFLOP_per_s": round(fl / us / 1e6, 1)})
            x, wq = rnd(M, 1536), rnd(8192, 1536, sc=1 / 32)
            y = torch.empty(M, 8192, dtype=bf, device="cuda")
            us = timed(lib.dsa_linear, (P(x), P(wq), P(y), M, 8192, 1536, dsa.DSA_BF16, sp))
            nb = (x.numel() + wq.numel() + y.numel()) * 2
            rows.append({"call": "dsa_linear (wq_b)", "M": M, "N": 8192, "K": 1536, "us": round(us, 2),
                         "GB_per_s": round(nb / us / 1e3, 1), "TFLOP_per_s": round(2.0 * M * 8192 * 1536 / us / 1e6, 1)})
    elif args.next == "paged":
        B, N, K, bs = 32, 131072, 2048, 64
        q_idx, k_idx = ints(-4, 4, B, 1, 64, 128), ints(-4, 4, B, N, 128)
        w = torch.pow(2.0, -torch.randint(0, 5, (B, 1, 64), device="cuda", generator=g).float()).to(bf)
        q, kv = rnd(B, 1, 128, 576), rnd(B, N, 576)
        lens = torch.full((B,), N, dtype=torch.int64, device="cuda")
        mb = N // bs
        table = torch.randperm(B * mb, device="cuda", generator=g).to(torch.int32).view(B, mb).contiguous()
        prow = (table.long()[:, :, None] * bs + torch.arange(bs, device="cuda")).reshape(-1)
        k_pool = torch.empty(B * N, 128, dtype=bf, device="cuda")
        kv_pool = torch.empty(B * N, 576, dtype=bf, device="cuda")
        k_pool[prow] = k_idx.reshape(-1, 128)
        kv_pool[prow] = kv.reshape(-1, 576)
        out = torch.empty(B, 1, 128, 512, dtype=bf, device="cuda")
        lse = torch.empty(B, 1, 128, dtype=torch.float32, device="cuda")
        wsp = torch.empty(lib.dsa_paged_workspace_size(B, 1, mb, bs, 128, 512, K, dsa.DSA_BF16), dtype=torch.uint8,
                          device="cuda")
        wss = torch.empty(lib.dsa_forward_workspace_size(B, 1, N, 128, 512, K, dsa.DSA_BF16), dtype=torch.uint8,
                          device="cuda")
        sc = 1.0 / 192 ** 0.5
        us_s = timed(lib.dsa_forward_varlen, (P(q_idx), P(k_idx), P(w), P(q), P(kv), P(out), P(lse), None, P(lens), B,
                                              1, N, 64, 128, 128, 576, 512, K, sc, dsa.DSA_BF16, P(wss), wss.numel(),
                                              sp))
        us_p = timed(lib.dsa_forward_paged, (P(q_idx), P(k_pool), P(w), P(q), P(kv_pool), P(out), P(lse), None, P(lens),
                                             P(table), B, 1, mb, bs, B * mb, 64, 128, 128, 576, 512, K, sc,
                                             dsa.DSA_BF16, P(wsp), wsp.numel(), sp))
        rows.append({"call": "dsa_forward_varlen (static caches)", "batch": B, "context": N, "us": round(us_s, 2),
                     "queries_per_s": round(B / us_s * 1e6, 1)})
        rows.append({"call": "dsa_forward_paged", "batch": B, "context": N, "block_size": bs, "us": round(us_p, 2),
                     "queries_per_s": round(B / us_p * 1e6, 1)})
    else:
        # V4 CSA: 128K tokens compressed at m = 4 into 32768 entries, index_topk = 512
        B, T, m, K = 32, 131072, 4, 512
        N = T // m
        q_idx, k_idx = ints(-4, 4, B, 1, 64, 128), ints(-4, 4, B, N, 128)
        w = torch.pow(2.0, -torch.randint(0, 5, (B, 1, 64), device="cuda", generator=g).float()).to(bf)
        scores = torch.empty(B, 1, N, dtype=torch.float32, device="cuda")
        idx = torch.empty(B, 1, K, dtype=torch.int32, device="cuda")
        tws = torch.empty(max(256, lib.dsa_topk_workspace_size(B, 1, N, K)), dtype=torch.uint8, device="cuda")
        us_i = timed(lib.dsa_index_scores_compressed, (P(q_idx), P(k_idx), P(w), P(scores), B, 1, N, T - 1, m, 64, 128,
                                                       dsa.DSA_BF16, sp))
        us_t = timed(lib.dsa_topk_compressed, (P(scores), P(idx), B, 1, N, T - 1, m, K, P(tws), tws.numel(), sp))
        # the pair with the decode pre-selection (the lists share the top-k workspace, so the indexer runs first)
        us_ip = timed(lib.dsa_index_scores_compressed_presel, (P(q_idx), P(k_idx), P(w), P(scores), B, 1, N, T - 1, m,
                                                               64, 128, K, dsa.DSA_BF16, P(tws), tws.numel(), sp))
        us_tp = timed(lib.dsa_topk_compressed_presel, (P(scores), P(idx), B, 1, N, T - 1, m, K, dsa.DSA_BF16, P(tws),
                                                       tws.numel(), sp))
        nb = B * N * 128 * 2 + B * N * 4
        rows.append({"call": "dsa_index_scores_compressed", "batch": B, "tokens": T, "rate_m": m, "entries": N,
                     "us": round(us_i, 2), "GB_per_s": round(nb / us_i / 1e3, 1)})
        rows.append({"call": "dsa_topk_compressed", "batch": B, "entries": N, "K": K, "us": round(us_t, 2)})
        rows.append({"call": "dsa_index_scores_compressed_presel", "batch": B, "tokens": T, "rate_m": m,
                     "entries": N, "us": round(us_ip, 2), "GB_per_s": round(nb / us_ip / 1e3, 1)})
        rows.append({"call": "dsa_topk_compressed_presel", "batch": B, "entries": N, "K": K, "us": round(us_tp, 2)})
    print(json.dumps({"next": args.next, "launches_per_call": reps, "calls": rows}), flush=True)


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the batch shards by sequence with no "
              f"exchange, so per-GPU throughput is the one-GPU figure.", file=sys.stderr)
        sys.exit(2)
    if args.record_traffic:
        record_traffic(args)
        return
    if args.record_mfma:
        record_mfma(args)
        return
    import numpy as np
    import torch

    if args.calib_copy:
        calib_copy()
        return
    if args.next:
        bench_next(args)
        return

    import long_context_sparse_14_amd as dsa
    import synth

    dsa.library()
    wl = synth.WORKLOADS[args.workload]
    if args.batch > 0:
        wl = wl.replace(B=args.batch)
    x = synth.make_inputs(wl)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    d = {k: dev(v) for k, v in x.items()}
    dtt = (d["q"] if "q" in d else d["q_idx"]).dtype
    B, Tq, N = wl.B, wl.Tq, wl.N
    has_idx = "index" in wl.stages
    has_mla = "mla" in wl.stages
    scores = torch.empty((B, Tq, N), dtype=torch.float32, device="cuda") if has_idx else None
    idx = torch.empty((B, Tq, wl.K), dtype=torch.int32, device="cuda") if has_idx else d["idx"]
    out = torch.empty((B, Tq, wl.H, wl.DV), dtype=dtt, device="cuda") if has_mla else None
    lse = torch.empty((B, Tq, wl.H), dtype=torch.float32, device="cuda") if has_mla else None
    lib = dsa.library()
    code = dsa.DSA_BF16 if dtt == torch.bfloat16 else dsa.DSA_F32

    def buf(nbytes):
        return torch.empty(max(256, nbytes), dtype=torch.uint8, device="cuda")

    mla_ws = buf(lib.dsa_sparse_mla_workspace_size(B, Tq, wl.H, wl.DV, wl.K, code))
    topk_ws = buf(lib.dsa_topk_workspace_size(B, Tq, N, wl.K))
    fwd_ws = buf(lib.dsa_forward_workspace_size(B, Tq, N, wl.H, wl.DV, wl.K, code)) if (has_idx and has_mla) else None
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def ptr(t):
        return t.data_ptr() if t is not None else None

    # Argument tuples built once: the timed loop only enqueues work through the C ABI.
    calls = {}
    if has_idx:
        # the staged pair that the fused call runs (the decode indexer leaves a pre-selection for the top-k)
        calls["index"] = (lib.dsa_index_scores_presel, (ptr(d["q_idx"]), ptr(d["k_idx"]), ptr(d["w"]), ptr(scores),
                                                        B, Tq, N, wl.q_pos0, wl.H_I, wl.D_I, wl.K, code, ptr(topk_ws),
                                                        topk_ws.numel(), sp))
        calls["topk"] = (lib.dsa_topk_presel, (ptr(scores), ptr(idx), B, Tq, N, wl.q_pos0, wl.K, code, ptr(topk_ws),
                                               topk_ws.numel(), sp))
    if has_mla:
        calls["mla"] = (lib.dsa_sparse_mla_fwd, (ptr(d["q"]), ptr(d["kv"]), ptr(idx), ptr(out), ptr(lse), B, Tq, N,
                                                 wl.H, wl.D, wl.DV, wl.K, wl.scale, code, ptr(mla_ws),
                                                 mla_ws.numel(), sp))
    if has_idx and has_mla:
        calls["fused"] = (lib.dsa_forward, (ptr(d["q_idx"]), ptr(d["k_idx"]), ptr(d["w"]), ptr(d["q"]), ptr(d["kv"]),
                                            ptr(out), ptr(lse), None, B, Tq, N, wl.q_pos0, wl.H_I, wl.D_I, wl.H,
                                            wl.D, wl.DV, wl.K, wl.scale, code, ptr(fwd_ws), fwd_ws.numel(), sp))

    fp8 = args.fp8_indexer
    if fp8:
        if not (has_idx and Tq <= 4 and dtt == torch.bfloat16):
            raise SystemExit("--fp8-indexer applies to bf16 decode workloads with an indexer stage")
        # the key cache is held as codes: quantised once, before timing (appended tokens are quantised as
        # they arrive); each step quantises its own queries
        k8 = torch.empty((B, N, wl.D_I), dtype=torch.uint8, device="cuda")
        ks = torch.empty((B, N), dtype=torch.float32, device="cuda")
        q8 = torch.empty((B, Tq, wl.H_I, wl.D_I), dtype=torch.uint8, device="cuda")
        qs = torch.empty((B, Tq, wl.H_I), dtype=torch.float32, device="cuda")
        rc = lib.dsa_indexer_quantize_fp8(ptr(d["k_idx"]), ptr(k8), ptr(ks), B * N, wl.D_I, code, sp)
        if rc != 0:
            raise RuntimeError(lib.dsa_last_error().decode())
        del d["k_idx"]
        calls["quant_q"] = (lib.dsa_indexer_quantize_fp8, (ptr(d["q_idx"]), ptr(q8), ptr(qs), B * Tq * wl.H_I,
                                                           wl.D_I, code, sp))
        # the staged pair that the fused FP8 call runs (its indexer also pre-selects at decode shapes)
        calls["index"] = (lib.dsa_index_scores_fp8_presel, (ptr(q8), ptr(qs), ptr(k8), ptr(ks), ptr(d["w"]),
                                                            ptr(scores), B, Tq, N, wl.q_pos0, wl.H_I, wl.D_I, wl.K,
                                                            code, ptr(topk_ws), topk_ws.numel(), sp))
        calls["topk"] = (lib.dsa_topk_presel_fp8, (ptr(scores), ptr(idx), B, Tq, N, wl.q_pos0, wl.K, ptr(topk_ws),
                                                   topk_ws.numel(), sp))
        if has_mla:
            calls["fused"] = (lib.dsa_forward_fp8, (ptr(q8), ptr(qs), ptr(k8), ptr(ks), ptr(d["w"]), ptr(d["q"]),
                                                    ptr(d["kv"]), ptr(out), ptr(lse), None, B, Tq, N, wl.q_pos0,
                                                    wl.H_I, wl.D_I, wl.H, wl.D, wl.DV, wl.K, wl.scale, code,
                                                    ptr(fwd_ws), fwd_ws.numel(), sp))

    def run(name):
        fn, a = calls[name]
        rc = fn(*a)
        if rc != 0:
            raise RuntimeError(f"{name}: {lib.dsa_last_error().decode()}")

    def step(evs=None):
        if fp8:
            if evs is not None:
                evs[4].record(stream)
            run("quant_q")
        if evs is not None:
            evs[0].record(stream)
        if has_idx:
            run("index")
            if evs is not None:
                evs[1].record(stream)
            run("topk")
        if evs is not None:
            evs[2].record(stream)
        if has_mla:
            run("mla")
        if evs is not None:
            evs[3].record(stream)

    def fused_step():
        if fp8:
            run("quant_q")
        run("fused")

    # Steps run the fused entry point where the workload has one (one C-ABI
    # call); every INSTR-th step of the timed region (at least five of them,
    # at most every tenth) instead runs the stages as separate calls with HIP
    # events between them, which measures each kernel's duration live on the
    # launch stream (--staged: every step).
    ceilings = measured_ceilings(dominant_stage(wl, fp8)[2])
    has_fused = has_idx and has_mla
    INSTR = 1 if (args.staged or not has_fused) else max(2, min(10, args.steps // 5))
    for _ in range(args.warmup):
        fused_step() if has_fused else step()
    torch.cuda.synchronize()

    graph = None
    if args.graph and has_fused:
        # the library launches only on the given stream and never allocates,
        # synchronises or clears memory, so one fused step captures as is; the
        # capture stream replaces the stream argument (the last one) of each call
        cap = torch.cuda.Stream()
        on_cap = {k: (fn, a[:-1] + (cap.cuda_stream,)) for k, (fn, a) in calls.items()}

        def cap_step():
            for name in (("quant_q", "fused") if fp8 else ("fused",)):
                fn, a = on_cap[name]
                if fn(*a) != 0:
                    raise RuntimeError(f"{name}: {lib.dsa_last_error().decode()}")
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            cap_step()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            cap_step()
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
    n_ev = (args.steps + INSTR - 1) // INSTR
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_ev)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % INSTR == 0:
            step(events[i // INSTR])
        elif graph is not None:
            graph.replay()
        else:
            fused_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    stage_ms = {}
    for name, (a, b) in {"index": (0, 1), "topk": (1, 2), "mla": (2, 3)}.items():
        if (name != "mla" and not has_idx) or (name == "mla" and not has_mla):
            continue
        stage_ms[name] = float(np.mean([e[a].elapsed_time(e[b]) for e in events]))
    if fp8:
        stage_ms["quantize_q"] = float(np.mean([e[4].elapsed_time(e[0]) for e in events]))
    timed = ("%s per step; every %dth step staged with HIP events per kernel"
             % ("replay of a HIP graph of the fused call" if graph is not None else "fused C-ABI call", INSTR)
             if INSTR > 1 else "staged C-ABI calls with HIP events per kernel")

    queries = B * Tq
    value = queries / (ms_per_step / 1e3)
    stage, kname, bound, work, wunit = dominant_stage(wl, fp8)
    roof = None
    if stage in stage_ms:
        sec = stage_ms[stage] / 1e3
        if bound == "hbm":
            ach = work / sec / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4)}
        else:
            ach = work / sec / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
        roof["traffic"] = stored_traffic(wl.name, kname)
        roof["measured_ceiling"] = ceilings
        if bound == "hbm":
            roof["frac_of_measured_read"] = round(ach / ceilings["read_GBps"], 4)
        else:
            roof["frac_of_library_gemm"] = round(ach / ceilings["library_gemm_bf16_TFLOPs"], 4)
        if bound == "mfma":
            roof["counters"] = stored_mfma(wl.name, kname)
        roof["kernel"] = kname
        roof["kernel_avg_us"] = round(stage_ms[stage] * 1e3, 2)
        roof["algorithmic_" + ("bytes" if wunit == "B" else "flops") + "_per_launch"] = int(work)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 (indexer: fp8-e4m3 codes widened to bf16)" if fp8 else "bf16") if dtt == torch.bfloat16
        else "f32",
        "data": "synthetic (seeded generator; integer-valued indexer inputs, N(0,1) latents)",
        "config": {"workload": wl.name, "batch": B, "queries_per_seq": Tq, "context": N, "index_topk": wl.K,
                   "indexer_heads": wl.H_I, "indexer_dim": wl.D_I, "mla_heads": wl.H, "latent_dim": wl.D,
                   "value_dim": wl.DV, "timed": timed,
                   "indexer": "fp8 (Hadamard-rotated E4M3 key cache, power-of-two row scales)" if fp8 else "bf16",
                   "parallelism": "single GPU"},
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "tokens_per_s": round(value, 1),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_fp8(wl, x, args.cpu_budget_s) if fp8 else \
            cpu_baseline(wl, x, args.cpu_budget_s)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
