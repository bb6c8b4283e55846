"""Benchmark of the W4A16 decode/verify matmul on one MI355X.

Default run: the down projection of the 27B decoder (K=17408, N=5120, group
128, A drawn as SiLU(x)*y) at the metric's row counts M = 1, 4, 8, 16, each
timed as `--steps` calls inside one HIP graph replay.  The weight blob,
scales, activations and outputs rotate over distinct buffer sets (>= 1 GiB in
total) so that no call finds its weights in the 256 MiB last-level cache:
every call streams its weights from HBM.  One step is one call at each M.

Prints ONE JSON line:
  value        algorithmic bytes of one step / its summed call times, GB/s
  config       per-M us/call, GB/s, % of 8 TB/s, plan; MFMA utilisation at
               M=16; extras: the other decoder shapes (QKV, attention out,
               gate/up, lm_head) and the 257-call decode step at M=1 and 8
  roofline     the same rates against MI355X's 8 TB/s, per M and for the step;
               traffic = HBM bytes per launch from the rocprofv3 counters
  cpu_baseline the fp64 CPU oracle on the same workload (M=1)

--workload W --m M times one call shape (the profiled runs use these);
--sweep prints one JSON line per (workload, M) instead (not the contract line);
--stack times one decode step's full sequence of linear shapes.
--ceiling measures a plain streaming read at the same byte counts.
--tp-shards times one GPU's share of each linear under tensor parallelism.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "achieved HBM GB/s (% of peak) for W4A16 matmul at M=1,4,8,16; µs/call"
METRIC_NVFP4 = "achieved HBM GB/s (% of peak) for the NVFP4 weight-only (W4A16) matmul; µs/call"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
# row counts of the headline line per workload: the metric's set (M = 1, 4, 8, 16)
HEADLINE_MS = {"down": (1, 4, 8, 16), "qkv": (1, 4, 8, 16), "attn_out": (1, 4, 8, 16), "gate_up": (1, 4, 8, 16),
               "lm_head": (1, 8, 16), "tiny": (1,)}
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
LLC_BYTES = 256 << 20          # MI355X Infinity Cache
ROTATE_BYTES = 1 << 30         # rotate over >= 1 GiB of buffer sets
# the files the matmul kernels are built from (their hash ties counters to a build)
KERNEL_SOURCES = (["weight_only_int4_gptq_amd/csrc/w4a16_kernels.hpp",
                   "weight_only_int4_gptq_amd/csrc/w4a16_variants.hpp",
                   "weight_only_int4_gptq_amd/build.py"] +
                  ["weight_only_int4_gptq_amd/csrc/" + u for u in
                   ("w4a16.hip",
                    "variants_plain_gemv.hip", "variants_plain_mfma12.hip", "variants_plain_mfma34.hip",
                    "variants_plain_rt.hip", "variants_epi_gemv.hip", "variants_epi_mfma12.hip",
                    "variants_epi_mfma34.hip", "variants_epi_rt.hip", "variants_nvfp4_gemv.hip",
                    "variants_nvfp4_mfma.hip", "variants_nvfp4_epi_gemv.hip", "variants_nvfp4_epi_mfma.hip")])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Problem:
    """Device buffers for one (K, N) shape, replicated over `sets` distinct buffer sets."""

    def __init__(self, torch, w4, K, N, seed, act, sets, Mmax=16):
        dev = torch.device("cuda:0")
        A, qw, sc = synth.gen_problem(K, N, seed, act, Mmax)
        self.host = (A, qw, sc)
        q = torch.from_numpy(qw.view(np.int32)).to(dev)
        blob = w4.repack_weights(q, K, N)
        del q
        # the checkpoint's bf16 scales [K/128, N], used as they are
        s = torch.from_numpy(sc.view(np.int16)).to(dev).view(torch.bfloat16)
        a = torch.from_numpy(A.view(np.int16)).to(dev).view(torch.bfloat16)
        self.blobs = [blob] + [blob.clone() for _ in range(sets - 1)]
        self.scales = [s] + [s.clone() for _ in range(sets - 1)]
        self.acts = [a] + [a.clone() for _ in range(sets - 1)]
        self.outs = [torch.empty((Mmax, N), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
        # gate/up outputs H[Mmax, N/2], contiguous, in the first half of each C buffer
        self.houts = ([o.view(-1)[: Mmax * (N // 2)].view(Mmax, N // 2) for o in self.outs]
                      if N % 32 == 0 else None)
        self.K, self.N, self.sets = K, N, sets
        torch.cuda.synchronize()

    fmt = "gptq"

    def call(self, w4, M, i):
        j = i % self.sets
        w4.gemm(self.acts[j][:M], self.blobs[j], self.scales[j], self.N, out=self.outs[j][:M])

    def bytes(self, M):
        return synth.algorithmic_bytes(M, self.N, self.K)

    def oracle_call(self, M, **kw):
        import oracle
        A, qw, sc = self.host
        return oracle.gemm(A, qw, sc, M, self.N, self.K, **kw)


class NvProblem:
    """NVFP4 buffers for one (K, N) shape over `sets` distinct buffer sets (same interface as Problem)."""

    fmt = "nvfp4"

    def __init__(self, torch, w4, K, N, seed, act, sets, Mmax=16):
        dev = torch.device("cuda:0")
        A, packed, sc = synth.gen_nvfp4_problem(K, N, seed, act, Mmax)
        self.host = (A, packed, sc)
        blob, s = w4.nvfp4_repack(torch.from_numpy(packed).to(dev), torch.from_numpy(sc).to(dev), K, N)
        a = torch.from_numpy(A.view(np.int16)).to(dev).view(torch.bfloat16)
        self.blobs = [blob] + [blob.clone() for _ in range(sets - 1)]
        self.scales = [s] + [s.clone() for _ in range(sets - 1)]
        self.acts = [a] + [a.clone() for _ in range(sets - 1)]
        self.outs = [torch.empty((Mmax, N), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
        self.K, self.N, self.sets = K, N, sets
        torch.cuda.synchronize()

    def call(self, w4, M, i):
        j = i % self.sets
        w4.nvfp4_gemm(self.acts[j][:M], self.blobs[j], self.scales[j], synth.NVFP4_ALPHA, self.N,
                      out=self.outs[j][:M])

    def bytes(self, M):
        return synth.algorithmic_bytes_nvfp4(M, self.N, self.K)

    def oracle_call(self, M, **kw):
        import oracle
        A, packed, sc = self.host
        return oracle.nvfp4_gemm(A, packed, sc, synth.NVFP4_ALPHA, M, self.N, self.K, **kw)


def sets_for(K, N, M):
    per = synth.algorithmic_bytes(M, N, K)
    return max(1, -(-ROTATE_BYTES // per)) if per < 4 * LLC_BYTES else 1


def time_graph(torch, fn, steps, warmup, sets=0):
    """Warm up eagerly, capture `steps` calls in one graph, replay and time it (ms/step).

    fn(i) makes call i (on buffer set i % sets when the caller rotates).  With
    fewer steps than sets, calls on the remaining sets run eagerly between the
    warm and the timed replay, so that every timed call's buffers were last
    touched (sets - 1) calls earlier, whatever `steps` is.
    """
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                fn(i)
    torch.cuda.synchronize()
    g.replay()                      # warm replay
    for i in range(steps, sets):    # the other buffer sets, untimed
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def graph_steps(args, nbytes):
    """Calls per captured graph for the sweeps: at least 100, so that the fixed
    cost of one replay is a small share of the per-call time, and at most
    --steps, or about 4 GB of weight reads, whichever is fewer (but not below 100)."""
    return max(100, min(args.steps, int(4e9 / nbytes)))


def measure(torch, w4, prob, M, steps, warmup):
    ms_graph = time_graph(torch, lambda i: prob.call(w4, M, i), steps, warmup, prob.sets)
    nbytes = prob.bytes(M)
    flops = 2.0 * M * prob.N * prob.K
    return {
        "ms_per_step": ms_graph,
        "us_per_call": ms_graph * 1e3,
        "gbs": nbytes / (ms_graph * 1e-3) / 1e9,
        "bytes": nbytes,
        "tflops": flops / (ms_graph * 1e-3) / 1e12,
    }


def copy_calibration(torch, mib, reps=4):
    """Plain device-to-device copies of a known size (a reference for the HBM byte counters)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: {reps} copies of {mib} MiB (read {n} B, write {n} B each)")


def cpu_baseline(prob, M, seconds=10.0):
    import oracle

    nthreads = oracle.max_threads()
    prob.oracle_call(M, cols=np.arange(64))    # load + warm
    reps, t0 = 0, time.perf_counter()
    while True:
        prob.oracle_call(M, nthreads=nthreads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    nbytes = prob.bytes(M) * reps
    return {"value": round(nbytes / el / 1e9, 3), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{reps} full calls of the same workload (M={M}, K={prob.K}, N={prob.N}), "
                      f"{el:.1f} s wall, fp64 C oracle with OpenMP over columns; "
                      f"{el / reps * 1e6:.0f} us/call",
            "host": {"cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
                     "usable_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def traffic_record(name):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(name)
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_profiles(args):
    """Turn rocprofv3 output (kernel trace + FETCH_SIZE/WRITE_SIZE passes) into profiles/.

    Writes profiles/traffic.json (HBM bytes per launch of the matmul kernel,
    each counter scaled by what it reads for a plain copy of known size) and
    two short text summaries named for the kernel and workload.
    """
    import statistics as st
    trace_dir, fetch_dir, write_dir = args.summarize
    wname, M, mib = args.workload, args.m, args.copy_calib
    wl = synth.WORKLOADS[wname]
    nv = args.format == "nvfp4"
    tag = f"{'nvfp4_' if nv else ''}{wname}_m{M}"
    fmt_flag = " --format nvfp4" if nv else ""
    copy_kib = float(mib << 10)

    def counter(d):
        rows = _csv_rows(os.path.join(d, "run_counter_collection.csv"))
        gemm = [float(r["Counter_Value"]) for r in rows if "gemm_kernel" in r["Kernel_Name"]]
        kname = next(r["Kernel_Name"] for r in rows if "gemm_kernel" in r["Kernel_Name"])
        # the calibration copies are the copy dispatches near the reference size
        cp = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]
              and float(r["Counter_Value"]) > 0.25 * copy_kib]
        return kname, st.median(gemm), len(gemm), st.median(cp), len(cp)

    kname, f_kib, nf, f_copy, ncf = counter(fetch_dir)
    _, w_kib, nw, w_copy, ncw = counter(write_dir)
    f_fac, w_fac = copy_kib / f_copy, copy_kib / w_copy
    nbytes = round((f_kib * f_fac + w_kib * w_fac) * 1024)
    algo = (synth.algorithmic_bytes_nvfp4 if nv else synth.algorithmic_bytes)(M, wl.N, wl.K)
    cmd_f = (f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run --output-format csv -- "
             f"python3 bench.py --workload {wname} --m {M}{fmt_flag} --steps 20 --warmup 5 --no-cpu "
             f"--copy-calib {mib}")
    cmd_w = cmd_f.replace("FETCH_SIZE", "WRITE_SIZE").replace(fetch_dir, write_dir)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[tag] = {"kernel": kname, "source_hash": kernel_source_hash(), "bytes_per_launch": nbytes,
                "algorithmic_bytes": algo, "fetch_kib": f_kib, "write_kib": w_kib,
                "fetch_factor": round(f_fac, 5), "write_factor": round(w_fac, 5),
                "reference": f"plain device copy of {mib} MiB (reads and writes {mib} MiB)",
                "commands": [cmd_f, cmd_w]}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")

    kshort = kname.split("(")[0].replace("void ", "").replace("w4a16::", "")
    with open(os.path.join(ROOT, "profiles", f"gemm_kernel_{tag}_hbm_bytes.md"), "w") as f:
        f.write(f"# HBM bytes per launch: {kshort}, {wl.desc}, M={M}{', NVFP4' if nv else ''}\n\n")
        f.write("Commands (repo root, TMPDIR=/tmp):\n\n")
        f.write(f"    {cmd_f}\n    {cmd_w}\n\n")
        f.write("| counter | matmul kernel, median KiB/dispatch | dispatches | "
                f"copy of {mib} MiB, median KiB | copies | scale |\n|---|---|---|---|---|---|\n")
        f.write(f"| FETCH_SIZE | {f_kib:.1f} | {nf} | {f_copy:.1f} | {ncf} | {f_fac:.4f} |\n")
        f.write(f"| WRITE_SIZE | {w_kib:.1f} | {nw} | {w_copy:.1f} | {ncw} | {w_fac:.4f} |\n\n")
        f.write(f"Scaled HBM traffic per launch: {nbytes} B; algorithmic bytes: {algo} B "
                f"(ratio {nbytes / algo:.4f}).\n")
        f.write(f"Kernel source hash: {kernel_source_hash()}\n")

    rows = [r for r in _csv_rows(os.path.join(trace_dir, "run_kernel_trace.csv")) if "gemm_kernel" in r["Kernel_Name"]]
    d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]
    stats = _csv_rows(os.path.join(trace_dir, "run_kernel_stats.csv"))
    sets = sets_for(wl.K, wl.N, 1)
    flush = max(0, sets - args.steps)            # untimed calls on the other buffer sets
    w = args.warmup
    a = w + args.steps                           # warm replay [w, a)
    b = a + flush                                # the other sets [a, b), eager
    e = b + args.steps                           # timed replay [b, e)
    timed = st.mean(d[b:e]) if len(d) >= e else None
    with open(os.path.join(ROOT, "profiles", f"gemm_kernel_{tag}_kernel_trace.md"), "w") as f:
        what = f"NVFP4 weights, M={M}" if nv else f"M={M}"
        f.write(f"# Kernel trace: {wl.desc}, {what}\n\n")
        f.write(f"Command (repo root, TMPDIR=/tmp):\n\n    rocprofv3 --kernel-trace --stats -d {trace_dir} "
                f"-o run --output-format csv -- python3 bench.py --workload {wname} --m {M}{fmt_flag} "
                f"--steps {args.steps} --warmup {args.warmup} --no-cpu\n\n")
        f.write("rocprofv3 --stats summary (run_kernel_stats.csv):\n\n| kernel | calls | average ns | min ns | max ns |\n|---|---|---|---|---|\n")
        for r in stats:
            f.write(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |\n")
        if timed is not None:
            f.write(f"\nMatmul kernel by phase: {w} eager warm-up launches average {st.mean(d[:w]):.0f} ns; "
                    f"warm graph replay average {st.mean(d[w:a]):.0f} ns; timed graph replay average "
                    f"{timed:.0f} ns over {args.steps} launches ({timed and synth_bytes(nv, M, wl) / timed:.1f} GB/s, "
                    f"{100 * synth_bytes(nv, M, wl) / timed / PEAK_HBM_GBS:.2f}% of 8 TB/s).\n")
        f.write(f"Kernel source hash: {kernel_source_hash()}\n")
    rec[tag]["trace_timed_avg_ns"] = round(timed) if timed is not None else None
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec[tag]))


# Hardware-counter passes of one matmul call shape (each its own rocprofv3 run;
# at most 8 SQ, 4 TCP and 4 TCC counters per pass).
COUNTER_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA "
    "SQ_VALU_MFMA_BUSY_CYCLES",
    "SQ_INSTS_SALU SQ_INSTS_VMEM SQ_INSTS_LDS SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_ANY",
    "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCC_HIT_sum TCC_MISS_sum",
]
CHIP_SES, CHIP_CUS, CHIP_SIMDS, CLOCK_GHZ = 32, 256, 1024, 2.4


def summarize_counters(args):
    """profiles/gemm_kernel_<workload>_m<M>_counters.md from rocprofv3 --pmc runs.

    Each directory holds one pass of COUNTER_PASSES (any order).  Values are
    the median over the matmul kernel's dispatches, summed over the chip.
    Derived figures: waves per SIMD; the share of wave-cycles spent waiting
    and issuing VALU instructions; instructions per (16-column tile,
    128-row group) unit; MFMA busy share of all SIMD-cycles of the call;
    the mean L1 -> L2 read latency.
    """
    import statistics as st
    wname, M = args.workload, args.m
    wl = synth.WORKLOADS[wname]
    nv = args.format == "nvfp4"
    tag = f"{'nvfp4_' if nv else ''}{wname}_m{M}"
    fmt_flag = " --format nvfp4" if nv else ""
    vals, cmds, kname = {}, [], None
    for d in args.summarize_counters:
        per = {}
        for r in _csv_rows(os.path.join(d, "run_counter_collection.csv")):
            if "gemm_kernel" not in r["Kernel_Name"]:
                continue
            kname = kname or r["Kernel_Name"]
            per.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for c, by_dispatch in per.items():
            vals[c] = (st.median(by_dispatch.values()), len(by_dispatch))
        cmds.append(f"rocprofv3 --pmc {' '.join(sorted(per))} -d {d} -o run --output-format csv -- "
                    f"python3 bench.py --workload {wname} --m {M}{fmt_flag} --steps 20 --warmup 5 --no-cpu")
    v = {c: x[0] for c, x in vals.items()}
    units = (wl.N // 16) * (wl.K // 128)
    kshort = kname.split("(")[0].replace("void ", "").replace("w4a16::", "")
    out = [f"# Hardware counters: {kshort}, {wl.desc}, M={M}{', NVFP4' if nv else ''}\n",
           "Commands (repo root, TMPDIR=/tmp), one pass each:\n"]
    out += [f"    {c}" for c in cmds]
    out += ["", "Median over the matmul kernel's dispatches (warm-up, flush and graph-replayed calls, all "
            "on cold weights) of each counter summed over the chip:", "",
            "| counter | value | dispatches |", "|---|---|---|"]
    out += [f"| {c} | {v[c]:.0f} | {vals[c][1]} |" for c in sorted(v)]
    derived = []

    def add(name, f):
        try:
            derived.append((name, f()))
        except (KeyError, ZeroDivisionError):
            pass

    busy = lambda: v["SQ_BUSY_CYCLES"] / CHIP_SES          # cycles the shader engines held waves
    add("waves per launch", lambda: f"{v['SQ_WAVES']:.0f} ({v['SQ_WAVES'] / CHIP_SIMDS:.2f} per SIMD)")
    add("shader-engine busy time", lambda: f"{busy():.0f} cycles = {busy() / CLOCK_GHZ / 1000:.2f} us at "
        f"{CLOCK_GHZ} GHz")
    add("mean wave lifetime", lambda: f"{4 * v['SQ_WAVE_CYCLES'] / v['SQ_WAVES']:.0f} cycles "
        f"({4 * v['SQ_WAVE_CYCLES'] / v['SQ_WAVES'] / busy():.2f} of the busy time)")
    add("wave-cycles waiting (any cause)", lambda: f"{v['SQ_WAIT_ANY'] / v['SQ_WAVE_CYCLES']:.1%}")
    add("wave-cycles issuing VALU", lambda: f"{v['SQ_ACTIVE_INST_VALU'] / v['SQ_WAVE_CYCLES']:.1%}")
    add("wave-cycles waiting to issue", lambda: f"{v['SQ_WAIT_INST_ANY'] / v['SQ_WAVE_CYCLES']:.1%}")
    add("VALU instructions per (tile, group)", lambda: f"{v['SQ_INSTS_VALU'] / units:.1f}")
    add("MFMA instructions per (tile, group)", lambda: f"{v['SQ_INSTS_MFMA'] / units:.2f}")
    add("SALU instructions per (tile, group)", lambda: f"{v['SQ_INSTS_SALU'] / units:.1f}")
    add("VMEM instructions per (tile, group)", lambda: f"{v['SQ_INSTS_VMEM'] / units:.2f}")
    add("LDS instructions per (tile, group)", lambda: f"{v['SQ_INSTS_LDS'] / units:.2f}")
    add("MFMA busy, share of all SIMD-cycles", lambda: f"{v['SQ_VALU_MFMA_BUSY_CYCLES'] / (CHIP_SIMDS * busy()):.1%}")
    add("LDS bank-conflict cycles per LDS-active cycle",
        lambda: f"{v['SQ_LDS_BANK_CONFLICT'] / (4 * v['SQ_ACTIVE_INST_LDS']):.2f}")
    add("mean L1 -> L2 read latency", lambda: f"{v['TCP_TCC_READ_REQ_LATENCY_sum'] / v['TCP_TCC_READ_REQ_sum']:.0f} cycles")
    add("L2 hit rate", lambda: f"{v['TCC_HIT_sum'] / (v['TCC_HIT_sum'] + v['TCC_MISS_sum']):.1%}")
    out += ["", f"Derived ({units} units of one 16-column tile x 128 rows; {CHIP_SES} shader engines, "
            f"{CHIP_SIMDS} SIMDs):", "", "| figure | value |", "|---|---|"]
    out += [f"| {a} | {b} |" for a, b in derived]
    out += ["", f"Kernel source hash: {kernel_source_hash()}", ""]
    path = os.path.join(ROOT, "profiles", f"gemm_kernel_{tag}_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    print(path)


def synth_bytes(nv, M, wl):
    return (synth.algorithmic_bytes_nvfp4 if nv else synth.algorithmic_bytes)(M, wl.N, wl.K)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="down", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--m", type=int, default=0,
                    help="one row count (default: the metric's set for the workload, M = 1, 4, 8, 16 for down)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the further keys (other decoder shapes, the full decode step)")
    ap.add_argument("--format", default="gptq", choices=("gptq", "nvfp4"),
                    help="weight format of the measured call (gptq: the headline INT4 group-128 path)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--sweep", action="store_true", help="one JSON line per (workload, M)")
    ap.add_argument("--stack", action="store_true", help="full decode-step sweep of linear shapes")
    ap.add_argument("--ceiling", action="store_true",
                    help="plain streaming-read bandwidth at the matmul byte counts (probe kernel)")
    ap.add_argument("--tp-shards", action="store_true",
                    help="one GPU's share of each decoder linear at TP = 2, 4, 8")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="after timing, copy MIB MiB a few times (reference for byte counters)")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ from rocprofv3 output of the bench (no GPU use)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="write profiles/..._counters.md from rocprofv3 --pmc runs of the bench (no GPU use)")
    args = ap.parse_args()
    if args.summarize:
        return summarize_profiles(args)
    if args.summarize_counters:
        return summarize_counters(args)

    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              f"(the matmul shards by columns without communication; one GPU's share is "
              f"measured by --tp-shards)", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_int4_gptq_amd as w4

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    name = torch.cuda.get_device_name(0)

    if args.sweep:
        return nvfp4_sweep(torch, w4, args) if args.format == "nvfp4" else sweep(torch, w4, args)
    if args.stack:
        return stack(torch, w4, args)
    if args.ceiling:
        return ceiling(torch, w4, args)
    if args.tp_shards:
        return tp_shards(torch, w4, args)

    wl = synth.WORKLOADS[args.workload]
    nv = args.format == "nvfp4"
    Ms = [args.m] if args.m else list(HEADLINE_MS.get(args.workload, (1,)))
    sets = sets_for(wl.K, wl.N, 1)
    log(f"bench: {wl.desc} M={Ms} ({args.format}) on {name}; {sets} buffer sets")
    if nv:
        prob = NvProblem(torch, w4, wl.K, wl.N, wl.seed + synth.NVFP4_SEED_OFFSET, wl.act, sets)
    else:
        prob = Problem(torch, w4, wl.K, wl.N, wl.seed, wl.act, sets)
    per_m, total_bytes, total_ms = [], 0, 0.0
    for M in Ms:
        r = measure(torch, w4, prob, M, args.steps, args.warmup)
        plan = (w4.nvfp4_get_plan if nv else w4.get_plan)(M, wl.N, wl.K).as_dict()
        tag = f"{'nvfp4_' if nv else ''}{args.workload}_m{M}"
        log(f"bench: M={M} {r['us_per_call']:.3f} us/call {r['gbs']:.0f} GB/s; plan {plan}")
        entry = {"M": M, "us_per_call": round(r["us_per_call"], 3), "GBps": round(r["gbs"], 1),
                 "pct_of_peak_hbm": round(100 * r["gbs"] / PEAK_HBM_GBS, 2),
                 "frac": round(r["gbs"] / PEAK_HBM_GBS, 4), "algorithmic_bytes": r["bytes"],
                 "traffic": traffic_record(tag), "plan": plan}
        if M == 16:
            entry["mfma_util"] = round(r["tflops"] / PEAK_BF16_TFLOPS, 4)
        per_m.append(entry)
        total_bytes += r["bytes"]
        total_ms += r["ms_per_step"]
    if args.copy_calib:
        copy_calibration(torch, args.copy_calib)

    # one step = one call at each of the M values, one kernel launch each; the
    # headline rate is the bytes of the step over its summed call times
    gbs = total_bytes / (total_ms * 1e-3) / 1e9
    traffics = [e["traffic"] for e in per_m]
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": (sum(traffics) if all(t is not None for t in traffics) else None),
            "algorithmic_bytes": total_bytes,
            "per_m": [{"M": e["M"], "achieved": e["GBps"], "frac": e["frac"], "traffic": e["traffic"],
                       "algorithmic_bytes": e["algorithmic_bytes"], "us_per_launch": e["us_per_call"]}
                      for e in per_m]}
    what = (f"{args.workload}: {wl.desc}, M in {{{','.join(map(str, Ms))}}}, "
            + ("NVFP4 weights (E2M1, E4M3 scale per 16)" if nv else "group 128"))
    out = {
        "metric": METRIC_NVFP4 if nv else METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": what,
            "K": wl.K, "N": wl.N, "group": 16 if nv else 128, "Ms": Ms,
            "step": "one call at each M (one kernel launch each); value = bytes of the step / summed call times",
            "per_m": per_m,
            "buffer_sets": sets,
            "timing": ("per M: HIP events around one graph replay of `steps` calls on the launch stream, "
                       "call i on buffer set i % buffer_sets, every set last touched >= 1 GiB of weights earlier"),
            "device": name,
        },
        "roofline": roof,
    }
    if not args.no_cpu:
        log("bench: timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(prob, Ms[0], args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    del prob
    torch.cuda.empty_cache()
    if not args.no_extras and not nv and args.m == 0 and args.workload == "down":
        out["config"]["extras"] = extras(torch, w4, args)
    print(json.dumps(out), flush=True)


def extras(torch, w4, args):
    """Further keys of the default line: the other decoder shapes and the
    full decode step, each timed the same way (graph replay, rotating sets)."""
    res = {}
    for wname, Ms in (("qkv", (1, 4, 8, 16)), ("attn_out", (1, 8)), ("gate_up", (1, 8)), ("lm_head", (1, 8, 16))):
        wl = synth.WORKLOADS[wname]
        sets = sets_for(wl.K, wl.N, 1)
        prob = Problem(torch, w4, wl.K, wl.N, wl.seed, wl.act, sets)
        for M in Ms:
            steps = graph_steps(args, prob.bytes(M))
            r = measure(torch, w4, prob, M, steps, min(args.warmup, 10))
            res[f"{wname}_m{M}"] = {"K": wl.K, "N": wl.N, "us_per_call": round(r["us_per_call"], 3),
                                    "GBps": round(r["gbs"], 1), "pct_of_peak_hbm": round(100 * r["gbs"] / PEAK_HBM_GBS, 2)}
            log(f"bench: {wname} M={M} {r['us_per_call']:.3f} us/call {r['gbs']:.0f} GB/s")
        del prob
        torch.cuda.empty_cache()
    for rec in stack(torch, w4, args, quiet=True):
        res[f"stack_m{rec['M']}"] = {k: rec[k] for k in ("calls", "bytes", "ms_per_step", "GBps", "pct_peak")}
        log(f"bench: stack M={rec['M']} {rec['ms_per_step']:.3f} ms {rec['GBps']:.0f} GB/s")
    return res


def nvfp4_sweep(torch, w4, args):
    """NVFP4 weight-only calls: one JSON line per (workload, M)."""
    for wname in ("qkv", "gate_up", "down", "lm_head"):
        wl = synth.WORKLOADS[wname]
        sets = sets_for(wl.K, wl.N, 1)
        prob = NvProblem(torch, w4, wl.K, wl.N, wl.seed + synth.NVFP4_SEED_OFFSET, wl.act, sets)
        for M in (1, 2, 4, 8, 16):
            r = measure(torch, w4, prob, M, graph_steps(args, prob.bytes(M)), min(args.warmup, 20))
            print(json.dumps({"format": "nvfp4", "workload": wname, "M": M, "K": wl.K, "N": wl.N,
                              "plan": w4.nvfp4_get_plan(M, wl.N, wl.K).as_dict(),
                              "us_per_call": round(r["us_per_call"], 3), "GBps": round(r["gbs"], 1),
                              "pct_peak": round(100 * r["gbs"] / PEAK_HBM_GBS, 2), "sets": sets}), flush=True)
        del prob
        torch.cuda.empty_cache()


def sweep(torch, w4, args):
    for wname in ("qkv", "gate_up", "down", "lm_head"):
        wl = synth.WORKLOADS[wname]
        Ms = sorted(set(wl.Ms) | {1, 4, 8, 16})
        sets = sets_for(wl.K, wl.N, 1)
        prob = Problem(torch, w4, wl.K, wl.N, wl.seed, wl.act, sets)
        for M in Ms:
            steps = graph_steps(args, synth.algorithmic_bytes(M, wl.N, wl.K))
            r = measure(torch, w4, prob, M, steps, min(args.warmup, 20))
            rec = {"workload": wname, "M": M, "K": wl.K, "N": wl.N, "plan": w4.get_plan(M, wl.N, wl.K).as_dict(),
                   "us_per_call": round(r["us_per_call"], 3), "GBps": round(r["gbs"], 1),
                   "pct_peak": round(100 * r["gbs"] / PEAK_HBM_GBS, 2),
                   "mfma_util": round(r["tflops"] / PEAK_BF16_TFLOPS, 4), "sets": sets}
            print(json.dumps(rec), flush=True)
        if wname == "gate_up":
            # the same weights with the SiLU(gate) * up epilogue: H[M, N/2]
            for M in Ms:
                def fcall(i, M=M):
                    j = i % prob.sets
                    w4.gemm_silu_mul(prob.acts[j][:M], prob.blobs[j], prob.scales[j], prob.N,
                                     out=prob.houts[j][:M])
                steps = graph_steps(args, synth.algorithmic_bytes(M, wl.N, wl.K))
                ms = time_graph(torch, fcall, steps, min(args.warmup, 20))
                nb = synth.algorithmic_bytes_silu_mul(M, wl.N, wl.K)
                print(json.dumps({"workload": "gate_up_silu_mul", "M": M, "K": wl.K, "N": wl.N,
                                  "us_per_call": round(ms * 1e3, 3), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                                  "pct_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                                  "sets": sets}), flush=True)
        if wname == "lm_head":
            # the same weights with the row-argmax epilogue (the greedy pick)
            for M in Ms:
                def acall(i, M=M):
                    j = i % prob.sets
                    w4.gemm_argmax(prob.acts[j][:M], prob.blobs[j], prob.scales[j], prob.N)
                steps = graph_steps(args, synth.algorithmic_bytes(M, wl.N, wl.K))
                ms = time_graph(torch, acall, steps, min(args.warmup, 20))
                nb = synth.algorithmic_bytes_argmax(M, wl.N, wl.K)
                print(json.dumps({"workload": "lm_head_argmax", "M": M, "K": wl.K, "N": wl.N,
                                  "us_per_call": round(ms * 1e3, 3), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                                  "pct_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                                  "sets": sets}), flush=True)
        del prob
        torch.cuda.empty_cache()


def ceiling(torch, w4, args):
    """Best plain streaming-read bandwidth at the byte counts of the matmul calls.

    The read-only probe kernel (libw4a16_probe.so) is swept over launch shapes;
    buffers rotate over >= 1 GiB like the matmul timing, so every read comes
    from HBM.  One JSON line per byte count.
    """
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_int4_gptq_amd", "libw4a16_probe.so"))
    lib.w4a16_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    sink = torch.zeros(8192 * 1024, dtype=torch.int32, device=dev)
    sizes = [("qkv_m1", synth.algorithmic_bytes(1, 8192, 5120)),
             ("down_m1", synth.algorithmic_bytes(1, 5120, 17408)),
             ("gate_up_m1", synth.algorithmic_bytes(1, 34816, 5120)),
             ("lm_head_m1", synth.algorithmic_bytes(1, 248320, 5120)),
             ("2GiB", 2 << 30)]
    for tag, nbytes in sizes:
        nbytes = (nbytes + 15) // 16 * 16
        nbuf = max(1, -(-ROTATE_BYTES // nbytes)) if nbytes < 4 * LLC_BYTES else 1
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        best = None
        for blocks in (512, 1024, 2048, 4096, 8192):
            for threads in (256, 512, 1024):
                for unroll in (1, 4, 8):
                    if blocks * threads > sink.numel() or nbytes // 16 < blocks * threads // 4:
                        continue

                    def call(i, b=blocks, t=threads, u=unroll):
                        st = lib.w4a16_probe_stream_read(bufs[i % nbuf].data_ptr(), nbytes, b, t, u,
                                                         sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
                        if st != 0:
                            raise RuntimeError(f"probe launch failed ({st})")

                    steps = 100 if nbytes < 1e8 else (20 if nbytes < 1e9 else 5)
                    ms = time_graph(torch, call, steps, 3)
                    if best is None or ms < best[0]:
                        best = (ms, blocks, threads, unroll)
        ms, b, t, u = best
        print(json.dumps({"ceiling": tag, "bytes": nbytes, "us_per_call": round(ms * 1e3, 3),
                          "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "pct_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                          "launch": {"blocks": b, "threads": t, "unroll": u}, "buffer_sets": nbuf}), flush=True)
        del bufs
        torch.cuda.empty_cache()


def tp_shards(torch, w4, args):
    """One GPU's share of each decoder linear under tensor parallelism (TP = 2, 4, 8):
    column shards (QKV; gate/up with its activation) and K shards with fp32
    partial sums (attention output; down projection).  One JSON line per call."""
    dev = torch.device("cuda:0")
    shapes = [("qkv_cols", 5120, 8192, "cols"), ("o_rows", 6144, 5120, "rows"),
              ("gate_up_cols_silu_mul", 5120, 34816, "cols_silu"), ("down_rows", 17408, 5120, "rows")]
    for tp in (2, 4, 8):
        for name, K, N, kind in shapes:
            Ki, Ni = (K // tp, N) if kind == "rows" else (K, N // tp)
            sets = sets_for(Ki, Ni, 1)
            prob = Problem(torch, w4, Ki, Ni, Ki + Ni, "normal", sets)
            f32_outs = [torch.empty((16, Ni), dtype=torch.float32, device=dev) for _ in range(sets)] \
                if kind == "rows" else None
            for M in (1, 8):
                if kind == "rows":
                    def call(i, M=M):
                        j = i % sets
                        w4.gemm_f32(prob.acts[j][:M], prob.blobs[j], prob.scales[j], Ni, out=f32_outs[j][:M])
                    nb = synth.algorithmic_bytes_f32(M, Ni, Ki)
                elif kind == "cols_silu":
                    def call(i, M=M):
                        j = i % sets
                        w4.gemm_silu_mul(prob.acts[j][:M], prob.blobs[j], prob.scales[j], Ni, out=prob.houts[j][:M])
                    nb = synth.algorithmic_bytes_silu_mul(M, Ni, Ki)
                else:
                    def call(i, M=M):
                        prob.call(w4, M, i)
                    nb = synth.algorithmic_bytes(M, Ni, Ki)
                steps = graph_steps(args, nb)
                ms = time_graph(torch, call, steps, min(args.warmup, 20))
                print(json.dumps({"tp": tp, "call": name, "M": M, "K": Ki, "N": Ni,
                                  "us_per_call": round(ms * 1e3, 3), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                                  "pct_peak": round(100 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}), flush=True)
            del prob, f32_outs
            torch.cuda.empty_cache()


def stack(torch, w4, args, quiet=False):
    """One decode step: 64 layers x (attn-in, attn-out, gate/up, down) + lm_head, all resident.

    Every layer has its own weights (11.9 GB in all, far beyond the 256 MiB
    last-level cache); one step is the 257 calls in order, at M = 1 and 8.
    Returns one record per M (and prints it unless quiet).
    """
    probs = {}
    for (K, N) in set(synth.STACK_LAYER_SHAPES) | {synth.LM_HEAD_SHAPE}:
        probs[(K, N)] = Problem(torch, w4, K, N, K + N, "normal", 1)
    layers = []
    for li in range(synth.STACK_LAYERS):
        for (K, N) in synth.STACK_LAYER_SHAPES:
            p = probs[(K, N)]
            blob = p.blobs[0] if li == 0 else p.blobs[0].clone()
            sc = p.scales[0] if li == 0 else p.scales[0].clone()
            layers.append((K, N, blob, sc, p.acts[0], p.outs[0]))
    K, N = synth.LM_HEAD_SHAPE
    p = probs[(K, N)]
    layers.append((K, N, p.blobs[0], p.scales[0], p.acts[0], p.outs[0]))
    recs = []
    for M in (1, 8):
        total = sum(synth.algorithmic_bytes(M, N, K) for (K, N, *_ ) in layers)

        def step(_i, M=M):
            for (K, N, blob, sc, a, o) in layers:
                w4.gemm(a[:M], blob, sc, N, out=o[:M])

        ms = time_graph(torch, step, 3, 2)
        rec = {"stack": "64 layers x 4 linear shapes + lm_head", "M": M, "calls": len(layers),
               "bytes": total, "ms_per_step": round(ms, 4),
               "GBps": round(total / (ms * 1e-3) / 1e9, 1),
               "pct_peak": round(100 * total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
        recs.append(rec)
        if not quiet:
            print(json.dumps(rec), flush=True)
    del layers, probs, p
    torch.cuda.empty_cache()
    return recs


if __name__ == "__main__":
    main()
