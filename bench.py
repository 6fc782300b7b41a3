"""Benchmark of the Recurrent Transformer prefill on one MI355X.

One step = the forward pass x -> z of the whole 6-layer RT stack at B=512,
N=2048, d_model=1024 (16 heads x 64), MLP 4096, bf16, over one batch of seeded
synthetic input resident in HBM: one HIP-graph replay of the stack plan, whose
layers run as a wavefront (each layer's per-position products share launches
with the other layers'; per layer and position: the fused blocked update +
finalize, output projection, MLP, persistent K/V projection; the queries and
ephemeral pairs projected in chunks). --per-layer replays one graph per layer
instead, one layer after another.

Prints one JSON line. value = tokens/s of the stack (B*N tokens per step).
roofline = the blocked-update kernel (the method's core, HBM-bound): its
algorithmic bytes per launch over its average launch duration; that average
is one layer's 2047 update launches captured as a HIP graph and replayed,
timed with HIP events on the launch stream around the replays.
cpu_baseline = the CPU oracle (naive schedule, fp64) on a bounded sample.
mfma_util = the layer's algorithmic products and update flops over the layer time
(the metric's MFMA utilisation, at the layer level).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RT layer prefill tokens/s at B=512 + blocked-update HBM GB/s / MFMA util"
HBM_PEAK_GBS = 8000.0
# the oracle timed as the CPU baseline, as it stands (oracle/build.py)
ORACLE_BUILD = ("oracle/rt_oracle.c, naive schedule, IEEE fp64 with bf16 storage emulation; "
                "gcc -O3 -ffp-contract=off -fopenmp, no -march flags; one OpenMP thread per core")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def update_bytes(t, n, p, dh, s):
    """Algorithmic HBM bytes of the fused update step t (1-based): KV block,
    queries, state read (not on first touch) and write (not for the finished
    row), and the finished row's ephemeral pair and output."""
    b = t & -t
    nq = min(b, n - t)
    if nq <= 0:
        return 0
    kv = b * p * dh * s * 2
    q = nq * p * dh * s
    st_row = p * (dh + 2) * 4
    reads = 0 if b == t else nq * st_row
    writes = (nq - 1) * st_row
    fin = 3 * p * dh * s
    return kv + q + reads + writes + fin


def update_flops(t, n, p, dh):
    b = t & -t
    nq = min(b, n - t)
    return 4 * dh * b * nq * p + 4 * dh * p  # block scores + PV, plus the ephemeral pair


TRAFFIC_WORKLOAD = "stack6_d1024_b512_n2048"  # the workload whose update launches the counters measured


def measured_traffic(workload):
    """HBM bytes per update launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None for another workload's launches, or when the update kernel's source has changed
    since those counters were taken."""
    if workload != TRAFFIC_WORKLOAD:
        return None
    import hashlib
    prof = os.path.join(ROOT, "profiles", "update_kernel_hbm_traffic_stack6_d1024_b512_n2048.txt")
    src = os.path.join(ROOT, "blocked_prefill_amd", "csrc", "update.hip")
    try:
        kv = dict(ln.split("=", 1) for ln in open(prof) if "=" in ln and not ln.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv["source_sha256"]:
            return None
        return int(kv["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def traffic_summary(fetch_dir, write_dir):
    """Summary of two rocprofv3 counter passes over `bench.py --counters` (FETCH_SIZE,
    then WRITE_SIZE; KiB per dispatch): each counter calibrated on the run's final
    1 GiB device copy, then averaged over the 2047 update launches just before it.
    Prints the text kept under profiles/ (with the update kernels' source hash)."""
    import csv
    import hashlib

    def rows(d, counter):
        out = []
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return sorted(out)

    fetch, write = rows(fetch_dir, "FETCH_SIZE"), rows(write_dir, "WRITE_SIZE")
    copy_bytes = 1 << 30

    def calibrate(rs):
        i = max(k for k, (_, name, _) in enumerate(rs) if "copy" in name.lower())
        factor = copy_bytes / (rs[i][2] * 1024)
        ups = [v for _, name, v in rs[:i] if "update_" in name][-2047:]
        return factor, rs[i][2], ups

    ff, fk, fu = calibrate(fetch)
    wf, wk, wu = calibrate(write)
    assert len(fu) == len(wu) == 2047, (len(fu), len(wu))
    N, P, dh, s_ = 2048, 512 * 16, 64, 2
    meas = [fu[t - 1] * 1024 * ff + wu[t - 1] * 1024 * wf for t in range(1, N)]
    alg = [update_bytes(t, N, P, dh, s_) for t in range(1, N)]
    rd = sum(fu) * 1024 * ff / 2047
    wr = sum(wu) * 1024 * wf / 2047
    src = os.path.join(ROOT, "blocked_prefill_amd", "csrc", "update.hip")
    per_b = []
    b = 1
    while b < N:
        ts = [t for t in range(1, N) if t & -t == b]
        per_b.append(f"b={b} {sum(meas[t - 1] for t in ts) / sum(alg[t - 1] for t in ts):.3f}")
        b *= 2
    lines = [
        "# HBM traffic of the fused blocked-update kernels, one layer of the 6-layer stack workload",
        "# (B=512, N=2048, d_model=1024, 16 heads x 64, bf16): 2047 launches (t = 1..2047).",
        "#",
        "# Commands (repository root, one MI355X; two passes, one counter each; then the summary):",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/fetch -o run -- python3 bench.py --counters",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/write -o run -- python3 bench.py --counters",
        "#   python3 bench.py --traffic-summary gpurun_out/fetch gpurun_out/write",
        "# bench.py --counters fills q, k', v' and the persistent caches with random values, runs",
        "# the layer's 2047 update launches t = 1..2047 (the ones counted here), then a plain",
        "# 1 GiB device copy (the calibration kernel).",
        "#",
        f"# Calibration on the 1 GiB copy ({copy_bytes} bytes read, {copy_bytes} written):",
        f"#   FETCH_SIZE = {fk:.0f} KiB  -> bytes read    = FETCH_SIZE * 1024 * {ff:.4f}",
        f"#   WRITE_SIZE = {wk:.0f} KiB  -> bytes written = WRITE_SIZE * 1024 * {wf:.4f}",
        "#",
        "# Per launch, averaged over the 2047 update launches (calibrated):",
        f"#   read {rd / 1e6:.2f} MB + written {wr / 1e6:.2f} MB = {(rd + wr) / 1e6:.2f} MB;  algorithmic model "
        f"{sum(alg) / 2047 / 1e6:.2f} MB;  ratio {(rd + wr) / (sum(alg) / 2047):.3f}",
        "# Per block size b (measured / algorithmic):",
        "#   " + "  ".join(per_b[:6]),
        "#   " + "  ".join(per_b[6:]),
        "#",
        "# Kernel source these counters were taken on (bench.py reports traffic only while it matches):",
        f"source_sha256 = {hashlib.sha256(open(src, 'rb').read()).hexdigest()}",
        f"bytes_per_launch = {round(rd + wr, -4):.0f}",
    ]
    print("\n".join(lines))


UPDATE_COUNTER_PASSES = [
    # one rocprofv3 --pmc pass each over `bench.py --counters` (at most 8 SQ counters per pass)
    "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_LDS SQ_INSTS_VALU_TRANS_F32",
    "GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VMEM_RD "
    "SQ_INSTS_VMEM_WR SQ_ACTIVE_INST_VMEM SQ_WAVES TA_BUSY_avr TCP_TCC_READ_REQ_sum TCP_TCC_WRITE_REQ_sum",
]


def counter_summary(dirs):
    """Per block size b, the update launches of `bench.py --counters` (t = 1..2047 of the
    stack workload's layer) from the rocprofv3 counter passes of UPDATE_COUNTER_PASSES, one
    directory per pass: time from the dispatch timestamps, the clock the CUs actually ran at,
    the vector ALU, matrix core, LDS and memory shares of the SIMDs' cycles, and instruction
    counts per step. Prints the text kept under profiles/."""
    import csv
    N, P = 2048, 512 * 16
    vals = {}  # (dispatch index among update launches, counter) -> value (one pass per counter)
    dur = {}   # dispatch index -> durations (ns) over the passes
    for d in dirs:
        rows = {}
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if "update_" not in r["Kernel_Name"]:
                continue
            e = rows.setdefault(int(r["Dispatch_Id"]), {})
            e[r["Counter_Name"]] = float(r["Counter_Value"])
            e["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        ids = sorted(rows)[-(N - 1):]  # the last 2047 update launches: the sequence t = 1..2047
        assert len(ids) == N - 1, (d, len(ids))
        for i, key in enumerate(ids):
            for c, v in rows[key].items():
                if c == "_ns":
                    dur.setdefault(i, []).append(v)
                elif (i, c) not in vals:
                    vals[(i, c)] = v
    simds = 1024
    lines = [
        "# Hardware counters of the blocked-update launches, one layer of the 6-layer stack workload",
        "# (B=512, N=2048, d_model=1024, 16 heads x 64, bf16): the 2047 launches t = 1..2047, by block size.",
        "#",
        "# Commands (repository root, one MI355X; one counter pass each; then the summary):",
    ]
    for i, ps in enumerate(UPDATE_COUNTER_PASSES):
        lines.append(f"#   rocprofv3 --pmc {ps} --output-format csv -d gpurun_out/upc{i} -o run -- "
                     "python3 bench.py --counters")
    lines += [
        "#   python3 bench.py --counter-summary " + " ".join(f"gpurun_out/upc{i}" for i in range(len(dirs))),
        "# (counter mode serialises the launches: times are those of single dispatches)",
        "#",
        "# us/step: End - Start timestamp of the dispatch, mean over the passes.",
        "# MHz: the clock the CUs ran at, SQ_BUSY_CU_CYCLES / 256 CUs / time (the counter sums the busy",
        "#   cycles of every CU; GRBM_GUI_ACTIVE / 8 XCDs gives the same within 2% on the large launches,",
        "#   while on launches of a few us it also counts the counters' own set-up).",
        "# Shares of the SIMDs' cycles (4 x SQ_BUSY_CU_CYCLES):",
        "#   valu = SQ_ACTIVE_INST_VALU x 4 (the counter is in units of 4 cycles);",
        "#   mfma = SQ_VALU_MFMA_BUSY_CYCLES (32 cycles per 32x32x16 bf16 MFMA); coexec = the part of",
        "#   the mfma cycles during which the SIMD also issued vector ALU work, SQ_VALU_MFMA_COEXEC_CYCLES;",
        "#   lds = SQ_ACTIVE_INST_LDS x 4; waves = SQ_WAVE_CYCLES x 4 / SIMD cycles (resident waves per",
        "#   SIMD); wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (resident wave time spent waiting on a memory",
        "#   or LDS result); ta = TA_BUSY_avr / per-CU cycles (address unit busy).",
        "# Per step: vector (MFMA included), transcendental (exp2), matrix, LDS, memory-read and -write",
        "#   instructions (wave level); LDS bank-conflict cycles per LDS instruction; L2 read / write",
        "#   requests per KB of algorithmic traffic.",
        "",
        "| b | steps | us/step | MHz | valu | mfma | coexec | lds | waves | wait | ta | VALU/step | TRANS | MFMA "
        "| LDS | VMEM rd | VMEM wr | bank confl/LDS inst | L2 rd req/KB | L2 wr req/KB |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    b = 1
    while b < N:
        ts = [t for t in range(1, N) if t & -t == b]
        get = lambda c: sum(vals.get((t - 1, c), 0.0) for t in ts)
        secs = sum(sum(dur[t - 1]) / len(dur[t - 1]) for t in ts) * 1e-9
        cu_cyc = max(get("SQ_BUSY_CU_CYCLES"), 1.0)   # summed over the 256 CUs
        simd_cyc = 4 * cu_cyc
        byts = sum(update_bytes(t, N, P, 64, 2) for t in ts)
        n = len(ts)
        row = [f"{b}", f"{n}", f"{secs / n * 1e6:.1f}", f"{simd_cyc / simds / secs / 1e6:.0f}",
               f"{get('SQ_ACTIVE_INST_VALU') * 4 / simd_cyc:.2f}", f"{get('SQ_VALU_MFMA_BUSY_CYCLES') / simd_cyc:.2f}",
               f"{get('SQ_VALU_MFMA_COEXEC_CYCLES') / simd_cyc:.2f}",
               f"{get('SQ_ACTIVE_INST_LDS') * 4 / simd_cyc:.2f}",
               f"{get('SQ_WAVE_CYCLES') * 4 / simd_cyc:.2f}",
               f"{get('SQ_WAIT_INST_ANY') / max(get('SQ_WAVE_CYCLES'), 1):.2f}",
               f"{get('TA_BUSY_avr') / (cu_cyc / 256):.2f}",
               f"{get('SQ_INSTS_VALU') / n:.3g}", f"{get('SQ_INSTS_VALU_TRANS_F32') / n:.3g}",
               f"{get('SQ_INSTS_MFMA') / n:.3g}", f"{get('SQ_INSTS_LDS') / n:.3g}",
               f"{get('SQ_INSTS_VMEM_RD') / n:.3g}", f"{get('SQ_INSTS_VMEM_WR') / n:.3g}",
               f"{get('SQ_LDS_BANK_CONFLICT') / max(get('SQ_INSTS_LDS'), 1):.2f}",
               f"{get('TCP_TCC_READ_REQ_sum') / (byts / 1024):.2f}",
               f"{get('TCP_TCC_WRITE_REQ_sum') / (byts / 1024):.2f}"]
        lines.append("| " + " | ".join(row) + " |")
        b *= 2
    print("\n".join(lines))


FAMILY_COUNTERS = ("GRBM_GUI_ACTIVE SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES "
                   "SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_INSTS_MFMA SQ_INSTS_VALU")


def _kernel_family(name, grid):
    """A short label for a kernel of the stack (template arguments: FLAGS first for the GEMMs)."""
    import re
    m = re.search(r"<([^<>]*)>\(", name)
    args = [a.strip() for a in m.group(1).split(",")] if m else re.findall(r"Li(\d+)E", name)
    ints = [int(a) for a in args if a.lstrip("-").isdigit()]
    if "gemm_pipe" in name and ints:
        flags, shape = ints[0], "x".join(str(v) for v in ints[1:3])
        kind = {20: "W_2", 10: "W_1", 8: "W_kv or QKV", 52: "W_o", 392: "W_kv + small step",
                24: "W_2", 40: "W_o"}.get(flags & 1023, f"flags {flags & 1023}")
        how = ("grouped " if "group" in name else "") + kind + f" {shape}"
        if flags & 1024:
            how += ", K tiles to LDS directly"
        if flags & 2048:
            how += ", XCD-grouped"
        return how
    for k in ("update_small_group", "update_small", "update_simt", "update_mfma_multi", "update_mfma", "row_sumsq"):
        if k in name:
            return k + (f"<{','.join(str(v) for v in ints[:2])}>" if k == "update_mfma" else "")
    return name[:60]


def family_summary(dirs):
    """MFMA and vector-ALU shares per kernel family of one eager stack forward, from one rocprofv3
    pass of FAMILY_COUNTERS over `bench.py --eager --steps 1 --warmup 0 --no-cpu --no-kernel-timing`.
    Time from the dispatch timestamps; SIMD cycles = 4 x SQ_BUSY_CU_CYCLES (the busy cycles of
    the CUs that had work, at the clock they ran at)."""
    import collections
    import csv
    fam = collections.defaultdict(lambda: collections.defaultdict(float))
    seen = set()
    for d in dirs:
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            name = r["Kernel_Name"]
            if "rt::" not in name and "_ZN2rt" not in name:
                continue
            f = fam[_kernel_family(name, int(r["Grid_Size"]))]
            f[r["Counter_Name"]] += float(r["Counter_Value"])
            key = (d, r["Dispatch_Id"])
            if key not in seen:
                seen.add(key)
                f["_n"] += 1
                f["_ns"] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    lines = [
        "| family | dispatches | ms | MHz | MFMA busy | VALU busy | waves/SIMD | wait any | wait LDS |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    for name, f in sorted(fam.items(), key=lambda kv: -kv[1]["_ns"]):
        cu = max(f["SQ_BUSY_CU_CYCLES"], 1.0)
        simd = 4 * cu
        secs = f["_ns"] * 1e-9
        wc = max(f["SQ_WAVE_CYCLES"], 1.0)
        lines.append(f"| {name} | {f['_n']:.0f} | {secs * 1e3:.2f} | {cu / 256 / max(secs, 1e-12) / 1e6:.0f} | "
                     f"{f['SQ_VALU_MFMA_BUSY_CYCLES'] / simd:.3f} | {f['SQ_ACTIVE_INST_VALU'] * 4 / simd:.3f} | "
                     f"{wc * 4 / simd:.2f} | {f['SQ_WAIT_INST_ANY'] / wc:.2f} | {f['SQ_WAIT_INST_LDS'] / wc:.2f} |")
    print("\n".join(lines))


def trace_summary(d, replays):
    """Tables from a rocprofv3 --kernel-trace --stats run of the stack bench (`replays` plan replays:
    warm-up + timed steps): kernels by total time, and per family the launches inside the plan
    replays, per replay, with the average of the grouped products' six-layer launches (grid z = 6)."""
    import collections
    import csv
    import gzip
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    out = ["| kernel (family) | calls | total ms | avg us | % |", "|---|---|---|---|---|"]
    for r in rows[:16]:
        out.append(f"| {_kernel_family(r['Name'], 0)} | {r['Calls']} | {int(r['TotalDurationNs']) / 1e6:.2f} | "
                   f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    tp = os.path.join(d, "run_kernel_trace.csv")
    f = gzip.open(tp + ".gz", "rt") if os.path.exists(tp + ".gz") else open(tp)
    tr = [r for r in csv.DictReader(f) if "rt::" in r["Kernel_Name"] or "_ZN2rt" in r["Kernel_Name"]]
    # the replays' window: from layer 0's row sums of all N*B rows (a replay's first launch)
    # to the end of the last product
    first = [int(r["Start_Timestamp"]) for r in tr
             if "row_sumsq" in r["Kernel_Name"] and int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) >= 1 << 26]
    ends = [int(r["End_Timestamp"]) for r in tr if "gemm_pipe" in r["Kernel_Name"]]
    if first and ends:
        lo, hi = min(first), max(ends)
        fam = collections.defaultdict(lambda: [0, 0.0, 0, 0.0])
        t0, t1 = None, None
        for r in tr:
            st, en = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            if st < lo or st > hi:
                continue
            t0 = st if t0 is None else min(t0, st)
            t1 = en if t1 is None else max(t1, en)
            e = fam[_kernel_family(r["Kernel_Name"], 0)]
            e[0] += 1
            e[1] += (en - st) * 1e-3
            if int(r["Grid_Size_Z"]) == 6:
                e[2] += 1
                e[3] += (en - st) * 1e-3
        out += ["", f"Inside the {replays} plan replays ({(t1 - t0) / 1e6:.1f} ms from the first launch to the last product), "
                    "per replay:", "",
                "| family | launches | ms | avg us | six-layer launches | their avg us |", "|---|---|---|---|---|---|"]
        for k, (n, us, n6, us6) in sorted(fam.items(), key=lambda kv: -kv[1][1]):
            out.append(f"| {k} | {n // replays} | {us / 1e3 / replays:.2f} | {us / n:.2f} | {n6 // replays} | "
                       f"{(us6 / n6) if n6 else float('nan'):.2f} |")
    print("\n".join(out))


def update_sequence(rt, attn, ws, k_cache, v_cache, N, B, H, D, stream, timing_torch, sync=True, t_range=None):
    """Replay one layer's fused update steps t = 1..N-1 on the workspace's q, k', v' and state
    (offsets as laid out by the library: q, k', v', m, l, o first). With timing_torch, each
    launch is bracketed by HIP events on the launch stream; returns per-launch ms."""
    import numpy as np
    import torch
    base = ws.data_ptr()
    es, al = 2, lambda v: (v + 255) // 256 * 256
    off_q = 0
    off_ke = off_q + al(N * B * D * es)
    off_ve = off_ke + al(N * B * D * es)
    off_m = off_ve + al(N * B * D * es)
    off_l = off_m + al(N * B * H * 4)
    off_o = off_l + al(N * B * H * 4)
    a_next = torch.empty((B, D), dtype=torch.bfloat16, device=k_cache.device)
    timed = timing_torch is not None
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(N - 1)] if timed else None
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(N - 1)] if timed else None
    if sync:
        torch.cuda.synchronize()
    for t in range(*(t_range or (1, N))):
        if timed:
            starts[t - 1].record(stream)
        rt.rt_update_finalize_step(attn, t, base + off_q, base + off_ke, base + off_ve, k_cache, v_cache,
                                   base + off_m, base + off_l, base + off_o, a_next, stream)
        if timed:
            ends[t - 1].record(stream)
    if sync:
        torch.cuda.synchronize()
    if not timed:
        return None
    return np.array([s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)])  # ms


def cpu_model():
    """The host CPU's model name (Linux), for the oracle's timing."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stream_probe():
    """The bandwidth probes' library (blocked_prefill_amd/librt_probe.so), or None."""
    import ctypes
    path = os.path.join(ROOT, "blocked_prefill_amd", "librt_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.rt_probe_stream.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                            ctypes.c_void_p]
    lib.rt_probe_stream.restype = ctypes.c_int
    return lib


def ceilings(dev):
    """Achievable ceilings of this GPU, measured beside the product as reference
    points for the roofline fractions (not part of the path): torch's device
    copy of 2 GiB (read once, written once); the library's streaming probe with
    three 1 GiB streams read and one written (the blocked update's ~3:1
    read:write mix) and with one read and one written; and torch's bf16
    product of two 8192 x 8192 matrices (hipBLASLt). Timed with events on
    torch's stream, mean of 5 after 2."""
    import torch
    stream = torch.cuda.current_stream()

    def timed(f):
        for _ in range(2):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 5 / 1e3

    n = 1 << 30
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    copy_gbs = 2 * 2 * n / timed(lambda: dst.copy_(src)) / 1e9
    del src, dst
    probe = stream_probe()
    stream_gbs = {}
    if probe is not None:
        n16 = (1 << 30) // 16
        bufs = [torch.empty(1 << 30, dtype=torch.uint8, device=dev) for _ in range(4)]
        for b_ in bufs:
            b_.fill_(7)
        ptr = [b_.data_ptr() for b_ in bufs]
        for reads in (3, 1):  # the best of a few grid sizes
            for blocks in (1024, 2048, 4096, 8192):
                def run(reads=reads, blocks=blocks):
                    rc = probe.rt_probe_stream(ptr[0], ptr[1], ptr[2], ptr[3], n16, reads, blocks, stream.cuda_stream)
                    assert rc == 0, rc
                gbs = (reads + 1) * (1 << 30) / timed(run) / 1e9
                stream_gbs[reads] = max(stream_gbs.get(reads, 0.0), gbs)
        del bufs
    k = 8192
    a = torch.randn((k, k), dtype=torch.bfloat16, device=dev)
    b = torch.randn((k, k), dtype=torch.bfloat16, device=dev)
    c = torch.empty((k, k), dtype=torch.bfloat16, device=dev)
    gemm_tflops = 2.0 * k ** 3 / timed(lambda: torch.matmul(a, b, out=c)) / 1e12
    del a, b, c
    torch.cuda.synchronize()
    log(f"ceilings: device copy {copy_gbs:.0f} GB/s, streams 3:1 {stream_gbs.get(3, 0):.0f} GB/s, "
        f"1:1 {stream_gbs.get(1, 0):.0f} GB/s, bf16 8192^3 product {gemm_tflops:.0f} TFLOP/s")
    return {"copy_GB_s": round(copy_gbs, 1), "stream_3r1w_GB_s": round(stream_gbs.get(3, 0.0), 1),
            "stream_1r1w_GB_s": round(stream_gbs.get(1, 0.0), 1), "gemm_TFLOP_s": round(gemm_tflops, 1),
            "measured": "torch device copy of 2 GiB (read + write); the library's streaming probe, three "
                        "1 GiB streams read and one written, and one read and one written; torch bf16 "
                        "8192^3 matmul"}


def update_only_bench(args, rt, wl):
    """The isolated blocked update (no layer around it): one step = the whole
    sequence's blocked attention with every pair known up front (rt_attn_forward:
    position 1, then each level of the schedule in one launch), replayed as one
    HIP graph on seeded q, k', v', k, v resident in HBM. value = B*N / step
    time; roofline = the steps' algorithmic bytes over the step time."""
    import numpy as np
    import torch
    import oracle
    import rt_inputs
    N, B, H, dh = wl.n_pos, wl.batch, wl.n_heads, wl.head_dim
    D, P = H * dh, B * H
    scale = 1.0 / math.sqrt(dh)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    t_np = rt_inputs.attn_inputs(wl)
    bf = {k: torch.from_numpy(v.reshape(N, B, D)).to(torch.bfloat16).to(dev) for k, v in t_np.items()}
    del t_np
    m = torch.empty((N, B, H), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    o = torch.empty((N, B, D), dtype=torch.float32, device=dev)
    a = torch.empty((N, B, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((N, B, H), dtype=torch.float32, device=dev)
    desc = rt.AttnDesc(batch=B, seq_len=N, n_heads=H, head_dim=dh, dtype=rt.RT_BF16, softmax_scale=scale)
    levels = 1 + max(0, (N - 1).bit_length())  # position 1's finalize + one launch per block size

    def sequence(st):
        rt.rt_attn_forward(desc, bf["q"], bf["k_eph"], bf["v_eph"], bf["k"], bf["v"], a, lse, m, l, o, st)

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            sequence(cap)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        g.replay()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tokens_per_s = B * N / (ms / 1e3)
    assert bool(torch.isfinite(a).all()), "non-finite output"
    byts = np.array([update_bytes(t, N, P, dh, 2) for t in range(1, N)], dtype=np.float64)
    flops = np.array([update_flops(t, N, P, dh) for t in range(1, N)], dtype=np.float64)
    avg_s = ms / 1e3 / levels
    achieved = byts.sum() / (ms / 1e3) / 1e9
    log(f"timed {args.steps} steps: {ms:.3f} ms/step, {tokens_per_s / 1e6:.3f} M tokens/s, "
        f"{achieved:.0f} GB/s algorithmic ({achieved / HBM_PEAK_GBS:.1%} of HBM peak)")
    cpu = None
    if not args.no_cpu:
        rows = list(range(min(args.cpu_rows or oracle.num_threads(), B)))
        tr = rt_inputs.attn_inputs(wl, rows=rows)
        t0 = time.time()
        oracle.attention(tr["q"], tr["k_eph"], tr["v_eph"], tr["k"], tr["v"], scale)
        cpu_s = time.time() - t0
        cpu = {"value": round(len(rows) * N / cpu_s, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
               "kind": "oracle", "build": ORACLE_BUILD,
               "sample": f"{len(rows)} batch rows x all {N} positions ({cpu_s:.1f} s)"}
        log(f"cpu oracle: {cpu_s:.1f}s for the sample")
    ceil = None if args.no_kernel_timing else ceilings(dev)
    if ceil:
        ceil["update_frac_of_copy"] = round(achieved / ceil["copy_GB_s"], 4)
        if ceil["stream_3r1w_GB_s"]:
            ceil["update_frac_of_stream_3r1w"] = round(achieved / ceil["stream_3r1w_GB_s"], 4)
    out = {
        "metric": "blocked-update tokens/s (isolated update, HBM GB/s)", "value": round(tokens_per_s, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k', v', k, v)",
        "config": {"workload": f"{wl.name}: isolated blocked update, bf16 inputs, fp32 state, B={B}, "
                               f"{H} heads x {dh}, N={N}", "batch": B, "seq_len": N},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "fused blocked update + finalize, one launch per level", "launches": levels,
                     "avg_launch_us": round(avg_s * 1e6, 2), "alg_bytes_per_launch": int(byts.sum() / levels)},
        "mfma_util": {"scope": "the update's scores and values (4*dh flops per visited (query, key) pair)",
                      "achieved_TFLOP_s": round(flops.sum() / (ms / 1e3) / 1e12, 1), "peak_TFLOP_s": 2500.0,
                      "frac": round(flops.sum() / (ms / 1e3) / 1e12 / 2500.0, 4)},
        "cpu_baseline": cpu,
        "ceilings": ceil,
    }
    print(json.dumps(out), flush=True)


SWEEP_VARIANTS = {"rt_blocked": 0, "rt_naive": 2, "transformer": 4}  # rt_layer_desc flags


def _sweep_layer(rt, n, flags, dev, stream, warm, reps):
    """Mean ms of `reps` graph replays of one layer (B=512, d=1024, 16x64 heads,
    MLP 4096, bf16) after `warm` replays."""
    import torch
    import rt_inputs
    wl = rt_inputs.Workload(f"sweep_n{n}", 512, n, 1024, 16, 64, 4096, 1, "bf16", 1003)
    x = torch.from_numpy(rt_inputs.layer_input(wl)).to(torch.bfloat16).to(dev)
    w = rt_inputs.layer_weights(wl, 0)
    w = {k: torch.from_numpy(w[k]).to(torch.bfloat16).to(dev) for k in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    attn = rt.AttnDesc(batch=512, seq_len=n, n_heads=16, head_dim=64, dtype=rt.RT_BF16, softmax_scale=0.125)
    desc = rt.LayerDesc(attn=attn, d_model=1024, d_ff=4096, rms_eps=1e-6, residual_scale=1.0, flags=flags)
    ws = torch.empty(rt.rt_layer_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    z, kc, vc = (torch.empty((n, 512, 1024), dtype=torch.bfloat16, device=dev) for _ in range(3))
    plan = rt.rt_layer_plan_create(desc, w, x, z, kc, vc, ws)
    for _ in range(warm):
        plan.launch(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        plan.launch(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    plan.destroy()
    return e0.elapsed_time(e1) / reps


def sweep(args):
    """Single-layer forward latency against N = 256..2048 at B=512, d=1024 for the
    RT layer under the blocked and the naive schedule and for the standard
    Transformer layer (the three curves of the translated paper's Figure 4), and
    each curve's log-log slope."""
    import numpy as np
    import torch

    import blocked_prefill_amd as rt
    rt.load()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    ns = (256, 512, 1024, 2048)
    res = {}
    for name, flags in SWEEP_VARIANTS.items():
        res[name] = {}
        for n in ns:
            slow = name == "rt_naive" and n >= 1024
            res[name][n] = _sweep_layer(rt, n, flags, dev, stream, 1 if slow else 3, 2 if slow else 5)
            log(f"sweep {name} N={n}: {res[name][n]:.2f} ms per layer")
    out = {"sweep": "single layer forward, bf16, B=512, d=1024, 16x64 heads, MLP 4096",
           "ms_per_layer": {k: {str(n): round(v[n], 3) for n in ns} for k, v in res.items()},
           "loglog_slope": {k: round(float(np.polyfit(np.log(ns), np.log([v[n] for n in ns]), 1)[0]), 3)
                            for k, v in res.items()}}
    print(json.dumps(out))


def backward(args):
    """Attention backward of the blocked schedule at the layer's attention shape
    (B=512, 16 heads x 64, N=2048, bf16 inputs, fp32 gradients): rt_attn_forward
    (saving the log-sum-exp) once, then rt_attn_backward timed (mean of 3 after 1).
    Algorithmic work: every causal (key, query) pair once, 10*dh flops (scores and
    value products recomputed, then the q, k, v gradient products), plus the
    per-query pass."""
    import torch

    import blocked_prefill_amd as rt
    import rt_inputs
    rt.load()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    B, H, dh, N = 512, 16, 64, 2048
    wl = rt_inputs.Workload("attn_b512_n2048", B, N, H * dh, H, dh, 0, 0, "bf16", 1003, update_only=True)
    t = rt_inputs.attn_inputs(wl)
    bf = {k: torch.from_numpy(t[k]).to(torch.bfloat16).to(dev) for k in ("q", "k_eph", "v_eph", "k", "v")}
    del t
    f32 = dict(dtype=torch.float32, device=dev)
    desc = rt.AttnDesc(batch=B, seq_len=N, n_heads=H, head_dim=dh, dtype=rt.RT_BF16, softmax_scale=0.125)
    a = torch.empty_like(bf["q"])
    lse, m, l = (torch.empty((N, B, H), **f32) for _ in range(3))
    o = torch.empty((N, B, H, dh), **f32)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rt.rt_attn_forward(desc, bf["q"], bf["k_eph"], bf["v_eph"], bf["k"], bf["v"], a, lse, m, l, o, stream=stream)
    e0.record(stream)
    rt.rt_attn_forward(desc, bf["q"], bf["k_eph"], bf["v_eph"], bf["k"], bf["v"], a, lse, m, l, o, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1)
    del m, l, o
    a_bar = torch.randn((N, B, H, dh), generator=torch.Generator(device=dev).manual_seed(5), **f32)
    outs = [torch.empty((N, B, H, dh), **f32) for _ in range(5)]
    delta = torch.empty((N, B, H), **f32)
    call = lambda: rt.rt_attn_backward(desc, bf["q"], bf["k_eph"], bf["v_eph"], bf["k"], bf["v"], a, lse, a_bar,
                                       *outs, delta, stream=stream)
    call()
    torch.cuda.synchronize()
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    P = B * H
    flops = 10.0 * dh * P * (N * (N - 1) / 2) + 12.0 * dh * P * N
    print(json.dumps({"backward": "blocked-schedule attention backward, B=512, 16x64 heads, N=2048, bf16 inputs",
                      "ms": round(ms, 3), "forward_with_lse_ms": round(fwd_ms, 3),
                      "tokens_per_s": round(B * N / (ms * 1e-3), 1),
                      "alg_TFLOP": round(flops / 1e12, 3), "TFLOP_s": round(flops / (ms * 1e-3) / 1e12, 2),
                      "bound": "mfma", "peak_TFLOP_s": 2500.0,
                      "frac": round(flops / (ms * 1e-3) / 1e12 / 2500.0, 4)}))


def layer_backward_bench(args):
    """The RT layer's backward (rt_layer_backward) at the stack workload's layer
    shape (B=512, N=2048, d=1024, 16x64 heads, F=4096, bf16): one layer forward
    (its stored output z), then the backward timed (mean of 2 after 1 warm-up),
    with z_bar ~ N(0,1). Algorithmic work: the batched recompute (projections
    of x and z, W_o, W_1, the attention with its log-sum-exp), the per-position
    adjoint products (W_kv^T, W_2^T, W_1^T, W_o^T), the attention backward, the
    batched input adjoint and the weight gradients."""
    import torch

    import blocked_prefill_amd as rt
    import rt_inputs
    rt.load()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    wl = rt_inputs.WORKLOADS["stack6_d1024_b512_n2048"]
    N, B, D, H, dh, F = wl.n_pos, wl.batch, wl.d_model, wl.n_heads, wl.head_dim, wl.d_ff
    x = torch.from_numpy(rt_inputs.layer_input(wl)).to(torch.bfloat16).to(dev)
    w = rt_inputs.layer_weights(wl, 0)
    w = {n: torch.from_numpy(w[n]).to(torch.bfloat16).to(dev) for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    attn = rt.AttnDesc(batch=B, seq_len=N, n_heads=H, head_dim=dh, dtype=rt.RT_BF16, softmax_scale=1.0 / math.sqrt(dh))
    desc = rt.LayerDesc(attn=attn, d_model=D, d_ff=F, rms_eps=1e-6, residual_scale=1.0, flags=0)
    z, kc, vc = (torch.empty((N, B, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
    ws_f = torch.empty(rt.rt_layer_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    rt.rt_layer_forward(desc, w, x, z, kc, vc, ws_f, stream=stream)
    torch.cuda.synchronize()
    del ws_f, kc, vc
    f32 = dict(dtype=torch.float32, device=dev)
    z_bar = torch.randn((N, B, D), generator=torch.Generator(device=dev).manual_seed(9), **f32)
    x_bar = torch.empty((N, B, D), **f32)
    grads = {n: torch.empty(w[n].shape, **f32) for n in w}
    grads["g_attn"] = torch.empty(D, **f32)
    grads["g_mlp"] = torch.empty(D, **f32)
    nbytes = rt.rt_layer_backward_workspace_bytes(desc)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    log(f"layer backward: workspace {nbytes / 2**30:.1f} GiB")
    call = lambda: rt.rt_layer_backward(desc, w, x, z, z_bar, x_bar, grads, ws, stream=stream)
    t0 = time.time()
    call()
    torch.cuda.synchronize()
    log(f"layer backward warm-up {time.time() - t0:.2f}s")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 2
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    assert bool(torch.isfinite(x_bar).all()) and all(bool(torch.isfinite(g).all()) for g in grads.values())
    NB, P = N * B, B * H
    pairs = N * (N - 1) / 2
    flops = {
        "recompute_products": 2.0 * NB * D * (3 * D + 2 * D + D + F),
        "recompute_attention": 4.0 * dh * P * (pairs + N),
        "position_adjoint_products": 2.0 * NB * (2 * D * D + D * F + F * D + D * D),
        "attention_backward": 10.0 * dh * P * pairs + 12.0 * dh * P * N,
        "input_adjoint_product": 2.0 * NB * 3 * D * D,
        "weight_gradients": 2.0 * NB * (6 * D * D + 2 * D * F),
    }
    total = sum(flops.values())
    print(json.dumps({"layer_backward": "RT layer backward, B=512, N=2048, d=1024, 16x64 heads, F=4096, bf16",
                      "ms": round(ms, 3), "tokens_per_s": round(B * N / (ms * 1e-3), 1),
                      "alg_TFLOP": {k: round(v / 1e12, 3) for k, v in flops.items()},
                      "TFLOP_s": round(total / (ms * 1e-3) / 1e12, 2), "bound": "mfma", "peak_TFLOP_s": 2500.0,
                      "frac": round(total / (ms * 1e-3) / 1e12 / 2500.0, 4),
                      "workspace_GiB": round(nbytes / 2**30, 2)}))


def decode(args):
    """One decode step (a new position per sequence against the persistent KV
    cache) of the B=512, d=1024 layer after a 2048-position prefill: mean of
    20 steps (the same position re-decoded), and the cache-read roofline."""
    import torch

    import blocked_prefill_amd as rt
    import rt_inputs
    rt.load()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    B, D, H, dh, F, n_past = 512, 1024, 16, 64, 4096, 2048
    wl = rt_inputs.Workload("decode_b512_n2048", B, n_past, D, H, dh, F, 1, "bf16", 1003)
    w = rt_inputs.layer_weights(wl, 0)
    w = {k: torch.from_numpy(w[k]).to(torch.bfloat16).to(dev) for k in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    attn = rt.AttnDesc(batch=B, seq_len=n_past + 1, n_heads=H, head_dim=dh, dtype=rt.RT_BF16, softmax_scale=0.125)
    desc = rt.LayerDesc(attn=attn, d_model=D, d_ff=F, rms_eps=1e-6, residual_scale=1.0, flags=0)
    pre = rt.LayerDesc(attn=rt.AttnDesc(batch=B, seq_len=n_past, n_heads=H, head_dim=dh, dtype=rt.RT_BF16,
                                        softmax_scale=0.125), d_model=D, d_ff=F, rms_eps=1e-6, residual_scale=1.0,
                       flags=0)
    x = torch.from_numpy(rt_inputs.layer_input(wl)).to(torch.bfloat16).to(dev)
    kc, vc = (torch.empty((n_past + 1, B, D), dtype=torch.bfloat16, device=dev) for _ in range(2))
    z = torch.empty((n_past, B, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rt.rt_layer_workspace_bytes(pre), dtype=torch.uint8, device=dev)
    rt.rt_layer_forward(pre, w, x, z, kc[:n_past], vc[:n_past], ws, stream=stream)
    torch.cuda.synchronize()
    del ws
    x_new = x[-1].clone()
    z_new = torch.empty((B, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rt.rt_layer_decode_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    for _ in range(3):
        rt.rt_layer_decode_step(desc, w, n_past, x_new, z_new, kc, vc, ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        rt.rt_layer_decode_step(desc, w, n_past, x_new, z_new, kc, vc, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    cache_bytes = 2 * n_past * B * D * 2
    weight_bytes = (4 * D * D + 2 * D * F) * 2
    floor_ms = (cache_bytes + weight_bytes) / (HBM_PEAK_GBS * 1e9) * 1e3
    print(json.dumps({"decode": "one RT layer, bf16, B=512, d=1024, 16x64 heads, MLP 4096, after 2048 positions",
                      "ms_per_step": round(ms, 4), "tokens_per_s": round(B / (ms * 1e-3), 1),
                      "hbm_floor_ms": round(floor_ms, 4), "frac_of_floor": round(floor_ms / ms, 4)}))


def vendor_gemm():
    """torch's bf16 products (the vendor GEMM library) on the shapes of the 6-layer stack's
    products: six per-position products of 512 rows in one batched call (the grouped launch),
    one of them alone, and a 65536-row chunk of the up-front q|k'|v' projection. Plain products,
    no fused normalisation, activation or residual; operands contiguous, weights pre-transposed.
    Timed as graph replays of back-to-back launches (the kernels' time, not the host's launch rate)."""
    import torch
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    rnd = lambda *s: torch.randn(*s, device=dev, generator=g).to(torch.bfloat16).contiguous()

    def timed(f, n):
        # n launches captured in one graph, so that the host's launch rate does not set the time
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for _ in range(3):
                f()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(n):
                f()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (n * reps)

    rows = []
    for name, (m, n, k) in (("W_o", (512, 1024, 1024)), ("W_1", (512, 4096, 1024)), ("W_2", (512, 1024, 4096)),
                            ("W_kv", (512, 2048, 1024))):
        a, b = rnd(6, m, k), rnd(6, k, n)
        us = timed(lambda: torch.bmm(a, b), 50)
        rows.append({"product": f"{name} x6", "shape": f"6 x [{m}x{k}] x [{k}x{n}]", "us": round(us, 2),
                     "TFLOP_s": round(2.0 * 6 * m * n * k / us * 1e-6, 1)})
        a1, b1 = rnd(m, k), rnd(k, n)
        us = timed(lambda: torch.mm(a1, b1), 50)
        rows.append({"product": f"{name} x1", "shape": f"[{m}x{k}] x [{k}x{n}]", "us": round(us, 2),
                     "TFLOP_s": round(2.0 * m * n * k / us * 1e-6, 1)})
    a, b = rnd(65536, 1024), rnd(1024, 3072)
    us = timed(lambda: torch.mm(a, b), 20)
    rows.append({"product": "q|k'|v' chunk", "shape": "[65536x1024] x [1024x3072]", "us": round(us, 2),
                 "TFLOP_s": round(2.0 * 65536 * 1024 * 3072 / us * 1e-6, 1)})
    for r in rows:
        print(json.dumps(r))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stack6_d1024_b512_n2048")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="batch rows of the CPU-oracle sample (0: one per oracle thread)")
    ap.add_argument("--cpu-positions", type=int, default=0,
                    help="CPU sample: the first P positions only (default: all, or 2048 when N > 8192; "
                         "outputs at positions <= P depend on those positions only)")
    ap.add_argument("--counters", action="store_true",
                    help="short run for hardware-counter passes: one layer forward, then its update "
                         "sequence, then a plain 1 GiB device copy (the calibration kernel)")
    ap.add_argument("--sweep", action="store_true",
                    help="single-layer latency at B=512, d=1024 for N = 256..2048: RT blocked, RT naive, "
                         "Transformer (log-log slopes)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 counter passes over --counters (no GPU needed)")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="summarise the update launches' counter passes (UPDATE_COUNTER_PASSES) over --counters, "
                         "one rocprofv3 output directory per pass, in order (no GPU needed)")
    ap.add_argument("--backward", action="store_true",
                    help="attention backward of the blocked schedule at B=512, 16x64 heads, N=2048")
    ap.add_argument("--layer-backward", action="store_true",
                    help="the RT layer's backward at B=512, N=2048, d=1024 (one layer)")
    ap.add_argument("--eager", action="store_true",
                    help="enqueue the stack directly (rt_stack_forward, no graph): the same launches, for "
                         "counter passes (rocprofv3's counter mode does not follow graph launches here)")
    ap.add_argument("--per-layer", action="store_true",
                    help="run the stack as one graph per layer, one after another (no layer wavefront)")
    ap.add_argument("--decode", action="store_true",
                    help="one decode step of the B=512, d=1024 layer against a 2048-position cache")
    ap.add_argument("--family-summary", nargs="+", metavar="DIR",
                    help="MFMA / vector-ALU shares per kernel family from a rocprofv3 pass of FAMILY_COUNTERS "
                         "over --eager (no GPU needed)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("DIR", "REPLAYS"),
                    help="tables from a rocprofv3 --kernel-trace --stats run of the stack bench (no GPU needed)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="the vendor library (torch bf16 bmm / mm) on the stack's product shapes, for comparison "
                         "with this library's kernels in the stack's kernel trace")
    args = ap.parse_args()

    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    if args.counter_summary:
        return counter_summary(args.counter_summary)
    if args.family_summary:
        return family_summary(args.family_summary)
    if args.trace_summary:
        return trace_summary(args.trace_summary[0], int(args.trace_summary[1]))
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (batch rows are independent; "
              "a multi-GPU run would shard the batch with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import blocked_prefill_amd as rt
    import rt_inputs

    if not os.path.exists(rt.library_path):
        from blocked_prefill_amd import build
        build.build()
    rt.load()

    if args.vendor_gemm:
        return vendor_gemm()
    if args.sweep:
        return sweep(args)
    if args.decode:
        return decode(args)
    if args.backward:
        return backward(args)
    if args.layer_backward:
        return layer_backward_bench(args)
    wl = rt_inputs.WORKLOADS[args.workload]
    if wl.update_only:
        return update_only_bench(args, rt, wl)
    N, B, D, H, dh, F, L = wl.n_pos, wl.batch, wl.d_model, wl.n_heads, wl.head_dim, wl.d_ff, wl.n_layers
    scale = 1.0 / math.sqrt(dh)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    t0 = time.time()
    x = torch.from_numpy(rt_inputs.layer_input(wl)).to(torch.bfloat16).to(dev)
    weights = []
    for layer in range(L):
        w = rt_inputs.layer_weights(wl, layer)
        weights.append({n: torch.from_numpy(w[n]).to(torch.bfloat16).to(dev)
                        for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")})
    log(f"inputs generated and resident in HBM in {time.time() - t0:.1f}s")

    attn = rt.AttnDesc(batch=B, seq_len=N, n_heads=H, head_dim=dh, dtype=rt.RT_BF16, softmax_scale=scale)
    desc = rt.LayerDesc(attn=attn, d_model=D, d_ff=F, rms_eps=1e-6, residual_scale=1.0, flags=0)
    layer_ws = rt.rt_layer_workspace_bytes(desc)
    ws_bytes = layer_ws if args.per_layer else rt.rt_stack_workspace_bytes(desc, L)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    zs = [torch.empty((N, B, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ks = [torch.empty((N, B, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    vs = [torch.empty((N, B, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]

    if args.counters:
        # q, k', v' (the workspace's first three slabs) and the KV cache filled with
        # random values (memory traffic does not depend on them; a whole layer forward
        # would be ~12k dispatches, each serialised by the counter collection), then
        # the layer's 2047 update launches, then the calibration copy
        slab = N * B * D
        qkv = torch.empty(0, dtype=torch.bfloat16, device=dev).set_(
            ws.untyped_storage(), 0, (3, slab), (((slab * 2 + 255) // 256 * 256) // 2, 1))
        qkv.normal_()
        ks[0].normal_()
        vs[0].normal_()
        torch.cuda.synchronize()
        for t0 in range(1, N, 256):
            update_sequence(rt, attn, ws, ks[0], vs[0], N, B, H, D, stream, None, t_range=(t0, min(t0 + 256, N)))
            log(f"counters: update launches t={t0}..{min(t0 + 255, N - 1)} done")
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("counters run done: 2047 update launches, 1 GiB copy")
        return

    t0 = time.time()
    plans = []
    if args.eager:  # no graph: the same launches enqueued on every step
        pass
    elif args.per_layer:  # one graph per layer, replayed one after another
        for layer in range(L):
            xin = x if layer == 0 else zs[layer - 1]
            plans.append(rt.rt_layer_plan_create(desc, weights[layer], xin, zs[layer], ks[layer], vs[layer], ws))
    else:  # the stack's wavefront as one graph
        plans.append(rt.rt_stack_plan_create(desc, weights, x, zs, ks, vs, ws))
    capture_s = time.time() - t0
    log(f"captured {len(plans)} graph(s) in {capture_s:.2f}s")

    def step():
        if args.eager:
            rt.rt_stack_forward(desc, weights, x, zs, ks, vs, ws, stream=stream)
        for p in plans:
            p.launch(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")

    torch.cuda.synchronize()
    # one event between consecutive steps: the first and last bracket the timed region,
    # the ones between give each step's time (their spread is reported)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    wall0 = time.time()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.time() - wall0
    elapsed_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = elapsed_ms / args.steps
    step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    tokens_per_s = B * N * args.steps / (elapsed_ms / 1e3)
    log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step (wall {wall / args.steps * 1e3:.2f} ms), "
        f"{tokens_per_s / 1e6:.3f} M tokens/s")
    assert bool(torch.isfinite(zs[-1]).all()), "non-finite output"

    roofline = None
    update_info = {}
    if not args.no_kernel_timing:
        # the last layer's q, k', v' and state are in the workspace, its caches in ks/vs:
        # replay its update sequence (t = 1..N-1), one event pair per launch
        ws_last = ws if args.per_layer else ws[(L - 1) * layer_ws:]  # the last layer's workspace
        durs = update_sequence(rt, attn, ws_last, ks[-1], vs[-1], N, B, H, D, stream, torch)
        # the roofline's average launch duration: the same 2047 launches captured as one HIP
        # graph and replayed back to back, two events on the launch stream around the replays
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                update_sequence(rt, attn, ws_last, ks[-1], vs[-1], N, B, H, D, cap, None, sync=False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        r0.record(stream)
        for _ in range(reps):
            g.replay()
        r1.record(stream)
        torch.cuda.synchronize()
        graph_avg_s = r0.elapsed_time(r1) / 1e3 / (reps * (N - 1))
        del g
        P = B * H
        byts = np.array([update_bytes(t, N, P, dh, 2) for t in range(1, N)], dtype=np.float64)
        flops = np.array([update_flops(t, N, P, dh) for t in range(1, N)], dtype=np.float64)
        avg_s = graph_avg_s
        achieved = byts.mean() / avg_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name),
                    "kernel": "fused blocked update + finalize (update_small / update_simt / update_mfma kernels)",
                    "launches": N - 1, "avg_launch_us": round(avg_s * 1e6, 2),
                    "alg_bytes_per_launch": int(byts.mean())}
        levels = {}
        for t in range(1, N):
            b = t & -t
            lv = levels.setdefault(b, [0.0, 0.0, 0.0, 0])
            lv[0] += durs[t - 1]
            lv[1] += byts[t - 1]
            lv[2] += flops[t - 1]
            lv[3] += 1
        update_info = {
            "update_ms_per_layer": round(avg_s * (N - 1) * 1e3, 3),
            "per_level_timing": "HIP events around each launch (adds the event records' overhead)",
            "update_alg_GB_per_layer": round(float(byts.sum()) / 1e9, 3),
            "per_level": {str(b): {"steps": v[3], "us_per_step": round(v[0] / v[3] * 1e3, 2),
                                   "GB_s": round(v[1] / (v[0] / 1e3) / 1e9, 1),
                                   "TFLOP_s": round(v[2] / (v[0] / 1e3) / 1e12, 2),
                                   # max(bytes / HBM peak, flops / MFMA peak) over the measured time
                                   "frac": round(max(v[1] / (v[0] / 1e3) / 1e9 / HBM_PEAK_GBS,
                                                     v[2] / (v[0] / 1e3) / 1e12 / 2500.0), 4)}
                          for b, v in sorted(levels.items())},
        }
        log(f"update kernel: {achieved:.0f} GB/s algorithmic ({achieved / HBM_PEAK_GBS:.1%} of HBM peak), "
            f"{avg_s * (N - 1) * 1e3:.2f} ms per layer")

    cpu = None
    if not args.no_cpu:
        import oracle
        rows = list(range(min(args.cpu_rows or oracle.num_threads(), B)))
        # long sequences: a prefix keeps the naive oracle (quadratic in N) within seconds
        npos = args.cpu_positions if 0 < args.cpu_positions < N else (2048 if N > 8192 else N)
        xr = rt_inputs.layer_input(wl, rows=rows)[:npos]
        w0 = rt_inputs.layer_weights(wl, 0)
        t0 = time.time()
        oracle.layer_forward(xr, w0, n_heads=H, softmax_scale=scale, round_bf16=True)
        cpu_s = time.time() - t0
        # the sample is one of the stack's L layers: the stack rate is L times slower
        cpu_value = len(rows) * npos / (cpu_s * L)
        span = f"all {N} positions" if npos == N else f"the first {npos} of {N} positions (later ones cost more)"
        cpu = {"value": round(cpu_value, 2), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "build": ORACLE_BUILD, "cpu_model": cpu_model(), "nproc": os.cpu_count(),
               "sample": f"{len(rows)} batch rows x {span} x layer 1 of {L} "
                         f"({cpu_s:.1f} s); stack rate = rows*positions/({L}*time)"}
        log(f"cpu oracle: {cpu_s:.1f}s for the sample -> {cpu_value:.1f} stack tokens/s")

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "ms_per_step_std": round(float(step_ms.std()), 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,1/d_in) weights)",
        "config": {"workload": f"{wl.name}: RT {L}-layer stack prefill x->z, bf16, B={B}, N={N}, d_model={D}, "
                               f"{H} heads x {dh}, MLP {F} GELU",
                   "batch": B, "seq_len": N, "layers": L, "ms_per_layer": round(ms_per_step / L, 3),
                   "tokens_per_s_per_layer": round(tokens_per_s * L, 1), "graph_capture_s": round(capture_s, 2),
                   "schedule": ("layer wavefront, eager launches (rt_stack_forward)" if args.eager else
                                "layer by layer, one graph each" if args.per_layer else
                                "layer wavefront, one graph (rt_stack_plan_create)"),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    # the metric's "MFMA util" at the layer level: the layer's algorithmic products (the up-front
    # projection 6*N*B*d^2, per position 2B(3d^2 + 2dF)) and the update's 4*dh per (query, key) pair
    # visited by the blocked schedule, over the measured layer time
    pairs_visited = sum((t & -t) * min(t & -t, N - t) for t in range(1, N))
    layer_flops = 6.0 * N * B * D * D + N * 2.0 * B * (3 * D * D + 2 * D * F) + 4.0 * dh * B * H * pairs_visited
    layer_tflops = layer_flops / (ms_per_step / L * 1e-3) / 1e12
    out["mfma_util"] = {"scope": "whole layer: all products and the update's scores/values, per layer time",
                        "alg_TFLOP_per_layer": round(layer_flops / 1e12, 3), "achieved_TFLOP_s": round(layer_tflops, 1),
                        "peak_TFLOP_s": 2500.0, "frac": round(layer_tflops / 2500.0, 4)}
    if update_info:
        out["update"] = update_info
        ceil = ceilings(dev)
        ceil["update_frac_of_copy"] = round(roofline["achieved"] / ceil["copy_GB_s"], 4)
        if ceil["stream_3r1w_GB_s"]:
            ceil["update_frac_of_stream_3r1w"] = round(roofline["achieved"] / ceil["stream_3r1w_GB_s"], 4)
            for v in out["update"]["per_level"].values():
                v["frac_of_stream_3r1w"] = round(v["GB_s"] / ceil["stream_3r1w_GB_s"], 4)
        ceil["layer_mfma_frac_of_gemm"] = round(layer_tflops / ceil["gemm_TFLOP_s"], 4)
        out["ceilings"] = ceil
    print(json.dumps(out), flush=True)
    for p in plans:
        p.destroy()


if __name__ == "__main__":
    main()
