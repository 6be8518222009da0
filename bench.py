"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path: fa_fwd on the long-context forward
batch (B=1, H=32, N=32768, d=128, causal) and fa_bwd on the backward batch
(B=4, H=16, N=4096, d=128, causal; its O and LSE come from fa_fwd on the
same batch, computed before timing).  Inputs are seeded synthetic bf16
tensors already resident in HBM.  Useful flops: forward 4 B H N^2 d, halved
when causal; backward 2.5x the forward of its batch (five matrix products
per tile pair, the recomputation of the scores included).

The same line carries a "next" object: one timed configuration for each of
the extensions past the five workloads (cross attention, grouped K/V heads,
a sliding window, split-KV decoding), each against its own roofline
(``--no-next`` skips them).

Prints ONE JSON line.  ``--gpus N`` with N > 1 exits: this path runs on one
GPU only (attention heads are independent, see the design notes for how
it would shard).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0

FWD = dict(name="fwd_b1_h32_n32768_d128_causal", B=1, H=32, N=32768, d=128, causal=True)
BWD = dict(name="bwd_b4_h16_n4096_d128_causal", B=4, H=16, N=4096, d=128, causal=True)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fwd_kernel_b1_h32_n32768_d128_causal_hbm_counters.json")
BWD_COUNTERS_FILE = os.path.join(ROOT, "profiles", "bwd_kernels_b4_h16_n4096_d128_causal_hbm_counters.json")
PIPE_FILE = os.path.join(ROOT, "profiles", "fwd_bwd_kernels_mfma_lds_counters.md")
# the forward kernel the long-context batch runs: 12 waves of 32 query rows
FWD_KERNEL = "fwd_kernel<128, 12, 64, true, false>"
FWD_KERNEL_DESC = "fwd_kernel<128,12,64,true,false> (12 waves, 384 query rows per workgroup, 64-key tiles)"
FWD_ROWS_PER_WG, FWD_THREADS_PER_WG = 384, 768
# the backward kernels the backward batch runs
BWD_DQ_KERNEL = "bwd_dq_kernel<128, 8, 64, true, false>"
BWD_MAIN_KERNEL = "bwd_main_kernel<128, true, false>"
CSRC = os.path.join(ROOT, "io_aware_tiled_fa_amd", "csrc")
# the forward kernel's sources (the HBM counter record is tied to these) and
# every kernel source (the kernel-trace and pipe summaries cover all kernels)
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("fa_fwd.hip", "fa_device.h", "fa_kernels.h", "fa_layout.h")]
BWD_KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("fa_bwd.hip", "fa_device.h", "fa_kernels.h", "fa_layout.h")]
ALL_KERNEL_SOURCES = [os.path.join(CSRC, f) for f in
                      ("fa_api.hip", "fa_bwd.hip", "fa_decode.hip", "fa_device.h", "fa_fwd.hip", "fa_kernels.h",
                       "fa_layout.h")]


def fwd_flops(c) -> float:
    f = 4.0 * c["B"] * c["H"] * c["N"] ** 2 * c["d"]
    return f / 2 if c["causal"] else f


def bwd_flops(c) -> float:
    return 2.5 * fwd_flops(c)


def fwd_algorithmic_bytes(c) -> float:
    """HBM bytes the forward must move: read Q, K, V, write O (bf16), write LSE (fp32)."""
    t = c["B"] * c["N"] * c["H"] * c["d"] * 2
    return 4 * t + c["B"] * c["H"] * c["N"] * 4


def visible_pairs(Nq: int, Nk: int, causal: bool, window: int = 0) -> int:
    """Query-key pairs inside the mask (keys aligned to the end of the
    queries; a window W keeps |i + N_k - N_q - j| < W)."""
    import numpy as np

    pos = np.arange(Nq, dtype=np.int64) + (Nk - Nq)
    hi = np.full(Nq, Nk - 1, dtype=np.int64)
    lo = np.zeros(Nq, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, pos)
    if window > 0:
        hi = np.minimum(hi, pos + window - 1)
        lo = np.maximum(lo, pos - window + 1)
    return int(np.maximum(hi - lo + 1, 0).sum())


def kernel_source_hash(paths=None) -> str:
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES if paths is None else paths):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel changed since."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


HBM_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/hbm_fetch -o p -- "
    "python3 bench.py --steps 2 --warmup 0 --no-cpu-baseline --no-next --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/hbm_write -o p -- "
    "python3 bench.py --steps 2 --warmup 0 --no-cpu-baseline --no-next --copy-calibration",
    "python3 bench.py --hbm-summary rocprof_out/hbm_fetch rocprof_out/hbm_write",
]


def bwd_algorithmic_bytes(c) -> dict:
    """HBM bytes each backward kernel must move at least, bf16 tensors of
    B N H d elements: the dQ kernel reads Q, dO, O, K, V and LSE and writes
    dQ and the two float32 row terms per query row; the dK / dV kernel reads
    Q, dO, K, V and the row terms and writes dK and dV."""
    t = c["B"] * c["N"] * c["H"] * c["d"] * 2
    rows = c["B"] * c["H"] * c["N"] * 4
    return {"dq": 6 * t + rows + 2 * rows, "main": 6 * t + 2 * rows}


def _counter_rows(d, counter):
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
    return rows


def _per_launch(rows, kernel, threads):
    vals = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"] and int(r["Grid_Size"]) == threads]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def hbm_summary(fetch_dir: str, write_dir: str) -> dict:
    """Turn the two rocprofv3 counter runs of HBM_COMMANDS into HBM bytes per
    launch of the forward kernel on the long-context batch and of the two
    backward kernels on the backward batch.  Each counter is scaled by what
    it reads for a plain 1 GiB device copy in the same run (the copy moves
    exactly 1 GiB each way)."""
    fr, wr = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")

    def copy_kib(rows):  # the 1 GiB copies (KiB units)
        vals = [float(r["Counter_Value"]) for r in rows
                if "fa::" not in r["Kernel_Name"] and float(r["Counter_Value"]) > 2 ** 18]
        if not vals:
            raise SystemExit("no counter rows for the 1 GiB calibration copy")
        return sum(vals) / len(vals), len(vals)

    f_copy, ncf = copy_kib(fr)
    w_copy, ncw = copy_kib(wr)
    gib_kib = 2.0 ** 20
    f_scale, w_scale = gib_kib / f_copy, gib_kib / w_copy
    bwd_alg = bwd_algorithmic_bytes(BWD)
    c2 = dict(B=4, H=16, N=2048, d=64, causal=False)
    c3 = dict(B=2, H=32, N=8192, d=128, causal=True)
    kernels = [
        ("fwd", FWD_KERNEL, FWD["B"] * FWD["H"] * (-(-FWD["N"] // FWD_ROWS_PER_WG)) * FWD_THREADS_PER_WG,
         FWD_KERNEL_DESC, FWD["name"], fwd_algorithmic_bytes(FWD)),
        ("fwd_d64", "fwd_kernel<64, 8, 64, true, false>", 4 * 16 * (2048 // 256) * 512,
         "fwd_kernel<64,8,64,true,false> (8 waves, 256 query rows per workgroup, unbounded band)",
         "fwd_b4_h16_n2048_d64",
         fwd_algorithmic_bytes(c2)),
        ("fwd_n8192", FWD_KERNEL, 2 * 32 * (-(-8192 // FWD_ROWS_PER_WG)) * FWD_THREADS_PER_WG, FWD_KERNEL_DESC,
         "fwd_b2_h32_n8192_d128_causal_peaked", fwd_algorithmic_bytes(c3)),
        ("bwd_dq", BWD_DQ_KERNEL, BWD["B"] * BWD["H"] * (BWD["N"] // 256) * 512,
         "bwd_dq_kernel<128,8,64,true,false> (dQ and the row terms; 8 waves, 256 query rows per workgroup)",
         BWD["name"], bwd_alg["dq"]),
        ("bwd_main", BWD_MAIN_KERNEL, BWD["B"] * BWD["H"] * (BWD["N"] // 128) * 512,
         "bwd_main_kernel<128,true,false> (dK and dV; 8 waves, 128 keys per workgroup)", BWD["name"],
         bwd_alg["main"]),
    ]
    recs = {}
    for key, kname, threads, desc, workload, alg in kernels:
        f_kib, nf = _per_launch(fr, kname, threads)
        w_kib, nw = _per_launch(wr, kname, threads)
        if f_kib is None or w_kib is None:
            raise SystemExit(f"no FETCH_SIZE / WRITE_SIZE rows for {kname} at {threads} threads")
        rd, wrb = f_kib * f_scale * 1024, w_kib * w_scale * 1024
        recs[key] = {
            "kernel": desc,
            "workload": workload,
            "fetch_kib_per_launch_raw": round(f_kib, 1),
            "write_kib_per_launch_raw": round(w_kib, 1),
            "hbm_read_bytes_per_launch": round(rd),
            "hbm_write_bytes_per_launch": round(wrb),
            "hbm_bytes_per_launch": round(rd + wrb),
            "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": round((rd + wrb) / alg, 3),
            "launches": {"fetch": nf, "write": nw},
        }
    calib = {"copy_1gib_fetch_kib_raw": round(f_copy, 1), "copy_1gib_write_kib_raw": round(w_copy, 1),
             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
             "copy_launches": {"fetch": ncf, "write": ncw}}
    fwd = dict(recs["fwd"], kernel_source_hash=kernel_source_hash(), **calib, commands=HBM_COMMANDS,
               other_forward_workloads={"fwd_b4_h16_n2048_d64": recs["fwd_d64"],
                                        "fwd_b2_h32_n8192_d128_causal_peaked": recs["fwd_n8192"]})
    bwd = {"kernel_source_hash": kernel_source_hash(BWD_KERNEL_SOURCES), "dq": recs["bwd_dq"],
           "main": recs["bwd_main"], **calib, "commands": HBM_COMMANDS}
    return {"fwd": fwd, "bwd": bwd}


# Pipe-utilisation counters of the kernels of one step: three rocprofv3
# passes (a pass holds at most 8 SQ and 4 TCC counters), then a summary into
# PIPE_FILE.
PIPE_PASSES = [
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS "
    "GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_BF16 TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
]
PIPE_COMMANDS = [
    f"rocprofv3 --pmc {c} --output-format csv -d rocprof_out/pipe{i} -o p -- "
    "python3 bench.py --steps 2 --warmup 0 --no-cpu-baseline --no-next" for i, c in enumerate(PIPE_PASSES)
] + ["python3 bench.py --pipe-summary " + " ".join(f"rocprof_out/pipe{i}" for i in range(len(PIPE_PASSES)))]


def pipe_summary(dirs) -> str:
    """Per kernel of the step (last dispatch of each): matrix-core busy and
    co-execution as a share of the cycles of all SIMDs, VALU and LDS issue
    as a share of wave cycles, LDS busy and bank-conflict cycles per CU; then
    the bf16 matrix flops the counters saw (512 per MOPS unit) beside the
    useful flops of the call, and the L2 hit rate."""
    import collections
    import csv
    import glob

    per = collections.defaultdict(dict)
    for d in dirs:
        last = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                k = r["Kernel_Name"].split("(")[0]
                if "fa::" not in k:
                    continue
                key = (k, int(r["Grid_Size"]))
                did = int(r["Dispatch_Id"])
                if last.get(key, -1) < did:
                    last[key] = did
                    per[key] = {kk: v for kk, v in per[key].items() if not kk.startswith(d + ":")}
                if did == last[key]:
                    per[key][d + ":" + r["Counter_Name"]] = per[key].get(d + ":" + r["Counter_Name"], 0.0) + \
                        float(r["Counter_Value"])
                    per[key][d + ":ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    lines = ["| kernel | grid threads | cycles (per XCD) | clock GHz | MFMA busy | MFMA+VALU co-exec | VALU issue / wave | "
             "LDS issue / wave | wait / wave | LDS busy / CU | LDS bank-conflict cycles / LDS busy |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for (k, grid), v in sorted(per.items()):
        c = {kk.split(":", 1)[1]: x for kk, x in v.items()}
        if "SQ_WAVE_CYCLES" not in c or "SQ_VALU_MFMA_BUSY_CYCLES" not in c:
            continue
        g = c["GRBM_GUI_ACTIVE"] / 8  # per XCD
        simd = g * 1024               # 256 CUs x 4 SIMDs over 8 XCDs
        wc = c["SQ_WAVE_CYCLES"]
        ns = c.get("ns", 0.0)
        clk = f"{g / ns:.2f}" if ns > 0 else "-"  # busy cycles of one XCD over the dispatch's duration
        lines.append(
            f"| `{k}` | {grid} | {g:.3g} | {clk} | {c['SQ_VALU_MFMA_BUSY_CYCLES'] / simd:.1%} | "
            f"{c['SQ_VALU_MFMA_COEXEC_CYCLES'] / simd:.1%} | {c['SQ_ACTIVE_INST_VALU'] / wc:.1%} | "
            f"{c['SQ_ACTIVE_INST_LDS'] / wc:.1%} | {c['SQ_WAIT_INST_ANY'] / wc:.1%} | "
            f"{c['SQ_LDS_IDX_ACTIVE'] / (g * 256):.1%} | "
            f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1):.1%} |")
    lines += ["", "| kernel | grid threads | MFMA instructions | bf16 matrix TFLOP executed | L2 hit rate |",
              "|---|---|---|---|---|"]
    for (k, grid), v in sorted(per.items()):
        c = {kk.split(":", 1)[1]: x for kk, x in v.items()}
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" not in c:
            continue
        hits, miss = c.get("TCC_HIT_sum", 0.0), c.get("TCC_MISS_sum", 0.0)
        lines.append(f"| `{k}` | {grid} | {c['SQ_INSTS_VALU_MFMA_BF16']:.4g} | "
                     f"{c['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e12:.4f} | {hits / max(hits + miss, 1):.1%} |")
    lines += ["", f"Useful flops per call: forward {fwd_flops(FWD) / 1e12:.4f} TFLOP (4 B H N^2 d, halved for "
              f"causal); backward {bwd_flops(BWD) / 1e12:.4f} TFLOP (2.5 x its forward). The backward kernels "
              "execute seven products per tile pair against the five of the useful count (S and dP are "
              "computed once for dK / dV and again for dQ), and whole tiles on the diagonal."]
    return "\n".join(lines)


STATS_FILE = os.path.join(ROOT, "profiles", "fwd_bwd_bench_kernel_stats.md")
STATS_COMMANDS = [
    "rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/prof_stats -o run -- "
    "python3 -u bench.py --steps 5 --warmup 1 --no-cpu-baseline",
    "python3 bench.py --stats-summary rocprof_out/prof_stats",
]


def stats_summary(d: str) -> str:
    """rocprofv3 --kernel-trace --stats of STATS_COMMANDS as a markdown table:
    the --stats rows, then each launch shape from the trace."""
    import collections
    import csv
    import glob

    stats = list(csv.DictReader(open(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0])))
    trace = list(csv.DictReader(open(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0])))
    per = collections.defaultdict(list)
    for r in trace:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]), r["Workgroup_Size_X"],
               r.get("Arch_VGPR_Count", r.get("VGPR_Count", "")), r["LDS_Block_Size"])
        per[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    def short(name):  # library kernels (torch's random fill) carry very long template names
        return name if len(name) <= 100 else name[:90] + " ..."

    out = ["## --stats (all dispatches of the run)", "", "| kernel | calls | avg ms | total ms | % |",
           "|---|---|---|---|---|"]
    for r in stats:
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
    out += ["", "## per launch shape (from the kernel trace)", "",
            "| kernel | workgroups | threads / WG | VGPRs | LDS bytes | dispatches | avg ms | avg ms after the first "
            "| median ms | min ms | max ms |",
            "|---|---|---|---|---|---|---|---|---|---|---|"]
    for (k, wgs, wgsz, vg, lds), v in per.items():
        rest = v[1:] or v
        out.append(f"| `{short(k)}` | {wgs} | {wgsz} | {vg} | {lds} | {len(v)} | {sum(v) / len(v):.4f} | "
                   f"{sum(rest) / len(rest):.4f} | {sorted(v)[len(v) // 2]:.4f} | {min(v):.4f} | {max(v):.4f} |")
    out += ["", "The first dispatch of a kernel in the process runs cold (code and caches); bench.py's "
            "roofline times the launches after its warmup, so it compares with the average after the first."]
    return "\n".join(out)


def device_tensor(bits, device):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def cpu_baseline(fwd_inp, bwd_inp, budget_s: float = 20.0):
    """Time the fp64 oracle on a bounded sample of the same step: the forward
    of whole heads of the long-context batch, then the backward of heads of
    the backward batch, until about ``budget_s`` seconds have been spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    scale = 1.0 / math.sqrt(FWD["d"])
    useful = 0.0
    t0 = time.perf_counter()
    f_heads = 0
    # forward: one whole head at a time (every query row of that head)
    while time.perf_counter() - t0 < 0.6 * budget_s and f_heads < FWD["H"]:
        h = f_heads
        q = fwd_inp.q[:, :, h:h + 1]
        k = fwd_inp.k[:, :, h:h + 1]
        v = fwd_inp.v[:, :, h:h + 1]
        oracle.attention_forward(q, k, v, scale, True)
        useful += fwd_flops(dict(FWD, H=1))
        f_heads += 1
    t_f = time.perf_counter() - t0
    b_heads = 0
    t1 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and b_heads < BWD["B"] * BWD["H"]:
        b, h = divmod(b_heads, BWD["H"])
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        oracle.attention_backward(bwd_inp.q[sl], bwd_inp.k[sl], bwd_inp.v[sl], bwd_inp.do[sl],
                                  scale, True)
        useful += bwd_flops(dict(BWD, B=1, H=1))
        b_heads += 1
    t_b = time.perf_counter() - t1
    total = t_f + t_b
    return {
        "value": useful / total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle: forward of {f_heads} whole head(s) of the "
                   f"B=1 H=32 N=32768 d=128 causal batch ({t_f:.1f} s) + backward of {b_heads} "
                   f"head(s) of the B=4 H=16 N=4096 d=128 causal batch ({t_b:.1f} s); "
                   f"useful-flop convention as the GPU value"),
        "seconds": round(total, 2),
        "cpu": cpu_model(),
    }


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (else the platform's)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the extension configurations")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the d = 64 and peaked N = 8192 forward workloads")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--stats-summary", metavar="DIR",
                    help="summarise the STATS_COMMANDS kernel trace into " + os.path.relpath(STATS_FILE, ROOT))
    ap.add_argument("--pipe-summary", nargs="+", metavar="PASS_DIR",
                    help="summarise the PIPE_COMMANDS counter passes into " + os.path.relpath(PIPE_FILE, ROOT))
    ap.add_argument("--hbm-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the forward kernel's HBM counter summary from two rocprofv3 runs")
    args = ap.parse_args(argv)

    if args.stats_summary:
        table = stats_summary(args.stats_summary)
        with open(STATS_FILE, "w") as f:
            f.write("# rocprofv3 kernel summary\n\n"
                    "Workloads: fa_fwd on B=1 H=32 N=32768 d=128 causal (the fwd_kernel<128, 12, ...> "
                    "launch of 2752 workgroups of 768 threads; the fwd_kernel<128, 8, ...> launch of 1024 "
                    "workgroups is the setup forward of the backward batch) and fa_bwd on B=4 H=16 N=4096 "
                    "d=128 causal (bwd_dq_kernel = dQ and the row terms, then bwd_main_kernel = dK/dV); "
                    "then the other forward workloads (B=4 H=16 N=2048 d=64: fwd_kernel<64, 8, ...> of "
                    "512 workgroups; B=2 H=32 N=8192 d=128 causal peaked: fwd_kernel<128, 12, ...> of "
                    "1408 workgroups) and the extension configurations of the bench line's `next` "
                    "(cross attention, grouped K/V heads forward and backward, a 4096-key window, split-KV "
                    "decoding: decode_kernel and decode_combine_kernel, and the general forward on the "
                    "decode shape); the `Cijk`/library rows are the same-board GEMM of `context_gemm`."
                    "\n\n"
                    f"Kernel sources hash (every file under csrc/): `{kernel_source_hash(ALL_KERNEL_SOURCES)}`"
                    "\n\nCommands (repo root, MI355X, ROCm 7.2):"
                    "\n\n```\n" + "\n".join(STATS_COMMANDS) + "\n```\n\n" + table + "\n")
        print(table)
        return 0

    if args.pipe_summary:
        table = pipe_summary(args.pipe_summary)
        with open(PIPE_FILE, "w") as f:
            f.write("# Pipe utilisation of the step's kernels (rocprofv3 counters)\n\n"
                    "One step of bench.py (long-context causal forward, then the backward batch), "
                    "three counter passes, last dispatch of each kernel. Shares of SIMD cycles assume "
                    "256 CUs x 4 SIMDs in 8 XCDs; the clock column is the shader clock each dispatch "
                    "held (busy cycles of an XCD over its duration), against the 2.4 GHz of the "
                    "quoted peak.\n\n"
                    f"Kernel sources hash (every file under csrc/): `{kernel_source_hash(ALL_KERNEL_SOURCES)}`"
                    "\n\nCommands (repo root):\n\n```\n"
                    + "\n".join(PIPE_COMMANDS) + "\n```\n\n" + table + "\n")
        print(table)
        return 0

    if args.hbm_summary:
        rec = hbm_summary(*args.hbm_summary)
        for path, part in ((COUNTERS_FILE, rec["fwd"]), (BWD_COUNTERS_FILE, rec["bwd"])):
            with open(path, "w") as f:
                json.dump(part, f, indent=1)
                f.write("\n")
        print(json.dumps(rec))
        return 0

    if args.gpus != 1:
        print(f"bench.py: this attention path runs on ONE GPU only (asked for {args.gpus}); "
              "heads are independent and would shard across GPUs without communication, "
              "but no multi-GPU path is built.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from io_aware_tiled_fa_amd import binding
    from io_aware_tiled_fa_amd.inputs import make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    binding.load_library()

    print(f"# generating inputs", file=sys.stderr, flush=True)
    fin = make_workload(FWD["name"])
    bin_ = make_workload(BWD["name"])
    fq, fk, fv = (device_tensor(getattr(fin, n + "_bits"), dev) for n in ("q", "k", "v"))
    bq, bk, bv, bdo = (device_tensor(getattr(bin_, n + "_bits"), dev) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(128)
    fo = torch.empty_like(fq)
    flse = torch.empty((FWD["B"], FWD["H"], FWD["N"]), dtype=torch.float32, device=dev)
    bo, blse = binding.forward(bq, bk, bv, causal=True, scale=scale)
    bdq, bdk, bdv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)
    ws = torch.empty(binding.bwd_workspace_size(BWD["B"], BWD["H"], BWD["N"], BWD["d"]),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        binding.forward(fq, fk, fv, causal=True, scale=scale, out=fo, lse=flse)
        if evs is not None:
            evs[1].record()
        binding.backward(bq, bk, bv, bo, blse, bdo, causal=True, scale=scale,
                         dq=bdq, dk=bdk, dv=bdv, workspace=ws)
        if evs is not None:
            evs[2].record()

    print(f"# warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_step = wall * 1e3 / args.steps
    ff, bf = fwd_flops(FWD), bwd_flops(BWD)
    f_med, b_med = statistics.median(fwd_ms), statistics.median(bwd_ms)
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    fwd_tf = ff / (f_med * 1e-3) / 1e12
    bwd_tf = bf / (b_med * 1e-3) / 1e12
    value = (ff + bf) / (ms_step * 1e-3) / 1e12
    achieved = ff / (fwd_avg * 1e-3) / 1e12

    def pct(xs, p):
        xs = sorted(xs)
        return xs[min(len(xs) - 1, int(round(p * (len(xs) - 1))))]

    rec = {
        "metric": "attention fwd/bwd TFLOP/s at 1 GPU + % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1), rounded to bf16)",
        "config": {
            "workload": "fa_fwd B=1 H=32 N=32768 d=128 causal + fa_bwd B=4 H=16 N=4096 d=128 causal",
            "fwd": {"B": 1, "H": 32, "N": 32768, "d": 128, "causal": True, "scale": "1/sqrt(d)"},
            "bwd": {"B": 4, "H": 16, "N": 4096, "d": 128, "causal": True, "scale": "1/sqrt(d)"},
            "parallelism": "single GPU",
        },
        "fwd": {
            "tflops": round(fwd_tf, 2), "frac_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
            "ms_median": round(f_med, 4), "ms_p10": round(pct(fwd_ms, 0.1), 4),
            "ms_p90": round(pct(fwd_ms, 0.9), 4), "useful_tflop": round(ff / 1e12, 4),
        },
        "bwd": {
            "tflops": round(bwd_tf, 2), "frac_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
            "ms_median": round(b_med, 4), "ms_p10": round(pct(bwd_ms, 0.1), 4),
            "ms_p90": round(pct(bwd_ms, 0.9), 4), "useful_tflop": round(bf / 1e12, 4),
        },
        "roofline": {
            "kernel": FWD_KERNEL_DESC,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": read_traffic(),
            "algorithmic_bytes": fwd_algorithmic_bytes(FWD),
            "avg_launch_ms": round(fwd_avg, 4),
        },
        "cpu_baseline": None,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_workloads:
        print("# the other forward workloads", file=sys.stderr, flush=True)
        rec["workloads"] = measure_workloads(binding, torch, dev)
    if not args.no_next:
        print("# extension configurations", file=sys.stderr, flush=True)
        rec["next"] = measure_next(binding, torch, dev)
        print("# dense bf16 GEMM of the vendor library on the same GPU (context)", file=sys.stderr, flush=True)
        rec["context_gemm"] = library_gemm_rate(torch, dev)
    if not args.no_cpu_baseline:
        print("# cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(fin, bin_, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


def library_gemm_rate(torch, dev, n: int = 8192, reps: int = 150) -> dict:
    """torch.matmul of two n x n bf16 matrices (hipBLASLt) on the same GPU:
    what a plain dense product sustains on this board, whose clock settles
    where its power limit holds it, timed over ~0.1 s of back-to-back calls
    like the attention steps.  Context for the percentages above (all
    against the 2.5 PFLOP/s published peak); no part of the attention path."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(30):  # (the library picks its kernel on the first calls)
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del c
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"what": f"torch.matmul bf16 {n}x{n}x{n} (vendor library)", "ms": round(ms, 4),
            "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def back_to_back_ms(torch, call, reps: int = 10, batches: int = 5) -> dict:
    """Kernel time of ``call`` (a raw C-ABI launch with its arguments already
    marshalled): ``batches`` runs of ``reps`` launches back to back between
    two events on the current stream, after one untimed launch; the median,
    min and max over the batches of the time per launch.  No host-side
    validation or synchronisation sits inside a timed batch."""
    call()
    torch.cuda.synchronize()
    per = []
    for _ in range(batches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / reps)
    return {"ms_median": round(statistics.median(per), 4), "ms_min": round(min(per), 4),
            "ms_max": round(max(per), 4), "launches": reps * batches}


def raw_forward(lib, torch, q, k, v, o, lse, causal, window=0, scale=None):
    """A zero-argument launcher of fa_fwd / fa_fwd_qk / fa_fwd_ex (the
    narrowest that covers the shapes), arguments marshalled once."""
    B, Nq, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    st = torch.cuda.current_stream().cuda_stream
    p = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    if Hkv == H and window == 0 and Nq == Nk:
        args, fn = p + (B, H, Nq, d, scale, int(causal), st), lib.fa_fwd
    elif Hkv == H and window == 0:
        args, fn = p + (B, H, Nq, Nk, d, scale, int(causal), st), lib.fa_fwd_qk
    else:
        args, fn = p + (B, H, Hkv, Nq, Nk, d, scale, int(causal), int(window), st), lib.fa_fwd_ex

    def call():
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"forward launch failed: {lib.fa_status_string(rc).decode()}")
    return call


def measure_workloads(binding, torch, dev) -> dict:
    """The two other d = 128 / d = 64 forward workloads at full size, timed
    back to back through the C ABI, each against its own roofline: the
    non-causal d = 64 batch (matrix-core bound with the softmax's VALU work
    close behind: at d = 64 a score costs half the matrix work of d = 128
    for the same exponential) and the peaked causal N = 8192 batch."""
    from io_aware_tiled_fa_amd.inputs import make_workload

    lib = binding.load_library()
    out = {}
    for name, causal in (("fwd_b4_h16_n2048_d64", False), ("fwd_b2_h32_n8192_d128_causal_peaked", True)):
        inp = make_workload(name)
        q, k, v = (device_tensor(getattr(inp, n + "_bits"), dev) for n in ("q", "k", "v"))
        B, N, H, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        t = back_to_back_ms(torch, raw_forward(lib, torch, q, k, v, o, lse, causal), reps=20 if N < 4096 else 5)
        cfg = dict(B=B, H=H, N=N, d=d, causal=causal)
        fl = fwd_flops(cfg)
        tf = fl / (t["ms_median"] * 1e-3) / 1e12
        byts = fwd_algorithmic_bytes(cfg)
        out[name] = dict(t, useful_tflop=round(fl / 1e12, 4), tflops=round(tf, 2), bound="mfma",
                         frac_peak=round(tf / PEAK_BF16_TFLOPS, 4), algorithmic_bytes=byts,
                         hbm_gbs_algorithmic=round(byts / (t["ms_median"] * 1e-3) / 1e9, 1))
        del q, k, v, o, lse, inp
    return out


def measure_next(binding, torch, dev) -> dict:
    """One configuration per extension, timed back to back through the C ABI
    (back_to_back_ms); inputs seeded N(0,1) bf16 made on the GPU."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    lib = binding.load_library()

    def rnd(*shape):
        return torch.randn(*shape, device=dev, dtype=torch.bfloat16, generator=g)

    out = {}

    def mfma_entry(name, desc, flops, t):
        tf = flops / (t["ms_median"] * 1e-3) / 1e12
        out[name] = dict(t, config=desc, tflops=round(tf, 2), bound="mfma", frac_peak=round(tf / PEAK_BF16_TFLOPS, 4))

    def empty_out(q):
        return torch.empty_like(q), torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=dev)

    # cross attention: 4096 queries at the end of a 16384-key context
    B, H, Nq, Nk, d = 1, 32, 4096, 16384, 128
    q, k, v = rnd(B, Nq, H, d), rnd(B, Nk, H, d), rnd(B, Nk, H, d)
    o, lse = empty_out(q)
    fl = 4.0 * B * H * d * visible_pairs(Nq, Nk, True)
    mfma_entry("fwd_cross_b1_h32_nq4096_nk16384_d128_causal", "fa_fwd_qk", fl,
               back_to_back_ms(torch, raw_forward(lib, torch, q, k, v, o, lse, True)))
    del q, k, v, o, lse

    # grouped K/V heads, forward and backward
    B, H, Hkv, N, d = 2, 32, 8, 8192, 128
    q, do = rnd(B, N, H, d), rnd(B, N, H, d)
    k, v = rnd(B, N, Hkv, d), rnd(B, N, Hkv, d)
    o, lse = empty_out(q)
    fl = 4.0 * B * H * d * visible_pairs(N, N, True)
    mfma_entry("fwd_gqa_b2_h32_hkv8_n8192_d128_causal", "fa_fwd_ex", fl,
               back_to_back_ms(torch, raw_forward(lib, torch, q, k, v, o, lse, True)))
    ws_bytes = binding.bwd_workspace_size(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = torch.cuda.current_stream().cuda_stream
    bargs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
             dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, N, d, 1.0 / math.sqrt(d), 1, 0, ws.data_ptr(), ws_bytes, st)

    def bwd_call():
        rc = lib.fa_bwd_ex(*bargs)
        if rc != 0:
            raise RuntimeError(lib.fa_status_string(rc).decode())
    mfma_entry("bwd_gqa_b2_h32_hkv8_n8192_d128_causal", "fa_bwd_ex", 2.5 * fl, back_to_back_ms(torch, bwd_call, reps=5))
    del q, k, v, do, o, lse, ws, dq, dk, dv

    # sliding window of 4096 keys over a 32768-token sequence
    B, H, N, d, W = 1, 32, 32768, 128, 4096
    q, k, v = rnd(B, N, H, d), rnd(B, N, H, d), rnd(B, N, H, d)
    o, lse = empty_out(q)
    fl = 4.0 * B * H * d * visible_pairs(N, N, True, W)
    mfma_entry("fwd_window4096_b1_h32_n32768_d128_causal", "fa_fwd_ex", fl,
               back_to_back_ms(torch, raw_forward(lib, torch, q, k, v, o, lse, True, window=W), reps=5))
    del q, k, v, o, lse

    # split-KV decoding: one new token per sequence against a 32768-token cache
    B, H, Hkv, Nq, Nk, d = 8, 32, 8, 1, 32768, 128
    q, k, v = rnd(B, Nq, H, d), rnd(B, Nk, Hkv, d), rnd(B, Nk, Hkv, d)
    need = lib.fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d, 1, 0, 0)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    o, lse = empty_out(q)
    st = torch.cuda.current_stream().cuda_stream
    dargs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv, Nq, Nk, d,
             1.0 / math.sqrt(d), 1, 0, 0, ws.data_ptr(), ws.numel(), st)

    def dec_call():
        rc = lib.fa_fwd_decode(*dargs)
        if rc != 0:
            raise RuntimeError(lib.fa_status_string(rc).decode())
    t = back_to_back_ms(torch, dec_call, reps=50)
    byts = 2 * B * Nk * Hkv * d * 2 + 2 * B * Nq * H * d * 2 + B * H * Nq * 4
    gbs = byts / (t["ms_median"] * 1e-3) / 1e9
    out["decode_b8_h32_hkv8_nq1_nk32768_d128"] = dict(
        t, config="fa_fwd_decode", gbs=round(gbs, 1), bound="hbm", frac_peak=round(gbs / PEAK_HBM_GBS, 4),
        algorithmic_bytes=byts)
    out["decode_b8_h32_hkv8_nq1_nk32768_d128"]["general_forward_ms"] = back_to_back_ms(
        torch, raw_forward(lib, torch, q, k, v, o, lse, True), reps=20)["ms_median"]
    return out


if __name__ == "__main__":
    sys.exit(main())
