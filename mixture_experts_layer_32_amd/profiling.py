"""Summaries of rocprofv3 output for the layer's kernels (text, for profiles/).

    python -m mixture_experts_layer_32_amd.profiling --workload latent_decode \
        --trace <trace dir> --fetch <FETCH_SIZE dir> --write <WRITE_SIZE dir> \
        --copy-fetch <copy FETCH_SIZE dir> --copy-write <copy WRITE_SIZE dir> \
        --bench-json <bench.py output of the traced run>

reads the CSV files of

  rocprofv3 --kernel-trace --stats -o trace --output-format csv -- python3 bench.py ...
  rocprofv3 --pmc FETCH_SIZE -o fetch --output-format csv -- python3 bench.py ...
  rocprofv3 --pmc WRITE_SIZE -o write --output-format csv -- python3 bench.py ...
  rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE ... -- python3 bench.py --copy-calibration

and writes profiles/<workload>_kernels_trace.md (per-kernel durations) and
profiles/<kernel>_<workload>_hbm.txt (HBM bytes per launch of the expert
kernels, scaled by what the same counters read for a 1 GiB device copy;
<kernel> is ffn_stream for the fused FC1 + FC2 kernel, gemm_stream for the
weight-streaming GEMMs, gemm_grouped for the persistent bf16 grouped GEMM,
gemm_fp8w for the fp8-weight one and gemm_tiled for the LDS-tiled one; with
--tokens T the workload is named <workload>_T<T>).  --sweep-summary writes
the table of a sweep over workloads and batches from their bench lines and
HBM files.
The HBM file records a hash of the sources its kernel depends on (its own
file, the shared headers, the host planner and the routing); bench.py
reports its traffic only while they still hash the same.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")
# sources that decide what the expert kernels read and write
# sources an expert kernel's HBM traffic depends on: its own file, the shared
# headers, the host planner (tiles, grids) and the routing (row order)
COMMON_SOURCES = ("csrc/common.hpp", "csrc/kernels.hpp", "csrc/api.cpp", "csrc/routing.hip")
KIND_SOURCE = {"ffn_stream": "csrc/ffn_stream.hip", "gemm_stream": "csrc/gemm_stream.hip",
               "gemm_tiled": "csrc/gemm_tiled.hip", "gemm_grouped": "csrc/gemm_grouped.hip",
               "gemm_fp8w": "csrc/gemm_fp8w.hip"}
COPY_BYTES = 1 << 30  # bench.py --copy-calibration: 1 GiB read + 1 GiB written per launch


def sources_hash(kind: str) -> str:
    """Hash of the sources the traffic of expert kernel `kind` depends on."""
    h = hashlib.sha256()
    for rel in COMMON_SOURCES + (KIND_SOURCE[kind],):
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    n = name.replace("void ", "").replace("lmoe::(anonymous namespace)::", "")
    return n.replace("lmoe::", "").replace("unsigned short", "bf16").replace("unsigned char", "u8")


def expert_kernel_kind(name: str) -> str | None:
    """Which expert-FFN kernel a profiled kernel name is: "ffn_stream" (fused
    FC1 + FC2), "gemm_stream" (weight streaming), "gemm_grouped" (the
    persistent 256 x 256 grouped kernel), "gemm_fp8w" (fp8 weights streamed
    into registers) or "gemm_tiled" (grouped LDS-tiled: the 128 x 256
    tile), else None (dense GEMMs and routing kernels)."""
    if "ffn_stream_kernel" in name:
        return "ffn_stream"
    if "gemm_grouped_kernel<" in name:
        # the third template argument (DENSE) marks the dense projections
        # run on the same tiles
        args = [a.strip() for a in name.split("<", 1)[1].split(">(")[0].split(",")]
        return None if len(args) > 2 and args[2] == "true" else "gemm_grouped"
    if "gemm_fp8w_kernel<" in name:
        return "gemm_fp8w"
    if "gemm_stream_kernel<" in name:
        return "gemm_stream"
    if "gemm_tiled_kernel<" in name and "TileCfg<128, 256" in name:
        return "gemm_tiled"
    # the 256 x 256 tile serves the dense projections too: only an instance
    # with an activation (the experts' FC1; the dense GEMMs have none, the
    # shared experts run on other tiles) is attributed
    if "gemm_tiled_kernel<" in name and "TileCfg<256, 256" in name and _act_arg(name) != "0":
        return "gemm_tiled"
    return None


def _act_arg(name: str) -> str:
    """The ACT template argument of an expert GEMM kernel name: the first of
    the grouped and fp8 kernels, the last of the LDS-tiled kernel, the second
    to last of the streaming kernel."""
    args = [a.strip() for a in name.split("<", 1)[1].split(">(")[0].split(",")]
    if "gemm_grouped_kernel<" in name or "gemm_fp8w_kernel<" in name:
        return args[0]
    if "gemm_tiled_kernel<" in name:
        return args[-1]
    return args[-2]


def expert_stage(name: str) -> str | None:
    """The stage an expert kernel runs: "ffn" for the fused kernel, else
    "fc1" when its activation template argument (ACT) is not 0 (squared ReLU
    1, SwiGLU 2), "fc2" when it is."""
    kind = expert_kernel_kind(name)
    if kind is None:
        return None
    if kind == "ffn_stream":
        return "ffn"
    return "fc1" if _act_arg(name) != "0" else "fc2"


def _one(path_dir: str, suffix: str) -> str:
    got = sorted(glob.glob(os.path.join(path_dir, "*" + suffix)))
    if not got:
        raise FileNotFoundError("no *%s under %s" % (suffix, path_dir))
    return got[0]


def kernel_stats(trace_dir: str):
    rows = []
    with open(_one(trace_dir, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return rows


def counter_per_dispatch(pmc_dir: str, counter: str):
    """kernel name -> (mean counter value per dispatch in KiB, dispatches)."""
    acc = defaultdict(list)
    with open(_one(pmc_dir, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def copy_reading(pmc_dir: str, counter: str) -> float:
    """The counter's per-dispatch reading (KiB) for the 1 GiB copy kernel."""
    per = counter_per_dispatch(pmc_dir, counter)
    copies = [v for k, (v, _) in per.items() if "copyBuffer" in k]
    if not copies:
        raise RuntimeError("no copy kernel in %s" % pmc_dir)
    return max(copies)


def write_trace_md(workload: str, trace_dir: str, bench_json: str | None, out: str):
    rows = kernel_stats(trace_dir)
    lines = ["# Kernel durations, workload %s" % workload, "",
             "Command (from a scratch directory, TMPDIR=/tmp):", "",
             "    rocprofv3 --kernel-trace --stats -d <dir> -o trace --output-format csv -- "
             "python3 bench.py --workload %s --steps 10 --warmup 3 --no-cpu-baseline" % workload,
             "", "rocprofv3 kernel_stats (durations in microseconds, all calls of the run):", "",
             "| kernel | calls | avg us | min us | max us | % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.1f |" % (
            short_name(r["name"])[:150], r["calls"], r["avg_us"], r["min_us"], r["max_us"], r["pct"]))
    if bench_json and os.path.exists(bench_json):
        with open(bench_json) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        lines += ["", "bench.py line of the same profiled run (HIP events per stage, ms):", "",
                  "    ms_per_step %s" % b["ms_per_step"],
                  "    " + " ".join("%s=%s" % kv for kv in b["stage_ms"].items())]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_hbm_txt(workload: str, kind: str, fetch_dir: str, write_dir: str, cfetch: str,
                  cwrite: str, trace_dir: str | None, out: str, tokens: int = 0):
    # factor: true KiB per counted KiB, from the copy's known 1 GiB each way
    cf, cw = copy_reading(cfetch, "FETCH_SIZE"), copy_reading(cwrite, "WRITE_SIZE")
    ff, fw = (COPY_BYTES / 1024) / cf, (COPY_BYTES / 1024) / cw
    fetch = counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = counter_per_dispatch(write_dir, "WRITE_SIZE")
    avg = {}
    if trace_dir:
        avg = {r["name"]: r["avg_us"] for r in kernel_stats(trace_dir)}
    tk = " --tokens %d" % tokens if tokens else ""
    lines = ["# HBM traffic of the expert GEMM kernels, workload %s%s" % (
                 workload, " at T=%d" % tokens if tokens else ""),
             "# commands (from a scratch directory, TMPDIR=/tmp):",
             "#   rocprofv3 --pmc FETCH_SIZE -d <dir> -o fetch --output-format csv -- "
             "python3 bench.py --workload %s%s --steps 2 --warmup 1 --no-cpu-baseline" % (workload, tk),
             "#   rocprofv3 --pmc WRITE_SIZE -d <dir> -o write --output-format csv -- "
             "python3 bench.py --workload %s%s --steps 2 --warmup 1 --no-cpu-baseline" % (workload, tk),
             "#   rocprofv3 --pmc FETCH_SIZE -d <dir> -o cf --output-format csv -- "
             "python3 bench.py --copy-calibration",
             "#   rocprofv3 --pmc WRITE_SIZE -d <dir> -o cw --output-format csv -- "
             "python3 bench.py --copy-calibration",
             "# a 1 GiB device copy (1048576 KiB each way) reads FETCH_SIZE %.1f and WRITE_SIZE"
             " %.1f KiB per dispatch: scale factors %.4f and %.4f" % (cf, cw, ff, fw),
             "workload=%s" % workload,
             "tokens=%d" % tokens,
             "sources_sha256=%s" % sources_hash(kind),
             "fetch_scale=%.6f" % ff,
             "write_scale=%.6f" % fw]
    for name, (fv, n) in sorted(fetch.items()):
        st = expert_stage(name)
        if not st:
            continue
        wv = write.get(name, (0.0, 0))[0]
        rd, wr = fv * ff * 1024.0, wv * fw * 1024.0
        lines.append("%s_kernel=%s" % (st, short_name(name)))
        lines.append("%s_fetch_kib_per_dispatch=%.1f" % (st, fv))
        lines.append("%s_write_kib_per_dispatch=%.1f" % (st, wv))
        lines.append("%s_dispatches=%d" % (st, n))
        lines.append("%s_hbm_read_bytes=%.0f" % (st, rd))
        lines.append("%s_hbm_write_bytes=%.0f" % (st, wr))
        lines.append("%s_hbm_bytes=%.0f" % (st, rd + wr))
        if name in avg:
            lines.append("%s_avg_us=%.2f" % (st, avg[name]))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


REGIME_KERNEL = {"fused": "ffn_stream", "stream": "gemm_stream", "tiled": "gemm_tiled",
                 "grouped": "gemm_grouped", "fp8w": "gemm_fp8w"}


def hbm_file(workload: str, kind: str) -> str:
    """kind: "ffn_stream", "gemm_stream", "gemm_tiled", "gemm_grouped" or "gemm_fp8w"."""
    return os.path.join(PROFILES, "%s_%s_hbm.txt" % (kind, workload))


def read_hbm(workload: str, stage: str, regime: str):
    """HBM bytes per launch of the FC1/FC2 (or fused, stage "ffn") kernel of
    the expert regime ("fused", "stream", "tiled", "grouped", "fp8w") from the committed
    summary, or None when there is none or the kernel sources changed since."""
    path = hbm_file(workload, REGIME_KERNEL[regime])
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k] = v
    if kv.get("sources_sha256") != sources_hash(REGIME_KERNEL[regime]):
        return None
    v = kv.get("%s_hbm_bytes" % stage)
    return float(v) if v is not None else None


COUNTER_PASSES = (
    "GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_MFMA",
    "GRBM_GUI_ACTIVE SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_LDS_DATA_FIFO_FULL "
    "SQ_LDS_CMD_FIFO_FULL SQ_VMEM_TA_ADDR_FIFO_FULL SQ_VMEM_TA_CMD_FIFO_FULL SQ_INST_LEVEL_VMEM",
    "GRBM_GUI_ACTIVE TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum TCP_PENDING_STALL_CYCLES_sum "
    "TCP_TCC_READ_REQ_sum TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum "
    "TCC_TAG_STALL_sum",
)
N_XCD, N_SIMD, N_CU = 8, 1024, 256
MFMA_PEAK_BF16 = 2.5e15      # dense bf16 MFMA, flop/s at the 2.4 GHz peak clock


def counter_means(pmc_dirs):
    """kernel name -> counter -> mean value per dispatch, over the passes."""
    out = defaultdict(dict)
    for d in pmc_dirs:
        acc = defaultdict(lambda: defaultdict(list))
        with open(_one(d, "counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for k, cs in acc.items():
            for c, v in cs.items():
                if c != "GRBM_GUI_ACTIVE" or c not in out[k]:
                    out[k][c] = sum(v) / len(v)
    return out


def write_counters_md(workload: str, pmc_dirs, trace_dir: str | None, out: str):
    """Per expert GEMM kernel: MFMA utilisation from the SQ counters, the
    wave-state split, LDS and vector-memory stalls and the L2 hit rate."""
    avg_us = {}
    if trace_dir:
        avg_us = {r["name"]: r["avg_us"] for r in kernel_stats(trace_dir)}
    m = counter_means(pmc_dirs)
    lines = ["# Hardware counters of the expert GEMM kernels, workload %s" % workload, "",
             "Commands (from a scratch directory, TMPDIR=/tmp), one pass per counter group:", ""]
    for p in COUNTER_PASSES:
        lines.append("    rocprofv3 --pmc %s -d <dir> -o pmc --output-format csv -- "
                     "python3 bench.py --workload %s --steps 2 --warmup 1 --no-cpu-baseline"
                     % (p, workload))
    lines += ["", "Reading the counters: GRBM_GUI_ACTIVE adds the 8 XCDs' busy cycles (per-XCD "
              "cycles = value / 8; over the kernel's traced duration this gives the clock); "
              "SQ_VALU_MFMA_BUSY_CYCLES adds the 1024 SIMDs' MFMA-busy cycles (busy fraction = "
              "value / (1024 x per-XCD cycles); a 32x32x16 bf16 MFMA counts 32 busy cycles, "
              "a 16x16x32 one 16); one SQ_INSTS_VALU_MFMA_MOPS_BF16 unit is 512 flop.  The "
              "wave-state counters are given as fractions of SQ_WAVE_CYCLES.", ""]
    for name, c in sorted(m.items()):
        st = expert_stage(name)
        if not st or "SQ_VALU_MFMA_BUSY_CYCLES" not in c:
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc)
        flop = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        lines.append("## %s: `%s`" % (st.upper(), short_name(name)[:140]))
        lines.append("")
        lines.append("- per-XCD busy cycles %.4g" % cyc)
        if name in avg_us:
            us = avg_us[name]
            lines.append("- traced average duration %.2f us: clock %.2f GHz" % (us, cyc / us / 1e3))
            lines.append("- MFMA work %.4g flop: %.1f TFLOP/s, %.3f of the %.0f TFLOP/s bf16 peak"
                         % (flop, flop / us / 1e6, flop / us / 1e6 / (MFMA_PEAK_BF16 / 1e12),
                            MFMA_PEAK_BF16 / 1e12))
        lines.append("- MFMA busy %.1f%% of SIMD cycles (%.4g MFMA instructions, %.1f busy "
                     "cycles each)" % (100 * busy, c.get("SQ_INSTS_MFMA", 0.0),
                                       c["SQ_VALU_MFMA_BUSY_CYCLES"] / max(c.get("SQ_INSTS_MFMA", 1.0), 1.0)))
        wc = c.get("SQ_WAVE_CYCLES", 0.0)
        if wc:
            lines.append("- wave cycles: issuing %.1f%%, waiting to issue %.1f%%, waiting on "
                         "s_waitcnt %.1f%%" % tuple(100 * c.get(k, 0.0) / wc for k in (
                             "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY")))
        if "SQ_LDS_IDX_ACTIVE" in c:
            lines.append("- LDS bank-conflict cycles %.1f%% of LDS-active cycles; VMEM TA "
                         "address / command FIFO full %.4g / %.4g cycles"
                         % (100 * c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1.0),
                            c["SQ_VMEM_TA_ADDR_FIFO_FULL"], c["SQ_VMEM_TA_CMD_FIFO_FULL"]))
        if "TCC_HIT_sum" in c:
            h, mi = c["TCC_HIT_sum"], c["TCC_MISS_sum"]
            lines.append("- L2 hit rate %.1f%% (%.4g requests from the CUs); TA busy %.1f%%, "
                         "TCP pending-stall %.1f%% of per-CU cycles"
                         % (100 * h / max(h + mi, 1.0), c.get("TCP_TCC_READ_REQ_sum", 0.0),
                            100 * c["TA_TA_BUSY_sum"] / (N_CU * cyc),
                            100 * c["TCP_PENDING_STALL_CYCLES_sum"] / (N_CU * cyc)))
        lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _read_kv(path):
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k] = v
    return kv


def _expert_weight_bytes(cfg, touched):
    """Expert-weight bytes that FC1 + FC2 of one layer call must read: both
    matrices of every expert with tokens (SwiGLU: FC1 holds up and gate
    rows; fp8: with the row scales), the benchmark's algorithmic bytes of the
    two expert GEMMs.  Token rows, H and Y are intermediates."""
    l, m = cfg["l"], cfg["m"]
    m1 = 2 * m if cfg.get("activation") == "swiglu" else m
    dt = cfg["expert_dtype"]
    if dt == "bf16":
        return float(touched * l * (m1 + m) * 2)
    if dt == "fp8_e4m3_rowscale":
        return float(touched * (l * (m1 + m) + 4 * (m1 + l)))
    raise ValueError("sweep summary: expert dtype %s not handled" % dt)


def write_sweep_md(entries, out):
    """Table of the alpha sweep: per (workload, T) the step time, the expert
    stages' event times, their algorithmic bytes (from the bench line) and
    their HBM bytes measured by FETCH_SIZE + WRITE_SIZE (copy-calibrated,
    from profiles/<kernel>_<workload>[_T<T>]_hbm.txt)."""
    rows = ["# LatentMoE cost curve: measured expert bytes across the compression ratio",
            "",
            "Per entry, from the repository root:",
            "",
            "    python3 bench.py --workload W --tokens T --steps 20 --warmup 3 --no-cpu-baseline",
            "    rocprofv3 --pmc FETCH_SIZE ... / --pmc WRITE_SIZE ... -- python3 bench.py "
            "--workload W --tokens T --steps 2 --warmup 1 --no-cpu-baseline",
            "",
            "(the HBM files name their exact commands).  Bytes are per layer call, "
            "FC1 + FC2 of the expert GEMMs.",
            "",
            "| workload | l | N' | K | T | touched experts | ms/step | FC1+FC2 us | "
            "algorithmic expert MB | measured HBM MB | measured / algorithmic |",
            "|---|---|---|---|---|---|---|---|---|---|---|"]
    for e in entries:
        wl, T, bj = e.split(":", 2)
        with open(bj) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        cfg = b["config"]
        alg = _expert_weight_bytes(cfg, b["experts"]["touched"])
        kind = REGIME_KERNEL[cfg["expert_kernel"]]
        name = wl + ("" if int(T) == 512 else "_T%s" % T)
        kv = _read_kv(hbm_file(name, kind))
        meas = sum(float(kv[k]) for k in kv if k.endswith("_hbm_bytes"))
        st = b["stage_ms"]
        rows.append("| %s | %d | %d | %d | %d | %d | %.3f | %.1f | %.1f | %.1f | %.3f |" % (
            wl, cfg["l"], cfg["n_experts"], cfg["top_k"], int(T), b["experts"]["touched"],
            b["ms_per_step"], 1e3 * (st["fc1"] + st["fc2"]), alg / 1e6, meas / 1e6, meas / alg))
    with open(out, "w") as f:
        f.write("\n".join(rows) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--bench-json")
    ap.add_argument("--counters", action="append", default=[],
                    help="rocprofv3 --pmc output directory of one counter pass (repeatable)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="batch of a run at a non-default T (names the HBM file ..._T<T>)")
    ap.add_argument("--sweep-summary", help="write the alpha-sweep summary (markdown) here")
    ap.add_argument("--sweep", action="append", default=[],
                    help="WORKLOAD:T:BENCH_JSON entry of the sweep summary (repeatable)")
    a = ap.parse_args()
    if a.sweep_summary:
        write_sweep_md(a.sweep, a.sweep_summary)
        print(a.sweep_summary)
        return
    os.makedirs(PROFILES, exist_ok=True)
    if a.trace:
        out = os.path.join(PROFILES, "%s_kernels_trace.md" % a.workload)
        write_trace_md(a.workload, a.trace, a.bench_json, out)
        print(out)
    if a.counters:
        out = os.path.join(PROFILES, "%s_expert_counters.md" % a.workload)
        write_counters_md(a.workload, a.counters, a.trace, out)
        print(out)
    if a.fetch and a.write and a.copy_fetch and a.copy_write:
        kinds = {expert_kernel_kind(n) for n in counter_per_dispatch(a.fetch, "FETCH_SIZE")}
        kinds.discard(None)
        if len(kinds) != 1:
            raise RuntimeError("expected one expert kernel kind, found %s" % sorted(kinds))
        wl = a.workload + ("_T%d" % a.tokens if a.tokens else "")
        kind = kinds.pop()
        out = hbm_file(wl, kind)
        write_hbm_txt(a.workload, kind, a.fetch, a.write, a.copy_fetch, a.copy_write, a.trace, out,
                      a.tokens)
        print(out)


if __name__ == "__main__":
    main()
