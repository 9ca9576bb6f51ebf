"""Summarise rocprofv3 output of bench.py into short text files.

    python -m sparse_mixture_experts_46_amd.profsum --workload NAME --trace DIR
        [--pmc DIR ...] [--bench-log FILE] [--sections a,b,...] --out profiles/
        --cmd "<the rocprofv3 command lines>"

--trace : directory of a `rocprofv3 --kernel-trace --stats --output-format csv` run
--pmc   : directories of `rocprofv3 --pmc <counters> --output-format csv` runs of
          `bench.py --copy-probe-mib M ...` (any counters, one run per set).  The
          probe kernel (one fp32 negation reading M MiB and writing M MiB) gives
          the factor that turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into
          bytes.  bench.py runs one probe before each measured part, so the
          launches between two probes form one section (--sections names them).
Writes <out>/kernels_<workload>.md (trace statistics, counters per kernel) and
<out>/counters_<workload>.json: per grouped-GEMM stage ("bf16:gemm1",
"int8:gemm2", ...) of the first section, the launches, the trace's average
duration and the counters per launch, each tied to the SHA-256 of the sources
of its kernel family (the prefill DMA kernels, or the decode kernels).
"""
from __future__ import annotations

import argparse
import bisect
import csv
import glob
import gzip
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# the sources each family of grouped-GEMM kernels is built from (its
# counter figures go stale when any of them changes)
FAMILY_SRCS = {
    "prefill": ["gemm_bf16.hip", "gemm_common.h", "gemm_pingpong.h", "gemm_tile.h", "lds_dma.h",
                "moe_common.h"],
    "decode": ["gemm_bf16.hip", "gemm_common.h", "gemm_decode.h", "lds_dma.h", "moe_common.h"],
}
PROBE = "torch neg (copy probe)"
N_SIMD = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
N_XCD = 8         # GRBM_GUI_ACTIVE is summed over the 8 XCDs


def family_of(kernel: str) -> str:
    return "decode" if "gemm_decode" in kernel else "prefill"


def source_sha256(family: str) -> str:
    """SHA-256 over the sources of one kernel family."""
    h = hashlib.sha256()
    for f in FAMILY_SRCS[family]:
        h.update(open(os.path.join(PKG, "csrc", f), "rb").read())
    return h.hexdigest()


def short(name: str) -> str:
    n = name
    if "moe::" in n:
        n = re.sub(r"\(.*\)$", "", n.replace("(anonymous namespace)::", ""))
        n = n.replace("void ", "")
        return n
    m = re.search(r"at::native::[^<(]*?(\w+_kernel\w*)", n)
    if "neg_kernel" in n:
        return PROBE
    return ("torch " + m.group(1)) if m else n[:60]


def stage_of(kernel: str):
    """(weights, stage) of a grouped-GEMM kernel from its template arguments
    (the epilogue argument is 2 for the second GEMM), else None."""
    m = re.match(r"moe::(gemm_\w+_kernel)<(.*)>$", kernel)
    if not m:
        return None
    name, args = m.group(1), [s.strip() for s in m.group(2).split(",")]
    if name in ("gemm_pingpong_kernel", "gemm_tile_kernel"):
        return "bf16", "gemm2" if args[-1] == "2" else "gemm1"
    if name == "gemm_decode_kernel":
        return ("int8" if args[2] == "true" else "bf16"), "gemm2" if args[1] == "2" else "gemm1"
    if name == "gemm_decode_q4_kernel":
        return "int4", "gemm2" if args[1] == "2" else "gemm1"
    return None


def one(pattern):
    """The first file matching pattern, or pattern + ".gz", opened as text."""
    f = glob.glob(pattern, recursive=True)
    if f:
        return open(f[0])
    f = glob.glob(pattern + ".gz", recursive=True)
    if f:
        return gzip.open(f[0], "rt")
    raise FileNotFoundError(pattern)


def stats_table(trace_dir):
    rows = list(csv.DictReader(one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))))
    out = []
    for r in rows:
        out.append((short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                    float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    out.sort(key=lambda x: -x[3])
    return out


def sectioned(rows, value):
    """{(kernel, section index): [value(row)]}, a section being the launches
    after the i-th copy probe (0: before the first)."""
    probes = sorted(int(r["Dispatch_Id"]) for r in rows if short(r["Kernel_Name"]) == PROBE)
    by = {}
    for r in rows:
        k = short(r["Kernel_Name"])
        if k == PROBE:
            continue
        sec = bisect.bisect_left(probes, int(r["Dispatch_Id"]))
        by.setdefault((k, sec), []).append(value(r))
    return by


def trace_durations(trace_dir):
    rows = list(csv.DictReader(one(os.path.join(trace_dir, "**", "*kernel_trace.csv"))))
    return sectioned(rows, lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)


def pmc_values(pmc_dirs):
    """({counter: {(kernel, section): [value per launch]}}, {counter: probe value})."""
    vals, probe = {}, {}
    for d in pmc_dirs:
        rows = list(csv.DictReader(one(os.path.join(d, "**", "*counter_collection.csv"))))
        for c in sorted({r["Counter_Name"] for r in rows}):
            rc = [r for r in rows if r["Counter_Name"] == c]
            p = [float(r["Counter_Value"]) for r in rc if short(r["Kernel_Name"]) == PROBE]
            if p:
                probe[c] = p[0]
            vals[c] = sectioned(rc, lambda r: float(r["Counter_Value"]))
    return vals, probe


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--pmc", nargs="*", default=[])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--cmd", required=True)
    ap.add_argument("--probe-mib", type=int, default=1024)
    ap.add_argument("--sections", default="layer",
                    help="comma-separated names of the parts after each copy probe")
    ap.add_argument("--bench-log", help="stdout of the traced bench.py run (its JSON line)")
    a = ap.parse_args()
    names = a.sections.split(",")

    def secname(i):
        return names[i - 1] if 1 <= i <= len(names) else f"part{i}"

    os.makedirs(a.out, exist_ok=True)
    lines = [f"# rocprofv3 summary: bench.py, workload {a.workload}", "",
             "Command(s):", "", "```", a.cmd.strip(), "```", "",
             "## Kernel statistics (--kernel-trace --stats)", "",
             "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for n, c, avg, tot, pct in stats_table(a.trace)[:25]:
        lines.append(f"| `{n}` | {c} | {avg:.1f} | {tot:.3f} | {pct:.2f} |")
    dur = trace_durations(a.trace)
    lines += ["", "## Library kernels per part of the run (kernel trace)", "",
              "| part | kernel | launches | avg us |", "|---|---|---|---|"]
    for (k, sec), v in sorted(dur.items(), key=lambda kv: (kv[0][1], -sum(kv[1]))):
        if "moe::" in k:
            lines.append(f"| {secname(sec)} | `{k}` | {len(v)} | {sum(v) / len(v):.1f} |")

    bench = None
    if a.bench_log:
        js = [json.loads(l) for l in open(a.bench_log) if l.startswith("{")]
        bench = js[-1] if js else None
    if bench:
        rf = bench["roofline"]
        lines += ["", "## bench.py's own HIP-event timings in the traced run", "",
                  f"{bench['config']['workload']}: ms_per_step {bench['ms_per_step']:.4f}; "
                  f"roofline kernel `{rf['kernel']}` avg {rf['avg_ms'] * 1e3:.1f} us, "
                  f"{rf['achieved']:.0f} {rf['unit']}, frac {rf['frac']:.3f}.", "",
                  "| stage | ms |", "|---|---|"]
        lines += [f"| {k} | {v:.4f} |" for k, v in bench["stage_ms"].items()]

    rec = {"workload": a.workload, "cmd": a.cmd.strip(), "stages": {}}
    vals, probe = pmc_values(a.pmc) if a.pmc else ({}, {})
    probe_bytes = a.probe_mib * (1 << 20)
    scale = {c: probe_bytes / (probe[c] * 1024.0) for c in ("FETCH_SIZE", "WRITE_SIZE")
             if probe.get(c)}
    keys = sorted((ks for ks in dur if "moe::" in ks[0]), key=lambda ks: (ks[1], -sum(dur[ks])))
    if vals:
        lines += ["", "## Counters per launch (--pmc runs)", ""]
        if scale:
            lines += [f"Copy probe: {a.probe_mib} MiB read + {a.probe_mib} MiB written; "
                      + "; ".join(f"{c} read {probe[c]:.0f} KiB (bytes = KiB x 1024 x "
                                  f"{scale[c]:.3f})" for c in scale) + ".", ""]
        if "GRBM_GUI_ACTIVE" in vals:
            lines += ["clock = GRBM_GUI_ACTIVE / 8 XCDs / trace duration (for launches of a few "
                      "us it includes the dispatch around the kernel); MFMA busy = "
                      "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); executed "
                      "flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.", ""]
        lines += ["| part | kernel | launches | avg us | fetch MB | write MB | clock GHz | "
                  "MFMA busy | executed TFLOP |", "|---|---|---|---|---|---|---|---|---|"]

        def avg(c, ks):
            v = vals.get(c, {}).get(ks)
            return sum(v) / len(v) if v else None

        for ks in keys:
            k, sec = ks
            us = sum(dur[ks]) / len(dur[ks])
            f, w = avg("FETCH_SIZE", ks), avg("WRITE_SIZE", ks)
            fb = f * 1024 * scale["FETCH_SIZE"] if f is not None and "FETCH_SIZE" in scale else None
            wb = w * 1024 * scale["WRITE_SIZE"] if w is not None and "WRITE_SIZE" in scale else None
            gui, busy = avg("GRBM_GUI_ACTIVE", ks), avg("SQ_VALU_MFMA_BUSY_CYCLES", ks)
            mops = avg("SQ_INSTS_VALU_MFMA_MOPS_BF16", ks)
            clk = gui / N_XCD / (us * 1e3) if gui else None
            util = busy / (gui / N_XCD * N_SIMD) if gui and busy is not None else None
            xfl = mops * 512 if mops is not None else None

            def fmt(x, p):
                return "" if x is None else f"{x:.{p}f}"

            lines.append(f"| {secname(sec)} | `{k}` | {len(dur[ks])} | {us:.1f} | "
                         f"{fmt(fb and fb / 1e6, 1)} | {fmt(wb and wb / 1e6, 1)} | "
                         f"{fmt(clk, 3)} | {fmt(util, 3)} | {fmt(xfl and xfl / 1e12, 4)} |")
            st = stage_of(k)
            if st and sec == 1:
                key = f"{st[0]}:{st[1]}"
                prev = rec["stages"].get(key)
                if prev is None or prev["avg_us"] * prev["launches"] < us * len(dur[ks]):
                    rec["stages"][key] = {"kernel": k, "source_sha256": source_sha256(family_of(k)),
                                          "launches": len(dur[ks]), "avg_us": us,
                                          "fetch_bytes": fb, "write_bytes": wb,
                                          "clock_ghz": clk, "mfma_busy": util,
                                          "executed_flops": xfl}
    known = {"FETCH_SIZE", "WRITE_SIZE", "GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES",
             "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CYCLES"}
    other = sorted(c for c in vals if c not in known)
    if other:
        lines += ["", "## Other counters (average per launch, summed over the chip)", "",
                  "| part | kernel | " + " | ".join(other) + " |",
                  "|---|---|" + "---|" * len(other)]
        for ks in keys:
            if not any(vals[c].get(ks) for c in other):
                continue
            cells = []
            for c in other:
                v = vals[c].get(ks)
                cells.append(f"{sum(v) / len(v):.4g}" if v else "")
            lines.append(f"| {secname(ks[1])} | `{ks[0]}` | " + " | ".join(cells) + " |")
    open(os.path.join(a.out, f"kernels_{a.workload}.md"), "w").write("\n".join(lines) + "\n")
    if rec["stages"]:
        json.dump(rec, open(os.path.join(a.out, f"counters_{a.workload}.json"), "w"), indent=1)


if __name__ == "__main__":
    main()
