"""Summarise rocprofv3 output of bench.py into short text files.

    python -m sparse_mixture_experts_46_amd.profsum --trace DIR [--fetch DIR --write DIR]
        --workload NAME --out profiles/ --cmd "<the rocprofv3 command lines>"

--trace : directory of a `rocprofv3 --kernel-trace --stats --output-format csv` run
--fetch / --write : directories of `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
          runs of `bench.py --copy-probe-mib M ...`.  The probe kernel (one fp32
          negation reading M MiB and writing M MiB) gives the factor that turns
          each counter (KiB per dispatch) into bytes.
Writes <out>/kernels_<workload>.md and, with counters, <out>/traffic_gemm1_<workload>.json
(HBM bytes per launch of the first grouped GEMM, tied to the SHA-256 of its source).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
GEMM_SRCS = ["gemm_bf16.hip", "gemm_common.h", "gemm_pingpong.h", "gemm_tile.h", "gemm_decode.h"]


def gemm_source_sha256() -> str:
    """SHA-256 over the grouped-GEMM sources (traffic figures go stale when
    any of them changes)."""
    h = hashlib.sha256()
    for f in GEMM_SRCS:
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
        return "torch neg (copy probe)"
    return ("torch " + m.group(1)) if m else n[:60]


def one(pattern):
    f = glob.glob(pattern, recursive=True)
    if not f:
        raise FileNotFoundError(pattern)
    return f[0]


def stats_table(trace_dir):
    rows = list(csv.DictReader(open(one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    out = []
    for r in rows:
        out.append((short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                    float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    out.sort(key=lambda x: -x[3])
    return out


PROBE = "torch neg (copy probe)"


def counters(pmc_dir, counter):
    """{(kernel, section): [value per launch]}.  bench.py runs the copy probe
    once before the forward and again before the backward: launches after the
    second probe are the backward section's (whose forward also keeps gate and
    up, so the same GEMM 1 kernel writes more there)."""
    rows = list(csv.DictReader(open(one(os.path.join(pmc_dir, "**", "*counter_collection.csv")))))
    rows = [r for r in rows if r["Counter_Name"] == counter]
    probes = sorted(int(r["Dispatch_Id"]) for r in rows if short(r["Kernel_Name"]) == PROBE)
    edge = probes[1] if len(probes) > 1 else float("inf")
    by = {}
    for r in rows:
        k = short(r["Kernel_Name"])
        sec = "" if k == PROBE else ("backward" if int(r["Dispatch_Id"]) > edge else "forward")
        by.setdefault((k, sec), []).append(float(r["Counter_Value"]))
    return by


def section_durations(trace_dir):
    """{(kernel, section): [duration us per launch]} from the kernel trace,
    split at the second copy probe as in counters()."""
    rows = list(csv.DictReader(open(one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))))
    probes = sorted(int(r["Dispatch_Id"]) for r in rows if short(r["Kernel_Name"]) == PROBE)
    edge = probes[1] if len(probes) > 1 else float("inf")
    by = {}
    for r in rows:
        k = short(r["Kernel_Name"])
        sec = "" if k == PROBE else ("later" if int(r["Dispatch_Id"]) > edge else "forward")
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        by.setdefault((k, sec), []).append(us)
    return by


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--cmd", required=True)
    ap.add_argument("--probe-mib", type=int, default=1024)
    ap.add_argument("--gemm1", default="gemm_pingpong_kernel<256, 256, 4, 2, 2, 3, true, 0>")
    ap.add_argument("--bench-log", help="stdout of the traced bench.py run (its JSON line)")
    a = ap.parse_args()
    os.makedirs(a.out, exist_ok=True)
    tab = stats_table(a.trace)
    lines = [f"# rocprofv3 kernel statistics: bench.py, workload {a.workload}", "",
             "Command(s):", "", "```", a.cmd.strip(), "```", "",
             "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for n, c, avg, tot, pct in tab[:25]:
        lines.append(f"| `{n}` | {c} | {avg:.1f} | {tot:.3f} | {pct:.2f} |")
    dur = section_durations(a.trace)
    lines += ["", "## The same kernel trace split at the second copy probe", "",
              "forward: the prefill forward's launches; later: the backward (with the forward "
              "that keeps gate and up), then the decode.", "",
              "| section | kernel | launches | avg us |", "|---|---|---|---|"]
    for (k, sec), v in sorted(dur.items(), key=lambda kv: -sum(kv[1]))[:30]:
        if "moe::" in k:
            lines.append(f"| {sec} | `{k}` | {len(v)} | {sum(v) / len(v):.1f} |")
    if a.bench_log:
        js = [json.loads(l) for l in open(a.bench_log) if l.startswith("{")]
        if js:
            b = js[-1]
            lines += ["", "## bench.py's own HIP-event timings in the traced run", "",
                      f"Prefill ({b['config']['workload']}): ms_per_step {b['ms_per_step']:.3f}; "
                      f"roofline kernel `{b['roofline']['kernel']}` avg "
                      f"{b['roofline']['avg_ms'] * 1e3:.1f} us, "
                      f"{b['roofline']['achieved']:.0f} TFLOP/s.", "",
                      "| stage | ms |", "|---|---|"]
            lines += [f"| {k} | {v:.3f} |" for k, v in b["stage_ms"].items()]
            if "backward" in b:
                bb = b["backward"]
                rf = bb["roofline"]
                lines += ["", f"Backward ({bb['workload']}): ms_per_step {bb['ms_per_step']:.3f}, "
                              f"{bb['active_tflops']:.0f} TFLOP/s algorithmic; dominant stage "
                              f"`{rf['kernel']}` {rf['avg_ms'] * 1e3:.1f} us, "
                              f"{rf['achieved']:.0f} TFLOP/s.", "",
                          "| stage | ms |", "|---|---|"]
                lines += [f"| {k} | {v:.3f} |" for k, v in bb["stage_ms"].items()]
            if "decode" in b:
                dd = b["decode"]
                lines += ["", f"Decode ({dd['workload']}): ms_per_step {dd['ms_per_step']:.3f}, "
                              f"{dd['hbm_gbs']:.0f} GB/s of expert weights.", "",
                          "| stage | ms |", "|---|---|"]
                lines += [f"| {k} | {v:.3f} |" for k, v in dd["stage_ms"].items()]
    if a.fetch and a.write:
        f = counters(a.fetch, "FETCH_SIZE")
        w = counters(a.write, "WRITE_SIZE")
        probe_bytes = a.probe_mib * (1 << 20)
        fk = f[(PROBE, "")][0]
        wk = w[(PROBE, "")][0]
        fscale = probe_bytes / (fk * 1024.0)
        wscale = probe_bytes / (wk * 1024.0)
        lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
                  f"Copy probe: {a.probe_mib} MiB read + {a.probe_mib} MiB written; "
                  f"FETCH_SIZE read {fk:.0f} KiB (scale x{fscale:.3f}), "
                  f"WRITE_SIZE read {wk:.0f} KiB (scale x{wscale:.3f}).", "",
                  "| section | kernel | launches | fetch MB/launch (scaled) | write MB/launch (scaled) |",
                  "|---|---|---|---|---|"]
        rec = {}
        for k, sec in sorted(set(f) & set(w), key=lambda ks: (ks[1] != "forward", ks[0])):
            if "moe::" not in k:
                continue
            fb = sum(f[(k, sec)]) / len(f[(k, sec)]) * 1024 * fscale
            wb = sum(w[(k, sec)]) / len(w[(k, sec)]) * 1024 * wscale
            rec[(k, sec)] = (fb, wb)
            lines.append(f"| {sec} | `{k}` | {len(f[(k, sec)])} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
        g1 = [k for k in rec if a.gemm1 in k[0] and k[1] == "forward"]
        if g1:
            fb, wb = rec[g1[0]]
            sha = gemm_source_sha256()
            json.dump({"workload": a.workload, "kernel": g1[0][0], "fetch_bytes": fb,
                       "write_bytes": wb, "bytes_per_launch": fb + wb,
                       "fetch_scale": fscale, "write_scale": wscale,
                       "gemm_source_sha256": sha, "cmd": a.cmd.strip()},
                      open(os.path.join(a.out, f"traffic_gemm1_{a.workload}.json"), "w"), indent=1)
    open(os.path.join(a.out, f"kernels_{a.workload}.md"), "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
