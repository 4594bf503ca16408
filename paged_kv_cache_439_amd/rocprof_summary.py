"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m paged_kv_cache_439_amd.rocprof_summary trace STATS_CSV OUT_MD --cmd "..." \
        [--kernel-trace TRACE_CSV --last N]
    python -m paged_kv_cache_439_amd.rocprof_summary traffic FETCH_CSV WRITE_CSV OUT_JSON OUT_MD \
        --copy-bytes N --cmd-fetch "..." --cmd-write "..."
    python -m paged_kv_cache_439_amd.rocprof_summary counters COUNTER_CSV OUT_MD --cmd "..."

trace:   kernel-trace statistics of this library's kernels as a table
         (with --last N, also the mean of each kernel's last N dispatches).
traffic: HBM bytes per dispatch from the FETCH_SIZE and WRITE_SIZE counter
         passes (KiB per dispatch), each scaled by what the same counter
         reads for a plain device copy of a known size in the same run (the
         last three copy dispatches whose WRITE_SIZE equals that size). The
         JSON carries the sha256 of the decode sources it was measured on;
         bench.py reports the traffic only while the sources still match.
counters: SQ/GRBM counters per dispatch of this library's kernels (median
         over dispatches), with the MFMA and VALU busy percentages (the
         MfmaUtil and VALUBusy expressions of rocprofiler-sdk's counter
         definitions, over the per-XCD active cycles), the shader clock the
         dispatch ran at and the bf16 MFMA flops the counters saw (512 per
         SQ_INSTS_VALU_MFMA_MOPS_BF16).
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_439_amd", "csrc", f)
                  for f in ("decode_device.h", "decode.hip", "pa_device.h")]


def decode_source_hash():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _ours(name):
    return "pa::" in name


def _short(name):
    name = re.sub(r"\(pa::\w+\)$", "", name.replace("void ", ""))
    return re.sub(r"\(char const\*.*$", "", name)


def _last_means(trace_csv, last):
    """Mean duration (us) of each kernel's last `last` dispatches in a
    kernel-trace CSV: the calls a benchmark times after its warm-up."""
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        if _ours(r["Kernel_Name"]):
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            per[_short(r["Kernel_Name"])].append((t0, (t1 - t0) / 1e3))
    return {k: sum(d for _, d in sorted(v)[-last:]) / len(sorted(v)[-last:]) for k, v in per.items()}


def trace(stats_csv, out_md, cmd, trace_csv=None, last=0):
    rows = [r for r in csv.DictReader(open(stats_csv)) if _ours(r["Name"])]
    tail = _last_means(trace_csv, last) if trace_csv and last > 0 else None
    head = "| kernel | calls | avg us | min us | max us |"
    rule = "|---|---|---|---|---|"
    if tail is not None:
        head += f" avg of last {last} us |"
        rule += "---|"
    lines = ["# Kernel trace: libpagedattn kernels", "", "Command:", "", "```", cmd, "```", ""]
    if tail is not None:
        lines += [f"The last column averages each kernel's last {last} dispatches (in start order), the calls a "
                  "benchmark leg times after its warm-up.", ""]
    lines += [head, rule]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        line = (f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        if tail is not None:
            t = tail.get(_short(r["Name"]))
            line += f" {t:.2f} |" if t is not None else " - |"
        lines.append(line)
    open(out_md, "w").write("\n".join(lines) + "\n")


# kernel template arguments -> workload name (dtype bf16, head_dim, heads per wave)
KERNEL_WORKLOAD = {
    ("64", "1"): "bf16_mha_decode_b64",
    ("128", "2"): "bf16_gqa_decode_b256_shared_prefix",
    ("128", "4"): "bf16_gqa_decode_b512_lognormal",
}


def _per_kernel(path, counter):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows if r["Counter_Name"] == counter]


def traffic(fetch_csv, write_csv, out_json, out_md, copy_bytes, cmd_fetch, cmd_write):
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    # the copy-probe dispatches are found in the write pass (WRITE_SIZE equals
    # the probe size); the fetch pass dispatches the same kernels in order
    wnames = [n for n, _ in write]
    probe_kib = copy_bytes / 1024
    probe_idx = [i for i, (n, v) in enumerate(write) if "copyBuffer" in n and abs(v - probe_kib) < 1][-3:]
    fs = probe_kib / (sum(fetch[i][1] for i in probe_idx) / len(probe_idx))
    ws = probe_kib / (sum(write[i][1] for i in probe_idx) / len(probe_idx))
    assert [fetch[i][0] for i in probe_idx] == [wnames[i] for i in probe_idx]
    per = collections.defaultdict(lambda: dict(fetch=[], write=[]))
    for (n, v), (n2, w) in zip(fetch, write):
        assert n == n2, "the two passes dispatched different kernels"
        if _ours(n):
            per[_short(n)]["fetch"].append(v * fs * 1024)
            per[_short(n)]["write"].append(w * ws * 1024)
    kernels = {k: dict(dispatches=len(v["fetch"]), fetch_bytes=sum(v["fetch"]) / len(v["fetch"]),
                       write_bytes=sum(v["write"]) / len(v["write"])) for k, v in per.items()}
    # per workload and split: the balanced split's two kernels, or the
    # fixed-slice split's main and merge kernels
    workloads = {}
    # Main kernels name the query and pool types (E4M3 pools: unsigned char;
    # the paired-head kernel of the b64 workload has one head per wave too),
    # merge kernels only the output type, so a merge kernel's average is
    # shared by a workload's bf16 and E4M3 calls (a few MB against GBs).
    merges = {}
    for k, v in kernels.items():
        m = re.search(r"paged_decode(_balanced)?_merge_kernel<unsigned short, (\d+), (\d+)>", k)
        if m:
            merges[("balanced" if m.group(1) else "fixed", m.group(2), m.group(3))] = (k, v)
    for k, v in kernels.items():
        m = re.search(r"paged_decode(_balanced)?_kernel<unsigned short, unsigned (short|char), (\d+), (\d+)", k)
        if not m:
            continue
        wname = KERNEL_WORKLOAD.get((m.group(3), m.group(4)))
        if not wname:
            continue
        wname += "_e4m3" if m.group(2) == "char" else ""
        split = "balanced" if m.group(1) else "fixed"
        w = workloads.setdefault(wname, {}).setdefault(split, dict(hbm_bytes_per_launch=0.0, kernels=[]))
        for kk, vv in [(k, v)] + ([merges[(split, m.group(3), m.group(4))]]
                                  if (split, m.group(3), m.group(4)) in merges else []):
            w["hbm_bytes_per_launch"] += vv["fetch_bytes"] + vv["write_bytes"]
            w["kernels"].append(kk)
    for ws_ in workloads.values():
        for w in ws_.values():
            w["hbm_bytes_per_launch"] = int(w["hbm_bytes_per_launch"])
    rec = dict(kernel_source_sha256=decode_source_hash(), fetch_scale=fs, write_scale=ws,
               copy_probe_bytes=copy_bytes, cmd_fetch=cmd_fetch, cmd_write=cmd_write,
               kernels={k: {kk: (int(vv) if "bytes" in kk else vv) for kk, vv in v.items()}
                        for k, v in kernels.items()},
               workloads=workloads)
    json.dump(rec, open(out_json, "w"), indent=1)
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             f"Calibration: a {copy_bytes} B device copy reads as FETCH_SIZE x{fs:.4f} and "
             f"WRITE_SIZE x{ws:.4f} of its true size; every value below is scaled by those factors.",
             "", "Commands:", "", "```", cmd_fetch, cmd_write, "```", "",
             "| kernel | dispatches | fetch MB | write MB |", "|---|---|---|---|"]
    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["fetch_bytes"]):
        lines.append(f"| `{k}` | {v['dispatches']} | {v['fetch_bytes'] / 1e6:.1f} | {v['write_bytes'] / 1e6:.2f} |")
    lines += ["", "Per decode call (main + merge kernels):", ""]
    for wname, ws_ in workloads.items():
        for split, w in ws_.items():
            lines.append(f"- {wname}, {split} split: {w['hbm_bytes_per_launch'] / 1e6:.1f} MB")
    open(out_md, "w").write("\n".join(lines) + "\n")


def counters(counter_csv, out_md, cmd, cus=256, simds_per_cu=4, xcds=8):
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names, dur = {}, {}
    for r in csv.DictReader(open(counter_csv)):
        if not _ours(r["Kernel_Name"]):
            continue
        d = int(r["Dispatch_Id"])
        names[d] = _short(r["Kernel_Name"])
        dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
    by_kernel = collections.defaultdict(list)
    for d in sorted(per):
        by_kernel[names[d]].append(d)
    cols = sorted({k for c in per.values() for k in c})

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]

    lines = ["# Counters per dispatch: libpagedattn kernels", "", "Command:", "", "```", cmd, "```", "",
             f"Each figure is the median over a kernel's dispatches. GRBM_GUI_ACTIVE is reported summed over "
             f"the {xcds} XCDs, so the elapsed cycles of a dispatch are GRBM_GUI_ACTIVE / {xcds}; divided by "
             f"the dispatch's duration they give the shader clock it ran at (shown for dispatches of 50 us "
             f"or more: the counters' window is a few us longer than the dispatch).", "",
             f"Derived ({cus} CUs, {cus * simds_per_cu} SIMDs):", "",
             f"- MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcds} x SIMDs) x 100",
             f"- VALU busy % = SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE / {xcds} x CUs) x 100",
             "- bf16 MFMA GFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / 1e9 (masked products included)", "",
             "| kernel | dispatches | us | clock GHz | MFMA busy % | VALU busy % | bf16 MFMA GFLOP |",
             "|---|---|---|---|---|---|---|"]
    avg = {}
    for k, ds in sorted(by_kernel.items()):
        a = {c: med([per[d].get(c, 0.0) for d in ds]) for c in cols}
        avg[k] = a
        t = med([dur[d] for d in ds])
        cyc = a.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        nan = float("nan")
        mf, va = nan, nan
        if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in a:
            mf = 100 * a["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * cus * simds_per_cu)
        if cyc and "SQ_ACTIVE_INST_VALU" in a:
            va = 100 * a["SQ_ACTIVE_INST_VALU"] / (cyc * cus)
        fl = a.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", nan) * 512 / 1e9
        # the counters' window is a few us longer than the dispatch itself,
        # so the clock is only given for dispatches long enough to hide that
        ghz = f"{cyc / t / 1e9:.2f}" if t >= 50e-6 else "-"
        fmt = lambda x, d: "-" if x != x else f"{x:.{d}f}"  # a counter the pass did not take
        lines.append(f"| `{k}` | {len(ds)} | {t * 1e6:.1f} | {ghz} | {fmt(mf, 1)} | {fmt(va, 1)} | {fmt(fl, 2)} |")
    lines += ["", "Raw medians per dispatch:", "", "| kernel | " + " | ".join(cols) + " |",
              "|---|" + "---|" * len(cols)]
    for k, a in sorted(avg.items()):
        lines.append(f"| `{k}` | " + " | ".join(f"{a[c]:.4g}" for c in cols) + " |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out_md")
    t.add_argument("--cmd", required=True)
    t.add_argument("--kernel-trace", default=None, help="kernel-trace CSV of the same run")
    t.add_argument("--last", type=int, default=0, help="also average each kernel's last N dispatches")
    f = sub.add_parser("traffic")
    f.add_argument("fetch_csv")
    f.add_argument("write_csv")
    f.add_argument("out_json")
    f.add_argument("out_md")
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--cmd-fetch", required=True)
    f.add_argument("--cmd-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("counter_csv")
    c.add_argument("out_md")
    c.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.mode == "counters":
        counters(a.counter_csv, a.out_md, a.cmd)
    elif a.mode == "trace":
        trace(a.stats_csv, a.out_md, a.cmd, a.kernel_trace, a.last)
    else:
        traffic(a.fetch_csv, a.write_csv, a.out_json, a.out_md, a.copy_bytes, a.cmd_fetch, a.cmd_write)


if __name__ == "__main__":
    main()
