"""Summarize rocprofv3 CSV output into the short text kept under profiles/.

    python -m verify_pass_sv_amd.rocprof_summary \
        --trace out/prof_kt --pmc out/prof_pmc \
        --kernel pass_kernel --copy-bytes 268435456 \
        --command "<the rocprofv3 command lines>" --out profiles/<name>

Reads `*_kernel_stats.csv` (rocprofv3 --kernel-trace --stats) and every
`*_counter_collection.csv` under the PMC directory (one rocprofv3 --pmc run
per subdirectory), and writes <name>.md (tables) and <name>.json (the
numbers the benchmark reports: average duration of the kernel, FETCH_SIZE /
WRITE_SIZE per dispatch scaled by what the same counters read for the plain
copy kernel of known size, and the SHA-256 of the kernel's sources so a
stale figure is recognised).
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"
# Sources whose change makes recorded counters stale, per kernel family.
KERNEL_SOURCES = {
    "pass_kernel": ["csrc/pass.hip", "csrc/w4_packed_dev.h", "csrc/sv_common.h"],
    "chain_kernel": ["csrc/pass_chain.hip", "csrc/w4_packed_dev.h", "csrc/sv_common.h"],
    "stats_kernel": ["csrc/verify_accept.hip", "csrc/sv_common.h", "csrc/sv_philox.h"],
    "decide_kernel": ["csrc/verify_accept.hip", "csrc/sv_common.h", "csrc/sv_philox.h"],
    "sampled_rows_kernel": ["csrc/verify_sampled.hip", "csrc/sv_common.h", "csrc/sv_philox.h"],
}


def sources_sha256(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name, width=72):
    n = name.replace("(anonymous namespace)::", "")
    return n if len(n) <= width else n[: width - 3] + "..."


def read_stats(trace_dir):
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*_kernel_stats.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["TotalDurationNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda r: -r[3])
    return rows


def read_counters(pmc_dir, largest=()):
    """Per kernel name, each counter averaged over its dispatches; for the
    kernels named in `largest`, the largest reading instead (the copy kernel
    of known size shares its name with the runtime's small copies)."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for f in glob.glob(os.path.join(pmc_dir, "**", "*_counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: (max(v) if any(n in k for n in largest) else sum(v) / len(v))
                for c, v in d.items()} for k, d in agg.items()}


def pick(d, key):
    for name, val in d.items():
        if key in name:
            return name, val
    raise KeyError(f"no kernel matching {key!r}")


# Single-GEMM launches (bench.py --profile-single): each entry point runs 13
# rounds of 32 GEMMs, 8 layers of (qkv, o, gate|up, down) in that order.
SINGLE_SHAPES = [("qkv", 12288, 4096), ("o", 4096, 4096), ("gate/up", 24576, 4096),
                 ("down", 4096, 12288)]
SINGLE_MODES = {  # template flags (row-major, int8 activations, 8-bit weights)
    ("true", "false", "false"): ("sv_qgemm_w4", "w4"),
    ("false", "false", "false"): ("sv_qgemm_w4_packed", "w4"),
    ("true", "true", "false"): ("sv_qgemm_w4_i8", "w4"),
    ("true", "false", "true"): ("sv_qgemm_w8", "w8"),
}


def single_gemm_summary(trace_dir, title, command, out):
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*_kernel_trace.csv"), recursive=True):
        rows += [r for r in csv.DictReader(open(f)) if "qgemm_w4p_kernel<" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    fam = collections.defaultdict(list)
    for r in rows:
        flags = tuple(x.strip() for x in r["Kernel_Name"].split(">")[0].split(",")[-3:])
        fam[SINGLE_MODES[flags]].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# {title}", "", "Commands (run from the repository root with TMPDIR=/tmp):", "",
             "```", command, "```", "",
             "Per-dispatch durations from the kernel trace; each entry point's first 3 rounds "
             "(96 dispatches) are dropped, the other 10 averaged per matrix shape. Algorithmic "
             "bytes: codes plus scales and zero points (W4: N K / 2 + N K / 16), codes plus "
             "channel scales (W8: N K + 2 N).", "",
             "| entry point | matrix (N x K) | avg us | TB/s |", "|---|---|---:|---:|"]
    summary = {}
    for (name, fmt), d in fam.items():
        per = collections.defaultdict(list)
        for i, us in enumerate(d[96:]):
            per[i % 4].append(us)
        tot_us, tot_b = 0.0, 0
        for j, (sn, N, K) in enumerate(SINGLE_SHAPES):
            avg = sum(per[j]) / len(per[j])
            b = N * K // 2 + N * (K // 64) * 4 if fmt == "w4" else N * K + 2 * N
            tot_us += avg
            tot_b += b
            lines.append(f"| `{name}` | {sn} {N} x {K} | {avg:.2f} | {b / (avg * 1e-6) / 1e12:.2f} |")
        summary[name] = {"pass_of_128_ms": round(32 * tot_us / 1e3, 4),
                         "TBps": round(tot_b / (tot_us * 1e-6) / 1e12, 3)}
        lines.append(f"| `{name}` | 128 GEMMs of a pass, sum | {32 * tot_us:.1f} | "
                     f"{tot_b / (tot_us * 1e-6) / 1e12:.2f} |")
    open(out + ".md", "w").write("\n".join(lines) + "\n")
    json.dump(summary, open(out + ".json", "w"), indent=1)
    print(json.dumps(summary))


def main():
    import sys
    if "--single-gemm" in sys.argv:
        sp = argparse.ArgumentParser()
        sp.add_argument("--single-gemm", required=True, help="rocprofv3 --kernel-trace directory")
        sp.add_argument("--title", required=True)
        sp.add_argument("--command", required=True)
        sp.add_argument("--out", required=True)
        a = sp.parse_args()
        single_gemm_summary(a.single_gemm, a.title, a.command, a.out)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--pmc", required=True)
    ap.add_argument("--kernel", required=True, help="substring of the kernel of interest")
    ap.add_argument("--copy-bytes", type=int, required=True,
                    help="bytes read (and written) by the plain copy kernel in the run")
    ap.add_argument("--algo-bytes", type=float, required=True,
                    help="algorithmic bytes per dispatch of the kernel of interest")
    ap.add_argument("--command", required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--out", required=True, help="output path without extension")
    a = ap.parse_args()

    stats = read_stats(a.trace)
    kname, kstat = None, None
    for r in stats:
        if a.kernel in r[0]:
            kname, kstat = r[0], r
            break
    cnt = read_counters(a.pmc, largest=(COPY_KERNEL,))
    kc_name, kc = pick(cnt, a.kernel)
    _, cc = pick(cnt, COPY_KERNEL)
    copy_kib = a.copy_bytes / 1024.0
    f_fetch = copy_kib / cc["FETCH_SIZE"]
    f_write = copy_kib / cc["WRITE_SIZE"]
    fetch_b = kc["FETCH_SIZE"] * f_fetch * 1024
    write_b = kc["WRITE_SIZE"] * f_write * 1024
    avg_us = kstat[2]
    out = {
        "kernel": short_name(kname, 200),
        "sources_sha256": sources_sha256(a.kernel.split("<")[0]),
        "avg_duration_us": round(avg_us, 3),
        "calls": kstat[1],
        "algorithmic_bytes": a.algo_bytes,
        "achieved_GBps_rocprof": round(a.algo_bytes / (avg_us * 1e-6) / 1e9, 1),
        "fetch_size_kib_per_dispatch": round(kc["FETCH_SIZE"], 1),
        "write_size_kib_per_dispatch": round(kc["WRITE_SIZE"], 1),
        "copy_kernel_bytes": a.copy_bytes,
        "copy_fetch_scale": round(f_fetch, 4),
        "copy_write_scale": round(f_write, 4),
        "traffic_bytes": round(fetch_b + write_b),
        "traffic_read_bytes": round(fetch_b),
        "traffic_write_bytes": round(write_b),
        "counters": {k: round(v, 1) for k, v in sorted(kc.items())},
    }
    with open(a.out + ".json", "w") as f:
        json.dump(out, f, indent=1)
    L = [f"# {a.title}", "", "Commands (run from the repository root with TMPDIR=/tmp; one PMC pass per run):", "",
         "```", a.command.strip(), "```", "",
         "## Kernel trace (rocprofv3 --kernel-trace --stats), top kernels", "",
         "| kernel | calls | avg us | total us | % |", "|---|---:|---:|---:|---:|"]
    for r in stats[:12]:
        L.append(f"| `{short_name(r[0])}` | {r[1]} | {r[2]:.2f} | {r[3]:.1f} | {r[4]:.2f} |")
    L += ["", f"## `{short_name(kname)}`", "",
          f"- average duration: **{avg_us:.1f} us** over {kstat[1]} dispatches",
          f"- algorithmic bytes per dispatch: {a.algo_bytes:.4g} -> "
          f"{out['achieved_GBps_rocprof']} GB/s",
          f"- FETCH_SIZE {kc['FETCH_SIZE']:.0f} KiB x {f_fetch:.4f} (copy-kernel scale: "
          f"{a.copy_bytes} B copy read as {cc['FETCH_SIZE']:.0f} KiB) = {fetch_b:.4g} B",
          f"- WRITE_SIZE {kc['WRITE_SIZE']:.0f} KiB x {f_write:.4f} (copy wrote "
          f"{cc['WRITE_SIZE']:.0f} KiB) = {write_b:.4g} B",
          f"- HBM traffic per dispatch: **{fetch_b + write_b:.4g} B** "
          f"({(fetch_b + write_b) / a.algo_bytes:.3f} x algorithmic)",
          f"- sources SHA-256: `{out['sources_sha256']}`", "",
          "| counter | per dispatch |", "|---|---:|"]
    for c, v in sorted(kc.items()):
        L.append(f"| {c} | {v:.4g} |")
    with open(a.out + ".md", "w") as f:
        f.write("\n".join(L) + "\n")
    print(json.dumps({k: out[k] for k in ("avg_duration_us", "traffic_bytes",
                                          "achieved_GBps_rocprof")}))


if __name__ == "__main__":
    main()
