"""Short text summaries of rocprofv3 runs of the layer step, for profiles/.

  python3 -m verify_step_amd.profsum stats  STATS_CSV  --workload W --cmd "..." --out FILE
  python3 -m verify_step_amd.profsum traffic --kernel K --workload W \
      --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV --cmds "..." --out FILE
  python3 -m verify_step_amd.profsum util CSV --workload W --cmd "..." --out FILE

`stats` reads the kernel_stats CSV of a `rocprofv3 --kernel-trace --stats
--output-format csv` run and tabulates the library's kernels.  `traffic`
reads the counter_collection CSVs of four `--pmc` runs (FETCH_SIZE and
WRITE_SIZE over the benchmark, and over `bench.py --calibrate-copy`, a 1 GiB
device copy) and converts the kernel's mean KiB per dispatch into bytes
with the factor that makes the copy's readings equal its known size.  The
traffic summary carries the SHA-256 of the kernel sources it was taken
with; bench.py reports its figure only while the sources still match.
`util` reads the counter_collection CSV of a `--pmc MfmaUtil VALUBusy` run
(rocprofv3's derived metrics: the matrix-core busy cycles per SIMD, and the
cycles with a vector ALU instruction in flight per CU, both as a percentage
of the GPU's busy cycles over each dispatch) and tabulates their mean per
kernel.
"""
import argparse
import csv
import hashlib
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def sources_digest():
    """SHA-256 over the kernel sources (file names and contents)."""
    d = os.path.join(ROOT, "verify_step_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def short_name(name):
    """`void msk::k_attn<2, 128>(msk::LayerArgs, ...)` -> `k_attn<2, 128>`."""
    m = re.search(r"msk::(k_\w+(?:<[^>]*>)?)", name)
    return m.group(1) if m else name.split("(")[0][:60]


def read_stats(path):
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append(dict(name=r["Name"], calls=int(r["Calls"]), total_ns=float(r["TotalDurationNs"]),
                         avg_ns=float(r["AverageNs"]), min_ns=float(r["MinNs"]),
                         max_ns=float(r["MaxNs"]), pct=float(r["Percentage"])))
    return rows


def stats_md(rows, workload, cmd):
    mine = [r for r in rows if "msk::" in r["name"]]
    other = [r for r in rows if "msk::" not in r["name"]]
    out = [f"# Kernel times: {workload}", "",
           "Produced by (from the repository root, on one MI355X):", "",
           "```", cmd, "```", "",
           "| kernel | calls | avg µs | min µs | max µs | total µs |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(mine, key=lambda r: -r["total_ns"]):
        out.append(f"| `{short_name(r['name'])}` | {r['calls']} | {r['avg_ns'] / 1e3:.2f} | "
                   f"{r['min_ns'] / 1e3:.2f} | {r['max_ns'] / 1e3:.2f} | "
                   f"{r['total_ns'] / 1e3:.1f} |")
    tot = sum(r["total_ns"] for r in other)
    out += ["", f"Other kernels in the run (input generation and copies outside the timed "
                f"steps): {len(other)} kinds, {tot / 1e3:.1f} µs in total.", ""]
    return "\n".join(out)


def read_counter(path, counter):
    """{kernel name: [per-dispatch values]} of one counter."""
    d = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return d


def kernel_mean(d, kernel):
    vals = [v for n, vs in d.items() if short_name(n).split("<")[0] == kernel for v in vs]
    if not vals:
        raise SystemExit(f"no dispatch of {kernel} in the counter file")
    return sum(vals) / len(vals), len(vals)


def traffic_md(kernel, workload, fetch, write, cfetch, cwrite, cmds):
    f_kib, nf = kernel_mean(read_counter(fetch, "FETCH_SIZE"), kernel)
    w_kib, nw = kernel_mean(read_counter(write, "WRITE_SIZE"), kernel)
    cf = read_counter(cfetch, "FETCH_SIZE")[COPY_KERNEL]
    cw = read_counter(cwrite, "WRITE_SIZE")[COPY_KERNEL]
    cf_kib, cw_kib = sum(cf) / len(cf), sum(cw) / len(cw)
    f_scale = COPY_BYTES / cf_kib        # bytes per KiB reading
    w_scale = COPY_BYTES / cw_kib
    fb, wb = f_kib * f_scale, w_kib * w_scale
    out = [f"# HBM traffic of `{kernel}`: {workload}", "",
           "Four `rocprofv3 --pmc` runs, one counter each (from the repository root, on one "
           "MI355X):", "", "```", cmds, "```", "",
           f"The copy kernel `{COPY_KERNEL}` moves {COPY_BYTES} bytes each way per dispatch; "
           "its mean readings give the scale from the counters' KiB to bytes.", "",
           "| counter | kernel mean KiB/dispatch (dispatches) | copy mean KiB/dispatch | "
           "bytes per KiB | kernel bytes/dispatch |", "|---|---:|---:|---:|---:|",
           f"| FETCH_SIZE | {f_kib:.1f} ({nf}) | {cf_kib:.1f} | {f_scale:.2f} | {fb:.0f} |",
           f"| WRITE_SIZE | {w_kib:.1f} ({nw}) | {cw_kib:.1f} | {w_scale:.2f} | {wb:.0f} |", "",
           "Machine-read by bench.py:", "",
           f"- kernel: `{kernel}`",
           f"- workload: `{workload}`",
           f"- sources_sha256: `{sources_digest()}`",
           f"- fetch_bytes_per_launch: {fb:.0f}",
           f"- write_bytes_per_launch: {wb:.0f}", ""]
    return "\n".join(out)


def util_md(path, workload, cmd):
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] not in ("MfmaUtil", "VALUBusy"):
            continue
        if "msk::" not in r["Kernel_Name"]:
            continue
        k = short_name(r["Kernel_Name"])
        vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = [f"# Matrix-core and vector-ALU utilisation: {workload}", "",
           "One `rocprofv3 --pmc` run of the benchmark (from the repository root, on one "
           "MI355X):", "", "```", cmd, "```", "",
           "MfmaUtil: matrix-core busy cycles over all SIMDs / (GPU busy cycles x SIMDs), %.  "
           "VALUBusy: cycles with a vector-ALU instruction in flight per CU / GPU busy "
           "cycles, %.  Means over the dispatches of each kernel.", "",
           "| kernel | dispatches | MfmaUtil % | VALUBusy % |", "|---|---:|---:|---:|"]
    def mean(v):
        return sum(v) / len(v) if v else float("nan")
    for k in sorted(vals, key=lambda k: -mean(vals[k].get("VALUBusy", [0]))):
        m, v = vals[k].get("MfmaUtil", []), vals[k].get("VALUBusy", [])
        out.append(f"| `{k}` | {max(len(m), len(v))} | {mean(m):.1f} | {mean(v):.1f} |")
    out.append("")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--workload", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for a in ("--kernel", "--workload", "--fetch", "--write", "--copy-fetch", "--copy-write",
              "--cmds", "--out"):
        t.add_argument(a, required=True)
    u = sub.add_parser("util")
    u.add_argument("csv")
    u.add_argument("--workload", required=True)
    u.add_argument("--cmd", required=True)
    u.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.what == "util":
        text = util_md(a.csv, a.workload, a.cmd)
    elif a.what == "stats":
        text = stats_md(read_stats(a.csv), a.workload, a.cmd)
    else:
        text = traffic_md(a.kernel, a.workload, a.fetch, a.write, a.copy_fetch, a.copy_write,
                          a.cmds)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    sys.exit(main())
