"""Summarise rocprofv3 CSV output of bench.py runs into a short markdown file.

Usage (after the rocprofv3 runs listed in the summary's header):
  python -m kv_cache_compression_04_amd.rocprof_summary --trace DIR \
      [--pmc DIR ...] [--copy-fetch DIR --copy-write DIR] --cmd "..." --out FILE

* --trace: a `rocprofv3 --kernel-trace --stats --output-format csv` directory;
  per-kernel launch counts and average durations of the library's kernels.
* --pmc: `rocprofv3 --pmc ... --output-format csv` directories; counter values
  averaged per (kernel, grid).
* --copy-fetch / --copy-write: FETCH_SIZE / WRITE_SIZE of `bench.py
  --copy-calibration` (a 512 MiB device copy), used to scale the byte counters
  to bytes ("traffic").
The summary records a hash of the kernel source so bench.py can tell whether
the counters still describe the current kernels.
"""
import argparse
import collections
import csv
import glob
import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "csrc", "tq_kernels.hip")
COPY_BYTES = 512 << 20


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")


def _rows(pattern):
    out = []
    for f in glob.glob(pattern, recursive=True):
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def trace_stats(d):
    acc = collections.defaultdict(list)
    for r in _rows(os.path.join(d, "**", "*kernel_trace.csv")):
        if "tq::" not in r["Kernel_Name"]:
            continue
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1))
        acc[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return acc


def pmc_stats(d, kernel_filter=None):
    acc = collections.defaultdict(list)
    for r in _rows(os.path.join(d, "**", "*counter_collection.csv")):
        name = r["Kernel_Name"]
        if kernel_filter and kernel_filter not in name:
            continue
        key = (_short(name), int(r.get("Grid_Size", 0) or 0), r["Counter_Name"])
        acc[key].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--pmc", nargs="*", default=[])
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--cmd", action="append", default=[])
    ap.add_argument("--title", default="rocprofv3 summary")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()

    lines = [f"# {a.title}", "", f"kernel source sha256[:16]: `{kernel_source_hash()}`", "",
             "Commands (run from /tmp with TMPDIR=/tmp, R = repository root):", ""]
    lines += [f"    {c}" for c in a.cmd]
    lines += ["", "## Kernel trace (durations in microseconds)", "",
              "| kernel | grid threads | launches | avg us | median us | min us | max us |",
              "|---|---|---|---|---|---|---|"]
    for (k, grid), v in sorted(trace_stats(a.trace).items()):
        med = sorted(v)[len(v) // 2]
        lines.append(f"| {k} | {grid} | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | {med / 1e3:.2f} | "
                     f"{min(v) / 1e3:.2f} | {max(v) / 1e3:.2f} |")

    scale_f = scale_w = None
    if a.copy_fetch and a.copy_write:
        f = pmc_stats(a.copy_fetch, "copyBuffer")
        w = pmc_stats(a.copy_write, "copyBuffer")
        fv = [v for (k, g, c), v in f.items() if c == "FETCH_SIZE"]
        wv = [v for (k, g, c), v in w.items() if c == "WRITE_SIZE"]
        if fv and wv:
            scale_f = COPY_BYTES / (max(fv) * 1024)
            scale_w = COPY_BYTES / (max(wv) * 1024)
            lines += ["", "## Byte-counter calibration", "",
                      f"A 512 MiB device copy reads FETCH_SIZE = {max(fv):.0f} KiB and writes WRITE_SIZE = "
                      f"{max(wv):.0f} KiB per launch: bytes = FETCH_SIZE x 1024 x {scale_f:.3f}, "
                      f"WRITE_SIZE x 1024 x {scale_w:.3f}."]

    merged = {}
    for d in a.pmc:
        merged.update(pmc_stats(d, "tq::"))
    if merged:
        by_kernel = collections.defaultdict(dict)
        for (k, g, c), v in merged.items():
            by_kernel[(k, g)][c] = v
        counters = sorted({c for (_, _, c) in merged})
        lines += ["", "## Counters (average per dispatch)", "",
                  "| kernel | grid | " + " | ".join(counters) + " |",
                  "|---|---|" + "---|" * len(counters)]
        for (k, g), cv in sorted(by_kernel.items()):
            lines.append(f"| {k} | {g} | " + " | ".join(f"{cv[c]:.4g}" if c in cv else "" for c in counters) + " |")
        if scale_f and scale_w:
            lines += ["", "## HBM traffic per launch (scaled byte counters)", ""]
            for (k, g), cv in sorted(by_kernel.items()):
                if "FETCH_SIZE" in cv and "WRITE_SIZE" in cv:
                    tb = cv["FETCH_SIZE"] * 1024 * scale_f + cv["WRITE_SIZE"] * 1024 * scale_w
                    lines.append(f"traffic_bytes_per_launch: {k} {g} {tb:.0f}")
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
