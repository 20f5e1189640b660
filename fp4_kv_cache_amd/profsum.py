"""Summaries of rocprofv3 output (CSV format) for the committed profiles.

  python -m fp4_kv_cache_amd.profsum kernels DIR [--match SUBSTR ...]
      Per (kernel, grid size) dispatch count and duration statistics from a
      `rocprofv3 --kernel-trace --output-format csv -d DIR ...` run.
  python -m fp4_kv_cache_amd.profsum traffic FETCH_DIR WRITE_DIR \\
          --kernel SUBSTR --grid N --alg-bytes N
      HBM bytes per dispatch of one kernel from two `--pmc FETCH_SIZE` /
      `--pmc WRITE_SIZE` runs, each scaled by what the same counter reads
      for the calibration copy (a float32 multiply-by-one over 64 Mi
      elements: 256 MiB read and 256 MiB written per dispatch).
"""
import argparse
import collections
import csv
import glob
import json
import os
import statistics
import sys

COPY_BYTES = 4 * (64 << 20)
COPY_KERNEL = "MulFunctor<float>"     # torch.mul(x, 1.0, out=y), float32
COPY_GRID = 64 << 20 >> 2            # 4 elements per thread


def _rows(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {d}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def _grid(r):
    if "Grid_Size" in r:
        return int(r["Grid_Size"])
    return (int(r.get("Grid_Size_X", 1)) * int(r.get("Grid_Size_Y", 1))
            * int(r.get("Grid_Size_Z", 1)))


def kernels(d, match):
    acc = collections.defaultdict(list)
    for r in _rows(d, "kernel_trace.csv"):
        name = r["Kernel_Name"]
        if match and not any(m in name for m in match):
            continue
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        acc[(name, _grid(r))].append(us)
    out = []
    for (name, grid), v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        out.append({"kernel": name, "grid_threads": grid, "dispatches": len(v),
                    "mean_us": statistics.fmean(v),
                    "median_us": statistics.median(v), "min_us": min(v),
                    "max_us": max(v)})
    return out


def _counter(d, counter, pred):
    per = collections.defaultdict(float)
    for r in _rows(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter or not pred(r):
            continue
        per[r.get("Dispatch_Id") or r.get("Correlation_Id")] += float(r["Counter_Value"])
    return list(per.values())


def traffic(fetch_dir, write_dir, kernel, grid, alg_bytes):
    is_k = lambda r: kernel in r["Kernel_Name"] and (grid is None or _grid(r) == grid)
    is_copy = lambda r: COPY_KERNEL in r["Kernel_Name"] and _grid(r) == COPY_GRID
    fk, wk = _counter(fetch_dir, "FETCH_SIZE", is_k), _counter(write_dir, "WRITE_SIZE", is_k)
    fc, wc = _counter(fetch_dir, "FETCH_SIZE", is_copy), _counter(write_dir, "WRITE_SIZE", is_copy)
    if not (fk and wk and fc and wc):
        sys.exit("missing dispatches for the kernel or the calibration copy")
    ff = COPY_BYTES / (statistics.fmean(fc) * 1024)
    wf = COPY_BYTES / (statistics.fmean(wc) * 1024)
    fetch = statistics.fmean(fk) * 1024 * ff
    write = statistics.fmean(wk) * 1024 * wf
    return {"kernel_match": kernel, "grid_threads": grid,
            "dispatches": [len(fk), len(wk)],
            "fetch_kib_per_dispatch": statistics.fmean(fk),
            "write_kib_per_dispatch": statistics.fmean(wk),
            "calibration_kib_per_dispatch": [statistics.fmean(fc), statistics.fmean(wc)],
            "fetch_factor": ff, "write_factor": wf,
            "hbm_bytes_per_launch": fetch + write,
            "algorithmic_bytes_per_launch": alg_bytes,
            "traffic_over_algorithmic": (fetch + write) / alg_bytes}


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("dir")
    k.add_argument("--match", nargs="*", default=[])
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--kernel", required=True)
    t.add_argument("--grid", type=int, default=None)
    t.add_argument("--alg-bytes", type=int, required=True)
    a = ap.parse_args()
    if a.cmd == "kernels":
        rows = kernels(a.dir, a.match)
        print("| kernel | grid threads | dispatches | mean us | median us | min us |")
        print("|---|---:|---:|---:|---:|---:|")
        for r in rows:
            print(f"| `{r['kernel'][:120]}` | {r['grid_threads']} | {r['dispatches']} "
                  f"| {r['mean_us']:.2f} | {r['median_us']:.2f} | {r['min_us']:.2f} |")
    else:
        print(json.dumps(traffic(a.fetch_dir, a.write_dir, a.kernel, a.grid,
                                 a.alg_bytes), indent=1))


if __name__ == "__main__":
    main()
