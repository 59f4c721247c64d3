"""Summaries of rocprofv3 output for this library's kernels.

    # kernel durations (rocprofv3 --kernel-trace --stats --output-format csv)
    python -m video_diffusion_transformer_block_amd.profiling stats <dir>/<name>_kernel_stats.csv

    # per-dispatch durations by kernel and grid (same run, kernel_trace.csv)
    python -m video_diffusion_transformer_block_amd.profiling trace <dir>/<name>_kernel_trace.csv

    # MFMA utilisation and clock of the GEMM kernels from one counter run
    # (--pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU)
    python -m video_diffusion_transformer_block_amd.profiling mfma <dir>/<name>_counter_collection.csv

    # HBM traffic per dispatch from two counter runs (FETCH_SIZE, WRITE_SIZE),
    # calibrated on the plain copy of known size that the run also performs
    python -m video_diffusion_transformer_block_amd.profiling traffic \
        <fetch>_counter_collection.csv <write>_counter_collection.csv \
        --copy-bytes 536870912 --copy-kernel neg_kernel --out profiles/traffic_5b.json

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  The scale factor
of each is the copy's known byte count divided by what the counter reads for
that copy.  The traffic file records a hash of the kernel sources it was
measured on; consumers treat it as stale once the sources change.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# every device source a profiled kernel is built from (the kernels and the
# headers they include): counters taken before a change to any of them no
# longer describe the kernels
KERNEL_SOURCES = ["csrc/qgemm.hip", "csrc/qgemm_mx.hip", "csrc/qgemm_w4a16.hip", "csrc/hadamard_quantize.hip",
                  "csrc/block_stats.hip", "csrc/bench_stream.hip", "csrc/qgemm_common.h", "csrc/hadamard_common.h",
                  "csrc/device_common.h", "csrc/lds_dma.h", "csrc/launch.h"]


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """Kernel name without return type, namespace and argument list; a
    hipBLASLt (Tensile) kernel is named by its layout and macro tile."""
    n = name.replace("void ", "").replace("vdtq::", "").replace("(anonymous namespace)::", "")
    n = n.split("(")[0]
    if n.startswith("Cijk_"):
        tile = next((f for f in n.split("_") if f.startswith("MT")), "")
        n = f"hipBLASLt {n.split('_')[1]} {tile}".rstrip()
    return n


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| {} | {} | {:.3f} | {:.1f} | {:.1f} | {:.1f} | {:.2f} |".format(
            short_name(r["Name"]), r["Calls"], float(r["TotalDurationNs"]) / 1e6,
            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["Percentage"])))
    return "\n".join(out)


def trace_table(path: str) -> str:
    """Median / min / mean duration per (kernel, grid) from a kernel trace."""
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        n = short_name(r["Kernel_Name"])
        if "FillFunctor" in n or "copyBuffer" in n or n.startswith("at::"):
            continue
        per[(n, int(r["Grid_Size_X"]))].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | grid (work-items) | dispatches | median us | min us | mean us |", "|---|---|---|---|---|---|"]
    for (n, g), v in sorted(per.items()):
        v = sorted(v)
        out.append(f"| {n} | {g} | {len(v)} | {v[len(v) // 2]:.1f} | {v[0]:.1f} | {sum(v) / len(v):.1f} |")
    return "\n".join(out)


def mfma_table(path: str, simds: int = 1024, xcds: int = 8) -> str:
    """Per (kernel, grid): MFMA busy share = SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE per XCD x SIMDs), the shader clock = GRBM_GUI_ACTIVE per
    XCD / duration, and non-MFMA VALU instructions per MFMA."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        n = short_name(r["Kernel_Name"])
        if not (n.startswith("qgemm_pipe") or n.startswith("qgemm_mx") or n.startswith("qgemm_a16")):
            continue
        k = (n, int(r["Grid_Size"]))
        per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[k][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = ["| kernel | grid (work-items) | dispatches | duration us | clock GHz | MFMA busy % | VALU / MFMA |",
           "|---|---|---|---|---|---|---|"]
    for k, c in sorted(per.items()):
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in c or "GRBM_GUI_ACTIVE" not in c:
            continue
        g = _mean(c["GRBM_GUI_ACTIVE"]) / xcds
        busy = _mean(c["SQ_VALU_MFMA_BUSY_CYCLES"])
        ds = sorted(dur[k].values())
        d = ds[len(ds) // 2] / 1e9
        vpm = ""
        if c.get("SQ_INSTS_MFMA") and c.get("SQ_INSTS_VALU"):
            mf = _mean(c["SQ_INSTS_MFMA"])
            vpm = f"{(_mean(c['SQ_INSTS_VALU']) - mf) / mf:.2f}" if mf else ""
        out.append(f"| {k[0]} | {k[1]} | {len(dur[k])} | {d * 1e6:.0f} | {g / d / 1e9:.2f} | "
                   f"{100 * busy / (g * simds):.1f} | {vpm} |")
    return "\n".join(out)


def l2_table(path: str) -> str:
    """Per (kernel, grid): L2 (TCC) hits and misses per dispatch, summed over
    the channels, and the hit rate = hits / (hits + misses)."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        n = short_name(r["Kernel_Name"])
        if "FillFunctor" in n or "copyBuffer" in n or n.startswith("at::"):
            continue
        per[(n, int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = ["| kernel | grid (work-items) | dispatches | L2 hits (M) | L2 misses (M) | hit rate % |",
           "|---|---|---|---|---|---|"]
    for k, c in sorted(per.items()):
        hits = c.get("TCC_HIT_sum") or c.get("TCC_HIT")
        miss = c.get("TCC_MISS_sum") or c.get("TCC_MISS")
        if not hits or not miss:
            continue
        h, m = _mean(hits), _mean(miss)
        rate = 100.0 * h / (h + m) if h + m else 0.0
        out.append(f"| {k[0]} | {k[1]} | {len(hits)} | {h / 1e6:.2f} | {m / 1e6:.2f} | {rate:.1f} |")
    return "\n".join(out)


def _counter_values(path: str, counter: str):
    """Counter values (KiB) per dispatch, keyed by (kernel name, grid size in
    work-items)."""
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[(short_name(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return per


def _mean(v):
    return sum(v) / len(v) if v else 0.0


def _by_kernel(per):
    out = collections.defaultdict(list)
    for (k, _), v in per.items():
        out[k].extend(v)
    return {k: _mean(v) for k, v in out.items()}


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int, copy_kernel: str = "neg_kernel"):
    """copy_kernel: substring naming the reference dispatch (an ordinary
    elementwise kernel reading and writing copy_bytes each)."""
    fg = _counter_values(fetch_csv, "FETCH_SIZE")
    wg = _counter_values(write_csv, "WRITE_SIZE")
    f, w = _by_kernel(fg), _by_kernel(wg)
    ref = [k for k in f if copy_kernel in k and k in w]
    if len(ref) != 1:
        raise SystemExit(f"expected one {copy_kernel} dispatch kind in the counter files, found {ref}")
    fs = copy_bytes / (f[ref[0]] * 1024.0)
    ws = copy_bytes / (w[ref[0]] * 1024.0)
    kernels = {}
    for k in sorted(set(f) | set(w)):
        fb = f.get(k, 0.0) * 1024.0 * fs
        wb = w.get(k, 0.0) * 1024.0 * ws
        grids = {}
        for g in sorted({g for (n, g) in list(fg) + list(wg) if n == k}):
            gf = _mean(fg.get((k, g), [])) * 1024.0 * fs
            gw = _mean(wg.get((k, g), [])) * 1024.0 * ws
            grids[str(g)] = {"fetch_bytes": gf, "write_bytes": gw, "bytes": gf + gw,
                             "dispatches": len(fg.get((k, g), []))}
        kernels[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes": fb + wb,
                      "fetch_kib_raw": f.get(k, 0.0), "write_kib_raw": w.get(k, 0.0), "grids": grids}
    return {"source_hash": source_hash(), "fetch_scale": fs, "write_scale": ws,
            "copy_bytes": copy_bytes, "copy_kernel": ref[0], "kernels": kernels}


def traffic_table(rec) -> str:
    out = [f"fetch scale {rec['fetch_scale']:.4f}, write scale {rec['write_scale']:.4f} "
           f"(reference: {rec['copy_kernel']}, {rec['copy_bytes']} bytes read and written)", "",
           "| kernel | grid (work-items) | dispatches | fetch MiB | write MiB |", "|---|---|---|---|---|"]
    for k, v in rec["kernels"].items():
        if "FillFunctor" in k or "copyBuffer" in k:
            continue
        for g, e in v["grids"].items():
            out.append(f"| {k} | {g} | {e['dispatches']} | {e['fetch_bytes'] / 2**20:.1f} | "
                       f"{e['write_bytes'] / 2**20:.1f} |")
    return "\n".join(out)


def load_traffic(path: str):
    """The traffic record if it was measured on the current kernel sources."""
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    return rec if rec.get("source_hash") == source_hash() else None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    t = sub.add_parser("trace")
    t.add_argument("csv")
    mf = sub.add_parser("mfma")
    mf.add_argument("csv")
    l2 = sub.add_parser("l2")
    l2.add_argument("csv")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--copy-kernel", default="neg_kernel")
    b.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats_table(args.csv))
    elif args.cmd == "trace":
        print(trace_table(args.csv))
    elif args.cmd == "mfma":
        print(mfma_table(args.csv))
    elif args.cmd == "l2":
        print(l2_table(args.csv))
    else:
        rec = traffic(args.fetch_csv, args.write_csv, args.copy_bytes, args.copy_kernel)
        with open(args.out, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(traffic_table(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
