"""Summaries of rocprofv3 runs of bench.py (text for the profiles folder).

Usage (from the repository root, after the rocprofv3 runs named in each
summary's header):

    python -m tree_indexed_sparse_zha_amd.profiling stats   <stats dir>   > summary.md
    python -m tree_indexed_sparse_zha_amd.profiling traffic <fetch dir> <write dir> <copy fetch dir> <copy write dir> \
        [--json traffic.json] > summary.md
    python -m tree_indexed_sparse_zha_amd.profiling counters <pmc dir> > summary.md

Each <dir> holds the CSV files of one `rocprofv3 ... --output-format csv -d <dir> -o run` run.

Dispatches of the routing kernels are named by level from their order: one
route call launches, from the top level down, a score kernel then a select
kernel per level, so the n-th score dispatch of a call is level
levels - n + 1.  The FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch)
are scaled by what they read for a plain copy of known size (the stream
probe's copy kernel: n bytes read and n written per dispatch).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import OrderedDict, defaultdict
from typing import Dict, List

HERE = os.path.dirname(os.path.abspath(__file__))


def _csv(path_glob: str) -> List[dict]:
    paths = sorted(glob.glob(path_glob, recursive=True))
    if not paths:
        raise FileNotFoundError(path_glob)
    rows: List[dict] = []
    for p in paths:
        with open(p, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def short_name(name: str) -> str:
    """`void zha::(anonymous namespace)::k_x<...>(args)` -> `k_x<...>`."""
    m = re.search(r"(k_[A-Za-z0-9_]+(<[^()]*>)?)\(", name)
    return m.group(1) if m else name


def is_library(name: str) -> bool:
    return "zha::" in name


def route_roles(dispatches: List[dict], levels: int) -> List[str]:
    """A role per dispatch (score_L<l>, select_L<l>, attend, combine, dense,
    build, probe, other), from kernel names and launch order."""
    roles = []
    level = None
    for d in dispatches:
        k = short_name(d["Kernel_Name"])
        if not is_library(d["Kernel_Name"]):
            roles.append("other")
            continue
        if k.startswith(("k_score_bf16", "k_score_leafw", "k_score_mask1", "k_score_smallr", "k_score_generic")):
            level = levels if (level is None or level <= 1) else level - 1
            roles.append(f"score_L{level}")
        elif k.startswith("k_select"):
            roles.append(f"select_L{level}" if level else "select")
        elif k.startswith("k_attend_cached"):
            roles.append("attend")
        elif k.startswith(("k_attend_mfma", "k_attend_pv16", "k_attend<")):
            roles.append("dense")
        elif k.startswith("k_combine"):
            roles.append("combine")
        elif k.startswith("k_build"):
            roles.append("build")
            level = None
        elif k.startswith("k_probe"):
            roles.append("probe")
        else:
            roles.append("other")
        if k.startswith("k_select") and level == 1:
            level = None
    return roles


def cmd_stats(args):
    rows = _csv(os.path.join(args.dir, "**", "*kernel_stats.csv"))
    lib = [r for r in rows if is_library(r["Name"])]
    lib.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("| kernel | calls | average ms | min ms | max ms | total ms |")
    print("|---|---|---|---|---|---|")
    for r in lib:
        print(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
              f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | {float(r['TotalDurationNs']) / 1e6:.3f} |")


def _counter_dispatches(d: str, counter: str) -> List[dict]:
    rows = [r for r in _csv(os.path.join(d, "**", "*counter_collection.csv")) if r["Counter_Name"] == counter]
    # one row per dispatch (a counter summed over its instances)
    by: Dict[int, dict] = OrderedDict()
    for r in rows:
        i = int(r["Dispatch_Id"])
        if i not in by:
            by[i] = dict(r)
            by[i]["value"] = 0.0
        by[i]["value"] += float(r["Counter_Value"])
    return [by[i] for i in sorted(by)]


def _copy_scale(d: str, counter: str, n_bytes: int) -> float:
    rows = [r for r in _counter_dispatches(d, counter) if "k_probe_copy" in r["Kernel_Name"]]
    if not rows:
        raise RuntimeError(f"no k_probe_copy dispatch in {d}")
    kib = sum(r["value"] for r in rows) / len(rows)
    return (n_bytes / 1024.0) / kib


def _source_hashes() -> Dict[str, str]:
    out = {}
    for src in ("zha_route.hip", "zha_attend.hip", "zha_build.hip", "zha_device.h", "zha_internal.h"):
        with open(os.path.join(HERE, "csrc", src), "rb") as f:
            out[src] = hashlib.sha256(f.read()).hexdigest()[:16]
    return out


SOURCE_OF = {"score": "zha_route.hip", "select": "zha_route.hip", "attend": "zha_attend.hip",
             "combine": "zha_attend.hip", "dense": "zha_attend.hip", "build": "zha_build.hip"}


def cmd_traffic(args):
    fs = _counter_dispatches(args.fetch, "FETCH_SIZE")
    ws = _counter_dispatches(args.write, "WRITE_SIZE")
    sf = _copy_scale(args.copy_fetch, "FETCH_SIZE", args.copy_bytes)
    sw = _copy_scale(args.copy_write, "WRITE_SIZE", args.copy_bytes)
    lib_f = [r for r in fs if is_library(r["Kernel_Name"])]
    lib_w = [r for r in ws if is_library(r["Kernel_Name"])]
    if len(lib_f) != len(lib_w):
        raise RuntimeError("the two runs launched different kernel sequences")
    roles = route_roles(lib_f, args.levels)
    agg = defaultdict(lambda: {"n": 0, "f": 0.0, "w": 0.0, "names": set()})
    for r, w, role in zip(lib_f, lib_w, roles):
        key = role
        if role == "build":  # split the full builds from the appends (the sub-span and merge passes)
            g = int(r["Grid_Size"])
            key = "build_full" if g >= args.full_build_threads else "append"
        a = agg[key]
        a["n"] += 1
        a["f"] += r["value"]
        a["w"] += w["value"]
        a["names"].add(short_name(r["Kernel_Name"]))
    print(f"Calibration: the stream probe's copy of {args.copy_bytes:,} bytes per dispatch reads FETCH_SIZE = "
          f"{args.copy_bytes / 1024 / sf:,.0f} KiB and WRITE_SIZE = {args.copy_bytes / 1024 / sw:,.0f} KiB, "
          f"so FETCH_SIZE is scaled by {sf:.3f} and WRITE_SIZE by {sw:.3f}.")
    print()
    print("| role | kernel(s) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes per dispatch |")
    print("|---|---|---|---|---|---|")
    rec = {"note": ("HBM bytes per dispatch (FETCH_SIZE x %.3f + WRITE_SIZE x %.3f, KiB -> bytes); valid only while "
                    "the kernel source and the shared device headers hash to these values" % (sf, sw)),
           "leaf_form": args.leaf_form, "sources": _source_hashes(), "kernels": {}}
    order = sorted(agg, key=lambda k: -(agg[k]["f"] * sf + agg[k]["w"] * sw) / agg[k]["n"])
    for key in order:
        a = agg[key]
        f, w = a["f"] / a["n"], a["w"] / a["n"]
        b = (f * sf + w * sw) * 1024
        names = ", ".join(f"`{n}`" for n in sorted(a["names"]))
        print(f"| {key} | {names} | {a['n']} | {f:,.0f} | {w:,.0f} | {b / 1e9:.3f} GB |")
        base = key.split("_")[0]
        if base in SOURCE_OF:
            rec["kernels"][key] = {"bytes": b, "source": SOURCE_OF[base]}
    if args.json:
        with open(args.json, "w") as fo:
            json.dump(rec, fo, indent=1)
            fo.write("\n")


def cmd_counters(args):
    rows = [r for r in _csv(os.path.join(args.dir, "**", "*counter_collection.csv")) if is_library(r["Kernel_Name"])]
    per = defaultdict(lambda: defaultdict(float))
    meta = {}
    for r in rows:
        key = (r["Dispatch_Id"], short_name(r["Kernel_Name"]))
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        meta[key] = r
    # the largest dispatch (the full build)
    key = max(per, key=lambda k: int(meta[k]["Grid_Size"]))
    c = per[key]
    m = meta[key]
    print(f"Dispatch {key[0]} `{key[1]}`: grid {int(m['Grid_Size']):,} threads, {m['VGPR_Count']} VGPRs "
          f"(+{m['Accum_VGPR_Count']} AGPRs), LDS {m['LDS_Block_Size']} bytes, scratch {m['Scratch_Size']} bytes.")
    print()
    blocks = args.blocks
    print(f"| counter | value | per 16-key block ({blocks:,} blocks) |")
    print("|---|---|---|")
    for name in sorted(c):
        v = c[name]
        per_blk = f"{v / blocks:,.1f}" if not name.startswith(("GRBM", "SQ_WAVES")) else ""
        print(f"| {name} | {v:,.0f} | {per_blk} |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c:
        xcd = c["GRBM_GUI_ACTIVE"] / args.xcds
        util = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd * args.simds)
        print()
        print(f"MFMA utilisation SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x {args.simds} SIMDs): "
              f"{100 * util:.1f}%; GRBM_GUI_ACTIVE per XCD {xcd:,.0f} cycles ({xcd / 2.4e6:.2f} ms at 2.4 GHz).")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("fetch")
    t.add_argument("write")
    t.add_argument("copy_fetch")
    t.add_argument("copy_write")
    t.add_argument("--copy-bytes", type=int, default=8 << 30)
    t.add_argument("--levels", type=int, default=6)
    t.add_argument("--leaf-form", default="weights2")
    t.add_argument("--full-build-threads", type=int, default=1 << 22)
    t.add_argument("--json", default=None)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--blocks", type=int, default=64 * (1 << 20) // 16)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--simds", type=int, default=1024)
    args = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.cmd](args)


if __name__ == "__main__":
    main()
