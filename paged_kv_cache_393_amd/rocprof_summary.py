"""Condense rocprofv3 CSV output into the short summaries kept under profiles/.

    # kernel durations (rocprofv3 --kernel-trace --stats --output-format csv)
    python -m paged_kv_cache_393_amd.rocprof_summary stats OUTDIR --out FILE --command "..."

    # HBM traffic per call of an operation (decode, or the KV write) from two
    # counter runs (FETCH_SIZE, then WRITE_SIZE) of a bench run that also
    # copied --copy-bytes bytes with the probe copy kernel, whose counter
    # readings calibrate those of the operation's kernels
    python -m paged_kv_cache_393_amd.rocprof_summary traffic --fetch DIR1 --write DIR2 \\
        --copy-bytes N --workload NAME --operation decode|write --out FILE \\
        --command "..." --command "..."

Only reads the CSV files rocprofv3 wrote; nothing here touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(_HERE, "csrc", "paged_attn.hip")
WRITE_SOURCE = os.path.join(_HERE, "csrc", "kv_write.hip")
EVICT_SOURCE = os.path.join(_HERE, "csrc", "kv_evict.hip")
PREFILL_SOURCE = os.path.join(_HERE, "csrc", "paged_prefill.hip")
COMPRESS_SOURCE = os.path.join(_HERE, "csrc", "kv_compress.hip")
KERNELS = ("pa_prefill_merge_kernel", "pa_decode_kernel", "pa_merge_kernel", "kv_write_kernel", "token_scores_kernel",
           "evict_lowest_block_kernel", "pa_prefill_kernel", "probe_copy_kernel",
           "probe_read_kernel", "compress_select_kernel", "compress_move_kernel",
           "compress_split_keys_kernel", "compress_split_pass_kernel", "compress_split_write_kernel",
           "compress_move_far_kernel")
# The kernels of each timed operation and the source files they are built from.
OPERATIONS = {
    "decode": (("pa_decode_kernel", "pa_merge_kernel"), (KERNEL_SOURCE,)),
    "write": (("kv_write_kernel",), (WRITE_SOURCE,)),
    "scores": (("token_scores_kernel",), (EVICT_SOURCE,)),
    "prefill": (("pa_prefill_kernel", "pa_prefill_merge_kernel"), (PREFILL_SOURCE,)),
    # a serving batch: the chunk's key-split prefill call and the decodes' call
    "serving": (("pa_prefill_kernel_split", "pa_prefill_merge_kernel", "pa_decode_kernel",
                 "pa_merge_kernel"), (PREFILL_SOURCE, KERNEL_SOURCE)),
    "compress": (("compress_select_kernel", "compress_split_keys_kernel", "compress_split_pass_kernel",
                  "compress_split_write_kernel", "compress_move_kernel", "compress_move_far_kernel"),
                 (COMPRESS_SOURCE,)),
}


def source_sha256(path: str = KERNEL_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short_name(name: str) -> str:
    # the key-split form of the prefill kernel (its last template argument true)
    if re.search(r"pa_prefill_kernel<[^>]*\btrue>", name):
        return "pa_prefill_kernel_split"
    for k in KERNELS:
        if k in name:
            return k
    return name.split("(")[0][-60:]


def _find(outdir: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(outdir, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {outdir}")
    return hits[0]


def kernel_stats(outdir: str) -> list:
    rows = []
    with open(_find(outdir, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append({"kernel": r["Name"], "calls": int(r["Calls"]),
                         "total_ns": float(r["TotalDurationNs"]), "avg_ns": float(r["AverageNs"]),
                         "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                         "pct": float(r["Percentage"])})
    return rows


def counter_means(outdir: str) -> dict:
    """{short kernel name: {counter: mean per-dispatch value}}"""
    vals: dict = {}
    with open(_find(outdir, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            k = short_name(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: statistics.fmean(v) for c, v in d.items()} for k, d in vals.items()}


def cmd_stats(a) -> int:
    rows = kernel_stats(a.outdir)
    lines = [f"# rocprofv3 kernel trace summary ({a.title})", "", "command:", f"  {a.command}", "",
             f"{'kernel':<28} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in rows:
        lines.append(f"{short_name(r['kernel']):<28} {r['calls']:>6} {r['avg_ns'] / 1e3:>9.2f} "
                     f"{r['min_ns'] / 1e3:>9.2f} {r['max_ns'] / 1e3:>9.2f} {r['pct']:>6.2f}")
    kernels, srcs = OPERATIONS[a.operation]
    lines += [""] + [f"{os.path.basename(src)} sha256: {source_sha256(src)}" for src in srcs]
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)
    return 0


def cmd_traffic(a) -> int:
    fetch = counter_means(a.fetch)
    write = counter_means(a.write)
    copy_f = fetch["probe_copy_kernel"]["FETCH_SIZE"]
    copy_w = write["probe_copy_kernel"]["WRITE_SIZE"]
    sf = a.copy_bytes / (copy_f * 1024.0)    # true bytes per counted byte
    sw = a.copy_bytes / (copy_w * 1024.0)
    per_kernel = {}
    total = 0.0
    kernels, srcs = OPERATIONS[a.operation]
    for k in kernels:
        fk = fetch.get(k, {}).get("FETCH_SIZE", 0.0)
        wk = write.get(k, {}).get("WRITE_SIZE", 0.0)
        b = fk * 1024.0 * sf + wk * 1024.0 * sw
        per_kernel[k] = {"fetch_kib": fk, "write_kib": wk, "bytes": b}
        total += b
    rec = {
        "workload": a.workload,
        "source": ", ".join(os.path.basename(src) for src in srcs),
        "source_sha256": ", ".join(source_sha256(src) for src in srcs),
        "copy_calibration": {"bytes": a.copy_bytes, "fetch_kib": copy_f, "write_kib": copy_w,
                             "fetch_scale": sf, "write_scale": sw},
        "kernels": per_kernel,
        "bytes_per_call": total,
        "commands": a.command,
    }
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("outdir")
    s.add_argument("--out", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--operation", choices=sorted(OPERATIONS), default="decode")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--operation", choices=sorted(OPERATIONS), default="decode")
    a = ap.parse_args(argv)
    return cmd_stats(a) if a.what == "stats" else cmd_traffic(a)


if __name__ == "__main__":
    sys.exit(main())
