#!/usr/bin/env python3
"""Turn rocprofv3 CSV output into the committed summaries under profiles/.

  rocprof_summary.py stats  KERNEL_STATS_CSV OUT_MD  "COMMAND"
      kernel-trace statistics (calls, average / min / max duration) as markdown
  rocprof_summary.py traffic CONFIG FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_BYTES "COMMANDS"
      HBM bytes per dflash_head_topk call from FETCH_SIZE / WRITE_SIZE (KiB per
      dispatch, summed over a dispatch's rows), each scaled by what the same
      counter reads for a plain device copy of COPY_BYTES bytes; merged into
      profiles/head_topk_traffic.json under CONFIG, with the sha of the head
      kernel source the counters were taken on.
"""

import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
# the head kernels' sources: the kernel file and the key-sort header it includes
HEAD_SRC = [os.path.join(ROOT, "block_draft_verification_amd", "csrc", f) for f in ("head_topk.hip", "keysort.hpp")]
TRAFFIC = os.path.join(ROOT, "profiles", "head_topk_traffic.json")


def short(name):
    name = name.replace("(anonymous namespace)::", "").split("(")[0]
    return name[5:] if name.startswith("void ") else name


def stats(csv_path, out_md, command):
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics\n", f"Command:\n\n```\n{command}\n```\n",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def per_kernel_kib(csv_path, counter):
    """Mean KiB per dispatch of each kernel (rows of one dispatch summed)."""
    per = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = short(r["Kernel_Name"])
    by = collections.defaultdict(list)
    for d, v in per.items():
        by[names[d]].append(v)
    return {k: sum(v) / len(v) for k, v in by.items()}, by


def traffic(config, fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes, commands):
    copy_bytes = float(copy_bytes)
    f, _ = per_kernel_kib(fetch_csv, "FETCH_SIZE")
    w, _ = per_kernel_kib(write_csv, "WRITE_SIZE")
    cf, _ = per_kernel_kib(cfetch_csv, "FETCH_SIZE")
    cw, _ = per_kernel_kib(cwrite_csv, "WRITE_SIZE")
    # the copy kernel is the one with the largest fetch
    ck = max(cf, key=cf.get)
    f_scale = copy_bytes / (cf[ck] * 1024.0)
    w_scale = copy_bytes / (cw[ck] * 1024.0)
    head = {k: v for k, v in f.items() if "dflash::head_" in k}
    kern = {}
    total = 0.0
    for k in sorted(head):
        fb = f[k] * 1024.0 * f_scale
        wb = w.get(k, 0.0) * 1024.0 * w_scale
        kern[k] = {"fetch_bytes": int(fb), "write_bytes": int(wb)}
        total += fb + wb
    h = hashlib.sha256()
    for path in HEAD_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()[:16]
    try:
        rec = json.load(open(TRAFFIC))
    except (OSError, ValueError):
        rec = {}
    rec[config] = {"head_source_sha": sha, "bytes_per_launch": int(total), "kernels": kern,
                   "copy_calibration": {"kernel": ck, "bytes": int(copy_bytes),
                                        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
                   "commands": commands}
    json.dump(rec, open(TRAFFIC, "w"), indent=1)
    md = [f"# HBM traffic of one dflash_head_topk call, workload {config}\n",
          f"Commands:\n\n```\n{commands}\n```\n",
          f"Counters are rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each taken in a run of its own "
          f"and scaled by what the same counter reads for a plain {int(copy_bytes)}-byte device copy "
          f"(`{ck}`): fetch x{f_scale:.4f}, write x{w_scale:.4f}.  Head kernel sources (head_topk.hip and keysort.hpp) sha256[:16] = `{sha}`.\n",
          "| kernel | fetched bytes | written bytes |", "|---|---:|---:|"]
    for k, v in kern.items():
        md.append(f"| `{k}` | {v['fetch_bytes']:,} | {v['write_bytes']:,} |")
    md.append(f"| **total per call** | | **{int(total):,}** |")
    open(os.path.join(ROOT, "profiles", f"head_topk_{config}_traffic.md"), "w").write("\n".join(md) + "\n")
    print(json.dumps(rec[config], indent=1))


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(*sys.argv[2:5])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:9])
    else:
        sys.exit(__doc__)
