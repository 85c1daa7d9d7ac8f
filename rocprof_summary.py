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
  rocprof_summary.py counters CONFIG PMC_CSV OUT_MD "COMMAND"
      SQ/GRBM counters per library kernel (mean per dispatch, summed over
      their instances), with the derived MfmaUtil = MFMA-busy cycles /
      (active cycles * 1024 SIMDs), LdsBankConflict = conflicts / (active -
      conflicts) and LdsUtil = LDS-active cycles / (active cycles * 256 CUs),
      where active cycles = GRBM_GUI_ACTIVE / 8 (rocprofv3 reports the
      counter summed over the 8 XCDs)
  rocprof_summary.py traffic_all CONFIG FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_BYTES OUT_MD "COMMANDS"
      HBM bytes per dispatch of every library kernel (calibrated as for
      `traffic`), beside its algorithmic bytes where they have a closed form
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


N_SIMD, N_CU = 1024, 256


def per_kernel_counters(csv_path):
    """{kernel: {counter: mean per dispatch}}, each counter summed over its
    rows (instances) of a dispatch."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(csv_path)):
        d, c, v = r["Dispatch_Id"], r["Counter_Name"], float(r["Counter_Value"])
        names[d] = short(r["Kernel_Name"])
        per[d][c] += v
    by = collections.defaultdict(list)
    for d, cs in per.items():
        by[names[d]].append(cs)
    out = {}
    for k, lst in by.items():
        keys = set().union(*lst)
        out[k] = {c: sum(x.get(c, 0.0) for x in lst) / len(lst) for c in keys}
        out[k]["dispatches"] = len(lst)
    return out


def counters(config, csv_path, out_md, command):
    ks = {k: v for k, v in per_kernel_counters(csv_path).items() if k.startswith("dflash::")}
    cols = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
            "SQ_WAIT_INST_LDS", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"]
    md = [f"# SQ counters per dispatch, workload {config}\n", f"Command:\n\n```\n{command}\n```\n",
          "Mean per dispatch over the run, each counter summed over its instances.  GRBM_GUI_ACTIVE arrives summed "
          "over the 8 XCDs (8x the dispatch's active cycles), so active = GRBM_GUI_ACTIVE / 8.  Derived as rocprofv3 "
          "defines them: MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (active x 1024 SIMDs) (16 busy cycles per "
          "v_mfma_f32_16x16x32_bf16); LdsBankConflict = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - "
          "SQ_LDS_BANK_CONFLICT), conflict cycles per access cycle; LdsUtil = SQ_LDS_IDX_ACTIVE / (active x 256 CUs).\n",
          "| kernel | MfmaUtil | LdsBankConflict | LdsUtil | " + " | ".join(c for c in cols) + " |",
          "|---|---:|---:|---:|" + "---:|" * len(cols)]
    for k in sorted(ks, key=lambda k: -ks[k].get("GRBM_GUI_ACTIVE", 0.0)):
        v = ks[k]
        gui = v.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        act, conf = v.get("SQ_LDS_IDX_ACTIVE", 0.0), v.get("SQ_LDS_BANK_CONFLICT", 0.0)
        mfma = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * N_SIMD) if gui else float("nan")
        bank = conf / (act - conf) if act > conf else float("nan")
        lds = act / (gui * N_CU) if gui else float("nan")
        md.append(f"| `{k}` | {100 * mfma:.1f} % | {bank:.4f} | {100 * lds:.1f} % | " +
                  " | ".join(f"{v.get(c, 0.0):,.0f}" for c in cols) + " |")
    open(out_md, "w").write("\n".join(md) + "\n")
    print("\n".join(md))


def algorithmic_bytes(config):
    """Closed-form bytes per dispatch of the cycle's kernels for a workload."""
    sys.path.insert(0, ROOT)
    from workload import get_config
    c = get_config(config)
    g = {"greedy": c.B, "sample": 0, "mixed": c.B // 2}[c.verify]
    return {
        "dflash::conv2tap_kernel": 8 * c.L * c.B * c.T * c.D,
        "dflash::head_": c.V * c.D * 2 + c.M * c.D * 2 + c.M * 16 * 8,
        "dflash::greedy_partial_kernel": g * c.T * c.V * 4,
        "dflash::sample_stats_kernel": (c.B - g) * c.T * c.V * 4,
    }


def traffic_all(config, fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes, out_md, commands):
    copy_bytes = float(copy_bytes)
    f, _ = per_kernel_kib(fetch_csv, "FETCH_SIZE")
    w, _ = per_kernel_kib(write_csv, "WRITE_SIZE")
    cf, _ = per_kernel_kib(cfetch_csv, "FETCH_SIZE")
    cw, _ = per_kernel_kib(cwrite_csv, "WRITE_SIZE")
    ck = max(cf, key=cf.get)
    f_scale = copy_bytes / (cf[ck] * 1024.0)
    w_scale = copy_bytes / (cw[ck] * 1024.0)
    alg = algorithmic_bytes(config)
    md = [f"# HBM traffic per dispatch of the cycle's kernels, workload {config}\n",
          f"Commands:\n\n```\n{commands}\n```\n",
          f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one run each) scaled by what the same counter reads for a "
          f"plain {int(copy_bytes)}-byte device copy (`{ck}`): fetch x{f_scale:.4f}, write x{w_scale:.4f}.  "
          f"Algorithmic bytes: conv 8 L B T D, head V D 2 + M D 2 + M 128 (the GEMM kernel), greedy partials "
          f"(greedy rows) T V 4, sampler statistics (sampled rows) T V 4.\n",
          "| kernel | fetched bytes | written bytes | algorithmic bytes | measured / algorithmic |",
          "|---|---:|---:|---:|---:|"]
    for k in sorted(f):
        if not k.startswith("dflash::"):
            continue
        fb = f[k] * 1024.0 * f_scale
        wb = w.get(k, 0.0) * 1024.0 * w_scale
        a = next((v for p, v in alg.items() if k.startswith(p) and "merge" not in k and "rank" not in k), None)
        ratio = f"{(fb + wb) / a:.3f}" if a else "—"
        md.append(f"| `{k}` | {int(fb):,} | {int(wb):,} | {a:,} | {ratio} |" if a else
                  f"| `{k}` | {int(fb):,} | {int(wb):,} | — | — |")
    open(out_md, "w").write("\n".join(md) + "\n")
    print("\n".join(md))


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(*sys.argv[2:5])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:9])
    elif sys.argv[1] == "counters":
        counters(*sys.argv[2:6])
    elif sys.argv[1] == "traffic_all":
        traffic_all(*sys.argv[2:10])
    else:
        sys.exit(__doc__)
