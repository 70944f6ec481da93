"""Summaries of rocprofv3 output for the fused LSH-attention forward pass.

  python -m lsh_attention_amd.prof_summary stats <rocprofv3 output dir> [K]
      Markdown table of the --kernel-trace --stats run (average duration per
      kernel, per launch); with K, also each kernel's average over its last K
      launches from the kernel trace (bench.py's K timed steps come last).
  python -m lsh_attention_amd.prof_summary traffic <pmc dir> <workload> <out.json>
      From --pmc runs of FETCH_SIZE and WRITE_SIZE (one sub-directory per
      pass, each holding *_counter_collection.csv) over a benchmark run that
      ends with one plain device copy of known size (bench.py
      --copy-probe-mib N): per-kernel HBM bytes per launch, with each counter
      scaled by (copy bytes / counter reading of the copy).  Each entry keeps
      the sha256 of the kernel's source so a later change invalidates it.
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
KERNEL_SOURCES = {
    "prep": ["hash.hip"], "hash": ["hash.hip"], "fixup": ["hash.hip"],
    "sort_hist": ["sort.hip"], "sort_scatter": ["sort.hip"],
    "chunk_attn": ["chunk_attn.hip"], "variant_rec": ["chunk_attn.hip"], "combine": ["combine.hip"],
    "bwd_prep": ["attn_bwd.hip", "lsh_bwd.h"], "attn_bwd": ["attn_bwd.hip", "lsh_bwd.h"],
    "bwd_reduce": ["attn_bwd.hip", "lsh_bwd.h"],
}


N_XCDS = 8      # GRBM_GUI_ACTIVE counts shader cycles on each of the 8 XCDs
N_SIMDS = 1024  # 256 CUs x 4 SIMDs; SQ counters are device totals
# Cycles one MFMA occupies its SIMD's matrix pipe: v_mfma_f32_32x32x16_bf16 (hash)
# and v_mfma_f32_16x16x32_bf16 (chunk attention) at 512 and 256 MACs per cycle.
MFMA_CYCLES = {"hash": 32, "chunk_attn": 16}


def kernel_key(name: str) -> str:
    m = re.search(r"(\w+)_kernel\b", name)
    if m:
        return m.group(1)
    return "copy" if "copy" in name.lower() else name[:40]


def source_sha256(key: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(key, []) + ["lsh_internal.h"]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def last_launches_us(d: str, k: int) -> dict:
    """{kernel name: mean duration (us) of its last k launches} from the kernel trace."""
    f = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0]
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(f)):
        per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    return {name: sum(e - s for s, e in sorted(v)[-k:]) / min(k, len(v)) / 1e3 for name, v in per.items()}


def stats_table(d: str, last: int = 0) -> str:
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    tail = last_launches_us(d, last) if last else {}
    extra = f" average of the last {last} (us) |" if last else ""
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |" + extra,
           "|---|---|---|---|---|---|" + ("---|" if last else "")]
    for r in rows:
        t = tail.get(r["Name"])
        out.append(f"| {kernel_key(r['Name'])} (`{r['Name'][:70]}`) | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} % |" +
                   ((f" {t:.2f} |" if t is not None else " - |") if last else ""))
    return "\n".join(out)


def counters(d: str):
    """{kernel: {counter: mean over dispatches of the per-dispatch value}} plus the copy kernel's bytes.
    Each kernel also gets "_dur_ns" (mean dispatch duration) and, when GRBM_GUI_ACTIVE was
    collected, "_clock_ghz" (mean over dispatches of that counter / 8 XCDs / duration)."""
    per = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    dur = collections.defaultdict(dict)
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = kernel_key(r["Kernel_Name"])
            key = f"{f}:{r['Dispatch_Id']}"
            per[k][r["Counter_Name"]][key] += float(r["Counter_Value"])
            dur[k][key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in per.items()}
    for k in out:
        out[k]["_dur_ns"] = sum(dur[k].values()) / len(dur[k])
        g = per[k].get("GRBM_GUI_ACTIVE")
        if g:
            clocks = [g[x] / N_XCDS / dur[k][x] for x in g if dur[k].get(x)]
            out[k]["_clock_ghz"] = sum(clocks) / len(clocks)
    # The probe is the run's largest copy (small read-backs use the same blit kernel).
    if "copy" in per:
        out["copy"] = {c: max(v.values()) for c, v in per["copy"].items()}
    return out


def traffic(d: str, workload: str, out_json: str, copy_mib: int = 256):
    c = counters(d)
    cp = c["copy"]
    copy_kib = copy_mib * 1024.0
    f_fac = copy_kib / cp["FETCH_SIZE"]
    w_fac = copy_kib / cp["WRITE_SIZE"]
    res = {"workload": workload, "copy_probe_bytes": copy_mib << 20,
           "fetch_scale": round(f_fac, 4), "write_scale": round(w_fac, 4), "kernels": {}}
    for k, v in c.items():
        if k == "copy" or "FETCH_SIZE" not in v:
            continue
        fetch = v["FETCH_SIZE"] * 1024 * f_fac
        write = v.get("WRITE_SIZE", 0.0) * 1024 * w_fac
        res["kernels"][k] = {"fetch_bytes": round(fetch), "write_bytes": round(write),
                             "traffic_bytes": round(fetch + write), "source_sha256": source_sha256(k)}
    json.dump(res, open(out_json, "w"), indent=1)
    return res


def counter_table(d: str, kernels=("hash", "fixup", "sort_scatter", "chunk_attn", "combine")) -> str:
    """Markdown table of SQ counters per dispatch (mean over the kernel's
    dispatches) from --pmc runs under `d`, with ratios of like units only."""
    c = counters(d)
    names = sorted({k for v in c.values() for k in v})
    out = ["| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for k in kernels:
        if k in c:
            out.append(f"| {k} | " + " | ".join(f"{c[k].get(n, float('nan')):.4g}" for n in names) + " |")
    out += ["", "| kernel | VALU insts per MFMA inst | MFMA-busy cycles with VALU co-executing | "
            "LDS bank-conflict cycles per LDS inst | transcendental share of VALU |", "|---|---|---|---|---|"]
    for k in kernels:
        v = c.get(k, {})
        def ratio(a, b):
            return f"{v[a] / v[b]:.3g}" if v.get(a) is not None and v.get(b) else "-"
        out.append(f"| {k} | {ratio('SQ_INSTS_VALU', 'SQ_INSTS_MFMA')} | "
                   f"{ratio('SQ_VALU_MFMA_COEXEC_CYCLES', 'SQ_VALU_MFMA_BUSY_CYCLES')} | "
                   f"{ratio('SQ_LDS_BANK_CONFLICT', 'SQ_INSTS_LDS')} | {ratio('SQ_INSTS_VALU_TRANS_F32', 'SQ_INSTS_VALU')} |")
    out += ["", "| kernel | dispatch (us) | shader clock (GHz) | MFMA pipe busy | MFMA busy from instruction count "
            "| VALU issue (non-MFMA) | wave-cycles waiting on dependencies | wave-cycles waiting to issue |",
            "|---|---|---|---|---|---|---|---|"]
    for k in kernels:
        v = c.get(k, {})
        ghz = v.get("_clock_ghz")
        cyc = v["_dur_ns"] * ghz if ghz else None  # shader cycles per dispatch

        def frac(x):
            return "-" if x is None else f"{x:.3f}"
        busy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMDS * cyc) if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in v else None
        by_count = (v["SQ_INSTS_MFMA"] * MFMA_CYCLES[k] / (N_SIMDS * cyc)
                    if cyc and k in MFMA_CYCLES and "SQ_INSTS_MFMA" in v else None)
        valu = ((v["SQ_INSTS_VALU"] - v.get("SQ_INSTS_MFMA", 0.0)) * 4 / (N_SIMDS * cyc)
                if cyc and "SQ_INSTS_VALU" in v else None)
        wc = v.get("SQ_WAVE_CYCLES")
        w_dep = v["SQ_WAIT_ANY"] / wc if wc and "SQ_WAIT_ANY" in v else None
        w_iss = v["SQ_WAIT_INST_ANY"] / wc if wc and "SQ_WAIT_INST_ANY" in v else None
        out.append(f"| {k} | {v['_dur_ns'] / 1e3:.1f} | {frac(ghz)} | {frac(busy)} | {frac(by_count)} | "
                   f"{frac(valu)} | {frac(w_dep)} | {frac(w_iss)} |")
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats_table(sys.argv[2], int(sys.argv[3]) if len(sys.argv) > 3 else 0))
    elif sys.argv[1] == "counters":
        print(counter_table(sys.argv[2]))
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], sys.argv[4]), indent=1))
    else:
        raise SystemExit(__doc__)
