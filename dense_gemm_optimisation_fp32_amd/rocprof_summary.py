"""Summaries of rocprofv3 output for this library's kernels (measurement
tooling; nothing here runs on the GPU).

    python -m dense_gemm_optimisation_fp32_amd.rocprof_summary stats DIR
        Markdown table of the kernel-trace statistics (``*_kernel_stats.csv``
        under DIR): calls, average / min / max duration per kernel.
    python -m dense_gemm_optimisation_fp32_amd.rocprof_summary counters DIR [--workload W]
        Per-kernel averages of the counters in ``*_counter_collection.csv``
        under DIR, with the derived figures the tile/occupancy sweep reports:
          cycles        GRBM_GUI_ACTIVE / 8 (it sums the 8 XCD instances)
          mfma_busy     SQ_VALU_MFMA_BUSY_CYCLES / (cycles * 1024 SIMDs)
          lds_conflict  SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
          l2_hit        TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)
          flop          512 * SQ_INSTS_VALU_MFMA_MOPS_F32
        and, for FETCH_SIZE / WRITE_SIZE (KiB per dispatch), the values as
        read; scale them by a copy kernel of known size run in the same
        program (bench.py --calibrate-copy).

The profiler's kernel names are the demangled template names; ``short_name``
maps them to the variant-style names the library reports
(``dma_256x256x16_s4``, ``dma_256x256x16_w4x2_s4`` (wavefront layouts other than 2 x 2
named), ``sk_dma_64x128x16_s2``, ``skinny_16x64_w16_d4`` ...).
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import sys
from collections import defaultdict

SIMDS = 1024          # 256 CUs x 4 SIMDs
XCDS = 8


def short_name(kernel: str) -> str:
    """A compact name for a kernel from its (demangled or mangled) name."""
    k = kernel
    m = re.search(r"DmaTile<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+)(?:, (?:true|false))?>", k)
    if m is None:
        m = re.search(r"DmaTileILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)", k)
    if m and "gemm_mfma_dma" in k:
        waves = "" if (m.group(4), m.group(5)) == ("2", "2") else f"_w{m.group(4)}x{m.group(5)}"
        base = f"dma_{m.group(1)}x{m.group(2)}x{m.group(3)}{waves}_s{m.group(6)}"
        if "sk_kernel" in k:
            return "sk_" + base + ("_bcol" if re.search(r"EEELb1EEEv|>, true>", k) else "")
        sliver = "_sliver" if "sliver_kernel" in k else ""
        flags = re.search(r">, (true|false), (true|false), (true|false), (true|false)>", k)
        if flags:
            tags = [t for t, f in zip(("bcol", "acol", "epi", "wide"), flags.groups()) if f == "true"]
            return base + "".join("_" + t for t in tags) + sliver
        return base + sliver
    m = (re.search(r"SkinnyTile<(\d+), (\d+), (\d+)(?:, (\d+))?>", k)
         or re.search(r"SkinnyTileILi(\d+)ELi(\d+)ELi(\d+)E(?:Li(\d+)E)?", k))
    if m:
        return f"skinny_{16 * int(m.group(4) or 1)}x{m.group(3)}_w{m.group(1)}_d{m.group(2)}"
    m = re.search(r"MfmaTile<(\d+), (\d+), (\d+), \d+, \d+>", k) or re.search(r"MfmaTileILi(\d+)ELi(\d+)ELi(\d+)", k)
    if m and "gemm_mfma_kernel" in k:
        return f"mfma_{m.group(1)}x{m.group(2)}x{m.group(3)}"
    m = (re.search(r"FewColTile<(\d+)(?:, (\d+), \d+(?:, (\d+))?)?>, (true|false)", k)
         or re.search(r"FewColTileILi(\d+)E(?:Li(\d+)ELi\d+E(?:Li(\d+)E)?)?EELb([01])", k))
    if m:
        r, waves, kc = int(m.group(1)), m.group(2), m.group(3)
        default_kc = 1024 if r == 8 else 2048
        return (f"fewcol_r{r}" + (f"_k{kc}" if kc and int(kc) != default_kc else "")
                + (f"_w{waves}" if waves and int(waves) != 4 else "")
                + ("_t" if "fewcol_t_" in k else "") + ("_bcol" if m.group(4) in ("true", "1") else ""))
    if "gemm_valu_kernel" in k:
        return "valu_128x128x8"
    if "zero_words_kernel" in k:
        return "zero_words"
    return k[:60]


def _rows(pattern):
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            yield from csv.DictReader(f)


def stats(directory: str) -> str:
    rows = list(_rows(os.path.join(directory, "**", "*kernel_stats.csv")))
    out = ["| kernel | short name | calls | average (us) | min (us) | max (us) | share of GPU time |",
           "|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        name = r.get("Name") or r.get("KernelName") or ""
        out.append(f"| `{name[:90]}` | {short_name(name)} | {r.get('Calls')} | "
                   f"{float(r.get('AverageNs', 0)) / 1e3:.2f} | {float(r.get('MinNs', 0)) / 1e3:.2f} | "
                   f"{float(r.get('MaxNs', 0)) / 1e3:.2f} | {float(r.get('Percentage', 0)):.1f} % |")
    return "\n".join(out)


def counters(directory: str):
    """{kernel name: {counter: average per dispatch}, with the derived figures}."""
    per = defaultdict(lambda: defaultdict(list))
    for r in _rows(os.path.join(directory, "**", "*counter_collection.csv")):
        name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
        cname = r.get("Counter_Name") or r.get("Counter-Name")
        val = r.get("Counter_Value") or r.get("Counter-Value")
        disp = r.get("Dispatch_Id") or r.get("Dispatch-Id")
        if cname is None or val is None:
            continue
        per[name][(cname, disp)].append(float(val))
    out = {}
    for name, vals in per.items():
        sums = defaultdict(list)
        for (cname, _disp), v in vals.items():
            sums[cname].append(sum(v))          # one value per dispatch (summed over instances)
        avg = {c: sum(v) / len(v) for c, v in sums.items()}
        avg["dispatches"] = max(len(v) for v in sums.values())
        if "GRBM_GUI_ACTIVE" in avg:
            avg["cycles"] = avg["GRBM_GUI_ACTIVE"] / XCDS
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg["cycles"]:
                avg["mfma_busy"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (avg["cycles"] * SIMDS)
        if avg.get("SQ_LDS_IDX_ACTIVE"):
            avg["lds_conflict"] = avg.get("SQ_LDS_BANK_CONFLICT", 0.0) / avg["SQ_LDS_IDX_ACTIVE"]
        hit, miss = avg.get("TCC_HIT_sum"), avg.get("TCC_MISS_sum")
        if hit is not None and miss is not None and hit + miss:
            avg["l2_hit"] = hit / (hit + miss)
        if "SQ_INSTS_VALU_MFMA_MOPS_F32" in avg:
            avg["flop"] = 512.0 * avg["SQ_INSTS_VALU_MFMA_MOPS_F32"]
        out[name] = avg
    return out


def counters_table(directory: str) -> str:
    res = counters(directory)
    cols = ["dispatches", "cycles", "mfma_busy", "lds_conflict", "l2_hit", "flop", "FETCH_SIZE", "WRITE_SIZE"]
    present = [c for c in cols if any(c in v for v in res.values())]
    out = ["| kernel | " + " | ".join(present) + " |", "|---|" + "---|" * len(present)]
    for name, v in sorted(res.items(), key=lambda kv: short_name(kv[0])):
        cells = []
        for c in present:
            x = v.get(c)
            if x is None:
                cells.append("")
            elif c in ("mfma_busy", "lds_conflict", "l2_hit"):
                cells.append(f"{x:.3f}")
            elif c == "flop":
                cells.append(f"{x:.4g}")
            else:
                cells.append(f"{x:.0f}")
        out.append(f"| {short_name(name)} | " + " | ".join(cells) + " |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["stats", "counters"])
    ap.add_argument("directory")
    args = ap.parse_args(argv)
    print(stats(args.directory) if args.mode == "stats" else counters_table(args.directory))


if __name__ == "__main__":
    sys.exit(main())
