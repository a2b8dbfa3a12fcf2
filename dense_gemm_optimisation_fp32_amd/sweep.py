"""Tile-shape / occupancy sweep over the compiled variant table.

For every variant and workload: the compiler's per-kernel resources (VGPRs,
AGPRs, LDS, scratch, waves per SIMD, from the build's resource report), the
occupancy the performance model derives from them, and the measured kernel
time and TFLOPS on the GPU.  This is the reuse-versus-occupancy trade-off of
"GPU 算子优化中的数据复用" (sections 3-8 and 12): bigger tiles reuse more and
keep fewer waves resident.

    python -m dense_gemm_optimisation_fp32_amd.sweep --workloads sq4096,ffn --out sweep.jsonl

The few-row path is swept with bench.py (--workload skinny --variant V
--rotate 8), which reads B from HBM at every launch.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys

from . import perfmodel as pm

RESOURCES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "kernel_resources.txt")


def kernel_resources(path: str = RESOURCES):
    """Parse the compiler's resource remarks: {mangled kernel name: {field: value}}."""
    out = {}
    cur = None
    if not os.path.exists(path):
        return out
    for line in open(path):
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?):\s+(\S+)", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = val
    return out


def kernel_tag(info: dict, layout_b: int) -> str:
    """Regular expression for the mangled name of the kernel a variant
    launches (the one-tile-per-workgroup kernel, row-major A, no epilogue) for
    one B layout."""
    b = f"Lb{layout_b}E"
    if info["kind"] == 1:
        return f"gemm_valu_kernelI{b}"
    if info["kind"] == 2:
        m = re.match(r"skinny_(\d+)x(\d+)_w(\d+)_d(\d+)", info["name"])
        rt = int(m.group(1)) // 16
        return f"SkinnyTileILi{m.group(3)}ELi{m.group(4)}ELi{m.group(2)}ELi{rt}EEE{b}"
    dims = (f"ILi{info['bm']}ELi{info['bn']}ELi{info['bk']}ELi{info['waves_m']}ELi{info['waves_n']}")
    if info["name"].startswith("dma_"):
        # DmaTile<..., STAGES, PRIO>, then B_COL, A_COL = false, EPI = false,
        # WIDE_C (the 8/16-byte C stores a row-major-B plan takes when N is a
        # multiple of the wavefront tile's 32-column blocks, as in every
        # sweep workload)
        wide = int(layout_b == 0 and info["wave_n"] // 32 in (2, 4))
        return (f"gemm_mfma_dma_kernelINS_7DmaTile{dims}ELi{info['stages']}ELb[01]EEE{b}"
                f"Lb0ELb0ELb{wide}EEEv")
    return f"gemm_mfma_kernelINS_8MfmaTile{dims}EEE{b}"


def resources_for(info: dict, layout_b: int, res: dict):
    """Resources of the kernel a variant launches for one B layout."""
    tag = re.compile(kernel_tag(info, layout_b))
    for name, r in res.items():
        if tag.search(name):
            vg = int(r.get("VGPRs", 0))
            ag = int(r.get("AGPRs", 0))
            lds = int(r.get("LDS Size [bytes/block]", 0))
            wgs, waves = pm.gfx950_occupancy(vg, ag, lds, info["threads"])
            return {"vgpr": vg, "agpr": ag, "sgpr": int(r.get("TotalSGPRs", 0)), "lds": lds,
                    "scratch": int(r.get("ScratchSize [bytes/lane]", 0)),
                    "compiler_waves_per_simd": int(r.get("Occupancy [waves/SIMD]", 0)),
                    "model_wgs_per_cu": wgs, "model_waves_per_simd": waves}
    return {}


def time_variant(g, torch, w, variant, steps, warmup, warmup_s=0.25):
    from workloads import workload_operands

    A, B = workload_operands(w)
    dev = torch.device("cuda", 0)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.empty((w.m, w.n), dtype=torch.float32, device=dev)
    ldb = w.n if w.layout_b == 0 else w.k
    plan = g.Plan(w.m, w.n, w.k, w.layout_b, w.k, ldb, w.n, variant)
    stream = torch.cuda.current_stream(dev)
    # Warm up for at least `warmup` launches and 0.25 s of GPU time: the
    # engine clock ramps for ~0.1 s under sustained matrix-core load.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    plan.run(dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), stream.cuda_stream)
    t1.record(stream)
    torch.cuda.synchronize()
    est = max(t0.elapsed_time(t1) / 1e3, 1e-6)
    for _ in range(max(warmup, int(warmup_s / est))):
        plan.run(dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    # Average launch duration: one event pair around `steps` back-to-back
    # launches on the launch stream.
    t0.record(stream)
    for _ in range(steps):
        plan.run(dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), stream.cuda_stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return plan.info, t0.elapsed_time(t1) / 1e3 / steps


def kernel_short_name(rec: dict, layout_b: int, n: int) -> str:
    """rocprof_summary.short_name of the kernel a sweep record ran (N
    decides whether a row-major-B plan takes the wide-store kernel)."""
    name = rec["name"]
    if name.startswith("dma_"):
        stages = re.search(r"_s(\d+)$", name).group(1)
        w = re.search(r"_w(\d+)x(\d+)_", name)
        waves = "" if w is None or w.groups() == ("2", "2") else f"_w{w.group(1)}x{w.group(2)}"
        base = f"dma_{rec['bm']}x{rec['bn']}x{rec['bk']}{waves}_s{stages}"
        if layout_b == 1:
            return base + "_bcol"
        nb = rec["wave_tile"][1] // 32
        return base + ("_wide" if nb in (2, 4) and n % nb == 0 else "")
    if name.startswith("mfma_"):
        return f"mfma_{rec['bm']}x{rec['bn']}x{rec['bk']}"
    if name.startswith("valu_"):
        return "valu_128x128x8"
    return name


def table(jsonl: str, counter_dirs: dict) -> str:
    """Markdown table of a sweep file: one row per variant, per workload the
    measured TFLOPS, and for the workloads with a counter run the matrix-core
    busy fraction, the LDS bank-conflict ratio and the L2 hit rate."""
    from workloads import WORKLOADS

    from . import rocprof_summary as rs

    recs = [json.loads(line) for line in open(jsonl) if line.strip()]
    workloads = list(dict.fromkeys(r["workload"] for r in recs))
    ctr = {w: {rs.short_name(k): v for k, v in rs.counters(d).items()} for w, d in counter_dirs.items()}
    head = ["variant", "tile", "wave tile", "stages", "VGPR", "AGPR", "SGPR", "LDS KiB", "scratch",
            "waves/SIMD (compiler / model)"]
    for w in workloads:
        head.append(f"{w} TFLOPS")
        if w in ctr:
            head += [f"{w} MFMA busy", f"{w} LDS conflicts", f"{w} L2 hit"]
    out = ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    by_variant = {}
    for r in recs:
        by_variant.setdefault(r["variant"], {})[r["workload"]] = r
    for v, per in by_variant.items():
        r0 = next(iter(per.values()))
        row = [f"`{r0['name']}`", f"{r0['bm']}x{r0['bn']}x{r0['bk']}", f"{r0['wave_tile'][0]}x{r0['wave_tile'][1]}",
               re.search(r"_s(\d+)$", r0["name"]).group(1) if r0["name"].startswith("dma_") else "2",
               str(r0.get("vgpr", "")), str(r0.get("agpr", "")), str(r0.get("sgpr", "")),
               str(r0.get("lds", 0) // 1024), str(r0.get("scratch", "")),
               f"{r0.get('compiler_waves_per_simd', '')} / {r0.get('model_waves_per_simd', '')}"]
        for w in workloads:
            r = per.get(w)
            row.append(f"{r['tflops']:.1f}" if r else "")
            if w in ctr:
                c = ctr[w].get(kernel_short_name(r0, WORKLOADS[w].layout_b, WORKLOADS[w].n), {}) if r else {}
                row += [f"{c['mfma_busy']:.3f}" if "mfma_busy" in c else "",
                        f"{c['lds_conflict']:.3f}" if "lds_conflict" in c else "",
                        f"{c['l2_hit']:.3f}" if "l2_hit" in c else ""]
        out.append("| " + " | ".join(row) + " |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="sq4096,sq4096t,ragged,ffn")
    ap.add_argument("--variants", default="all")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--out", default="sweep.jsonl")
    ap.add_argument("--warmup-s", type=float, default=0.25,
                    help="GPU time of warm-up launches per variant (the clock ramps for ~0.1 s)")
    ap.add_argument("--table", metavar="JSONL", help="print the markdown table of a sweep file instead")
    ap.add_argument("--counters", action="append", default=[], metavar="WORKLOAD=DIR",
                    help="with --table: rocprofv3 counter output of a sweep run over one workload")
    args = ap.parse_args(argv)
    if args.table:
        print(table(args.table, dict(c.split("=", 1) for c in args.counters)))
        return 0

    import torch

    import dense_gemm_optimisation_fp32_amd as g
    from workloads import WORKLOADS

    res = kernel_resources()
    nvar = g.gemm_f32_num_variants()
    variants = range(nvar) if args.variants == "all" else [int(v) for v in args.variants.split(",")]
    os.makedirs(os.path.dirname(args.out) or ".", exist_ok=True)
    with open(args.out, "a") as f:
        for name in args.workloads.split(","):
            w = WORKLOADS[name]
            for v in variants:
                kind = g.gemm_f32_variant_info(v)["kind"]
                if (kind == g.GEMM_F32_KIND_SKINNY) != (w.m <= 64) or kind == g.GEMM_F32_KIND_FEWCOL:
                    continue   # the few-row, few-column and tiled paths serve different shape classes
                info, avg = time_variant(g, torch, w, v, args.steps, args.warmup, args.warmup_s)
                rec = {"workload": name, "variant": v, "name": info["name"], "kind": info["kind"],
                       "bm": info["bm"], "bn": info["bn"], "bk": info["bk"],
                       "waves": info["waves_m"] * info["waves_n"], "wave_tile": [info["wave_m"], info["wave_n"]],
                       "grid": info["grid"], "t_avg_us": round(avg * 1e6, 2),
                       "tflops": round(pm.tflops(w.m, w.n, w.k, avg), 2),
                       "pct_peak": round(100 * pm.tflops(w.m, w.n, w.k, avg) * 1e12 / pm.MI355X_FP32_MATRIX_PEAK, 2),
                       "hbm_gbs": round(pm.compulsory_bytes(w.m, w.n, w.k) / avg / 1e9, 1)}
                rec.update(resources_for(info, w.layout_b, res))
                f.write(json.dumps(rec) + "\n")
                f.flush()
                print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    sys.exit(main())
