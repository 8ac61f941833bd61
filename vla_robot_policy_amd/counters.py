"""Hardware-counter summaries of the policy step's kernels, per kernel label.

Reads the CSV output of rocprofv3 counter passes taken over
``bench.py --only-label <labels> --kernel-reps 1`` (each label's captured
launches relaunched once, in graph order, label after label; bench.py prints
that launch sequence to stderr) and attributes the trailing dispatches of
each pass to labels. HBM bytes come from FETCH_SIZE and WRITE_SIZE scaled by
what the same counters read for a plain device copy of known size.

Usage (after the passes, from the repository root):

    python -m vla_robot_policy_amd.counters --dir <out> --passes fetch write mfma lds \\
        --calib-fetch cfetch --calib-write cwrite --copy-bytes 268435456 \\
        --bench <bench.json> --config 4 --md <summary.md> --traffic profiles/hbm_traffic.json

where <out>/<pass>/<pass>_counter_collection.csv and <out>/<pass>.log are
one pass's CSV and bench.py stderr.
"""

from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys

SIMDS = 1024          # 256 compute units x 4 SIMDs
XCDS = 8              # GRBM_GUI_ACTIVE is summed over the accelerator complex dies
CLOCK_HZ = 2.4e9
HBM_BPS = 8.0e12


def _rows(pdir: str, name: str):
    return list(csv.DictReader(open(os.path.join(pdir, name, f"{name}_counter_collection.csv"))))


def dispatches(pdir: str, name: str):
    """Per-dispatch counter sums of one pass, in dispatch order."""
    disp = collections.OrderedDict()
    for r in _rows(pdir, name):
        d = int(r["Dispatch_Id"])
        e = disp.setdefault(d, {"kernel": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "wg": int(r["Workgroup_Size"]),
                                "vgpr": int(r["VGPR_Count"]), "agpr": int(r["Accum_VGPR_Count"]),
                                "lds": int(r["LDS_Block_Size"]), "scratch": int(r["Scratch_Size"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def attribute(pdir: str, name: str):
    """Per-label means of one --only-label pass: the last dispatches of the
    process are the relaunched labels, in the logged order."""
    log = open(os.path.join(pdir, f"{name}.log")).read()
    m = re.search(r"launch sequence (\[.*\])", log)
    if not m:
        raise SystemExit(f"{name}.log: no launch sequence")
    seq = json.loads(m.group(1))
    ds = dispatches(pdir, name)
    total = sum(s["launches"] for s in seq)
    tail = ds[-total:]
    out, i = {}, 0
    for s in seq:
        part = tail[i:i + s["launches"]]
        i += s["launches"]
        agg = collections.defaultdict(float)
        for d in part:
            for k, v in d.items():
                if isinstance(v, (int, float)):
                    agg[k] += v
        n = len(part)
        out[s["label"]] = {"n": n, "per_step": s["per_step"], "kernel": part[0]["kernel"], **{k: v / n for k, v in agg.items()}}
    return out


def copy_factor(pdir: str, name: str, counter: str, nbytes: int) -> float:
    """Bytes per counted unit: a copy of nbytes reads and writes nbytes."""
    vals = [d[counter] for d in dispatches(pdir, name) if counter in d and "copy" in d["kernel"].lower()]
    if not vals:
        vals = [d[counter] for d in dispatches(pdir, name) if counter in d]
    v = max(vals)
    return nbytes / (v * 1024.0)


def algorithmic(cfg):
    """Algorithmic bytes and FLOPs per launch by label (roofline operators)."""
    from . import roofline
    ops = {o.name: o for o in roofline.step_ops(cfg)}
    ops.update(roofline.fused_ops(cfg))
    return {k: (o.bytes, o.flops, o.compute) for k, o in ops.items()}


def summarise(res, factors, alg, times):
    rows = []
    for lb, v in res.items():
        g = v.get("GRBM_GUI_ACTIVE")
        row = {"label": lb, "kernel": v["kernel"], "launches_per_step": v["per_step"], "grid": v.get("grid"),
               "workgroup": v.get("wg"), "vgpr": v.get("vgpr"), "agpr": v.get("agpr"), "lds_bytes": v.get("lds")}
        t = times.get(lb)
        row["us"] = t
        if "FETCH_SIZE" in v:
            row["fetch_bytes"] = v["FETCH_SIZE"] * 1024.0 * factors["fetch"]
        if "WRITE_SIZE" in v:
            row["write_bytes"] = v["WRITE_SIZE"] * 1024.0 * factors["write"]
        if lb in alg:
            b, f, comp = alg[lb]
            row["alg_bytes"], row["alg_flops"] = b, f
            if t:
                row["alg_GBps"] = b / (t * 1e-6) / 1e9
                row["hbm_frac"] = b / (t * 1e-6) / HBM_BPS
            if "fetch_bytes" in row and "write_bytes" in row and b:
                row["measured_over_alg"] = (row["fetch_bytes"] + row["write_bytes"]) / b
        mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + v.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
        if mops and t:
            row["mfma_TFLOPs"] = mops * 512 / (t * 1e-6) / 1e12
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            row["mfma_busy_pct"] = 100.0 * v["SQ_VALU_MFMA_BUSY_CYCLES"] / (g / XCDS * SIMDS)
        if "SQ_INSTS_LDS" in v and v.get("SQ_INSTS_MFMA"):
            row["lds_per_mfma"] = v["SQ_INSTS_LDS"] / v["SQ_INSTS_MFMA"]
        if g and "SQ_LDS_BANK_CONFLICT" in v:
            row["lds_bank_conflict_pct"] = 100.0 * v["SQ_LDS_BANK_CONFLICT"] / (g / XCDS * 256)
        if "SQ_LDS_IDX_ACTIVE" in v and g:
            row["lds_active_pct"] = 100.0 * v["SQ_LDS_IDX_ACTIVE"] / (g / XCDS * 256)
        rows.append(row)
    return rows


def _f(x, fmt):
    return "" if x is None else format(x, fmt)


def markdown(rows, header: str) -> str:
    out = [header, "",
           "| label | launches/step | us | alg MB | fetch MB | write MB | meas/alg | alg GB/s | HBM frac | MFMA TF/s | MFMA busy % | LDS instr / MFMA | LDS active % | bank conflict % | VGPR+AGPR | grid/wg |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---|"]
    for r in sorted(rows, key=lambda r: -(r.get("us") or 0) * (r.get("launches_per_step") or 0)):
        out.append("| `{}` | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {}/{} |".format(
            r["label"], r["launches_per_step"], _f(r.get("us"), ".2f"),
            _f(r.get("alg_bytes") and r["alg_bytes"] / 1e6, ".2f"), _f(r.get("fetch_bytes") and r["fetch_bytes"] / 1e6, ".2f"),
            _f(r.get("write_bytes") and r["write_bytes"] / 1e6, ".2f"), _f(r.get("measured_over_alg"), ".2f"),
            _f(r.get("alg_GBps"), ".0f"), _f(r.get("hbm_frac"), ".3f"), _f(r.get("mfma_TFLOPs"), ".1f"),
            _f(r.get("mfma_busy_pct"), ".1f"), _f(r.get("lds_per_mfma"), ".2f"), _f(r.get("lds_active_pct"), ".1f"),
            _f(r.get("lds_bank_conflict_pct"), ".1f"), int((r.get("vgpr") or 0) + (r.get("agpr") or 0)),
            int(r.get("grid") or 0) // max(1, int(r.get("workgroup") or 1)), int(r.get("workgroup") or 0)))
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--dir", required=True)
    ap.add_argument("--passes", nargs="+", required=True)
    ap.add_argument("--calib-fetch")
    ap.add_argument("--calib-write")
    ap.add_argument("--copy-bytes", type=int, default=256 << 20)
    ap.add_argument("--bench", help="bench.py JSON line of the same build (per-label HIP-event durations)")
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--md")
    ap.add_argument("--traffic", help="write per-label HBM bytes for bench.py's roofline.traffic")
    ap.add_argument("--header", default="")
    a = ap.parse_args(argv)
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from synth import get_config
    res = {}
    for name in a.passes:
        for lb, v in attribute(a.dir, name).items():
            res.setdefault(lb, {}).update(v)
    factors = {"fetch": copy_factor(a.dir, a.calib_fetch, "FETCH_SIZE", a.copy_bytes) if a.calib_fetch else 1.0,
               "write": copy_factor(a.dir, a.calib_write, "WRITE_SIZE", a.copy_bytes) if a.calib_write else 1.0}
    times = {}
    if a.bench:
        line = json.loads(open(a.bench).read().strip().splitlines()[-1])
        times = {k: v["avg_us"] for k, v in line.get("kernels_us", {}).items()}
    rows = summarise(res, factors, algorithmic(get_config(a.config)), times)
    if a.md:
        with open(a.md, "w") as f:
            f.write(markdown(rows, a.header))
    if a.traffic:
        import importlib.util
        spec = importlib.util.spec_from_file_location("bench", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
        bench = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(bench)
        t = {"kernel_source_sha": bench.kernel_source_sha(), "fetch_factor": factors["fetch"], "write_factor": factors["write"],
             "config": a.config,
             "labels": {r["label"]: {"fetch_bytes_per_launch": r["fetch_bytes"], "write_bytes_per_launch": r["write_bytes"],
                                     "algorithmic_bytes_per_launch": r.get("alg_bytes")}
                        for r in rows if "fetch_bytes" in r and "write_bytes" in r},
             "source": os.path.relpath(a.md, os.path.dirname(os.path.dirname(os.path.abspath(__file__)))) if a.md else None}
        with open(a.traffic, "w") as f:
            json.dump(t, f, indent=1)
    print(markdown(rows, a.header))


if __name__ == "__main__":
    main()
