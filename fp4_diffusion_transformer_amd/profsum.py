"""Summarise rocprofv3 output of bench.py runs into profiles/.

Usage (after the three profiling runs named in the summary header):
  python -m fp4_diffusion_transformer_amd.profsum TRACE_DIR FETCH_DIR WRITE_DIR OUT_TXT [CALIB_MIB] [CMDS]
  python -m fp4_diffusion_transformer_amd.profsum --sq SQ_DIR OUT_TXT [CMDS]

TRACE_DIR: `rocprofv3 --kernel-trace --stats --output-format csv` output;
FETCH_DIR / WRITE_DIR: `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
(csv) of a bench.py run with --calib-mib CALIB_MIB, which fills a buffer of
that size (a known write) and sums it (a known read).  FETCH_SIZE is scaled
by the ratio of the known read to what it reports for the sum, WRITE_SIZE by
that of the known write to what it reports for the fill.  CMDS (optional) is
a text file with the commands that produced the inputs, copied into OUT_TXT.
Writes OUT_TXT (kernel time table + per-launch HBM traffic) and
profiles/hbm_traffic.json (traffic per kernel, with the hash of the kernel
sources it was taken on; bench.py reports it only while the hash matches).

--sq: SQ_DIR is a `rocprofv3 --pmc` run (csv) of SQ_VALU_MFMA_BUSY_CYCLES,
SQ_BUSY_CU_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F6F4, SQ_INSTS_MFMA,
SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, SQ_INSTS_VALU, SQ_INSTS_LDS and
GRBM_GUI_ACTIVE.  OUT_TXT gets, per GEMM kernel, the averages per dispatch:
MFMA utilisation (MFMA busy cycles over 4 SIMDs x CU-busy cycles), the FP4
work the MFMA counter implies (512 flops per MOP, to check against 2MNK),
the bank-conflict share of LDS-active cycles, instruction counts, and the
SGPRs, LDS bytes and scratch (spill) bytes of the dispatch.
"""

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_diffusion_transformer_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _find(d, pattern):
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError("no %s under %s" % (pattern, d))
    return hits[0]


def kernel_key(name):
    """Short key of a kernel name (template arguments kept)."""
    n = name.replace("fp4dit::(anonymous namespace)::", "").replace("fp4dit::", "").replace(
        "(anonymous namespace)::", "")
    for a, b in (("gemm_fp4_kernel<0,", "gemm_none<"), ("gemm_fp4_kernel<1,", "gemm_rmsnorm_head<"),
                 ("gemm_fp4_kernel<2,", "gemm_swiglu<"), ("gemm_fp4_kernel<3,", "gemm_swiglu_transform<")):
        n = n.replace(a, b)
    return n.split("(")[0].replace("void ", "").replace(" ", "").strip()


def counters(d, counter):
    path = _find(d, "*counter_collection.csv")
    per_kernel = defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                per_kernel[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return per_kernel


def main(argv):
    trace_dir, fetch_dir, write_dir, out_txt = argv[1:5]
    copy_mib = int(argv[5]) if len(argv) > 5 else 256
    cmds = open(argv[6]).read().strip().splitlines() if len(argv) > 6 else []
    stats = _find(trace_dir, "*kernel_stats.csv")
    with open(stats) as f:
        rows = list(csv.DictReader(f))
    fetch = counters(fetch_dir, "FETCH_SIZE")
    write = counters(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib << 20

    def calib(per_kernel, tag):
        # the calibration kernel is the largest dispatch of its kind (other
        # small fills, e.g. of a zeroed index buffer, share the name)
        best = None
        for name, vals in per_kernel.items():
            if tag in name:
                v = max(vals)
                best = v if best is None or v > best else best
        return copy_bytes / (best * 1024.0) if best else None
    f_fac, w_fac = calib(fetch, "reduce_kernel"), calib(write, "FillFunctor")
    lines = ["# rocprofv3 kernel statistics and HBM traffic of bench.py", ""]
    lines += ["# " + c for c in cmds] + [""] if cmds else []
    lines += ["source hash of fp4_diffusion_transformer_amd/csrc: " + source_hash(), ""]
    lines.append("%-48s %8s %12s %12s %10s" % ("kernel", "calls", "avg_us", "min_us", "pct"))
    for r in rows:
        lines.append("%-48s %8s %12.2f %12.2f %10s" % (kernel_key(r["Name"])[:48], r["Calls"],
                     float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, r.get("Percentage", "")[:6]))
    lines += ["", "calibration: fill + sum of %d MiB; FETCH_SIZE factor %s, WRITE_SIZE factor %s" % (
        copy_mib, "%.4f" % f_fac if f_fac else "n/a", "%.4f" % w_fac if w_fac else "n/a"), ""]
    lines.append("%-48s %16s %16s" % ("kernel", "read MB/launch", "write MB/launch"))
    traffic = {}
    for name in sorted(set(fetch) | set(write)):
        fr = sum(fetch.get(name, [0])) / max(len(fetch.get(name, [1])), 1) * 1024 * (f_fac or 1.0)
        wr = sum(write.get(name, [0])) / max(len(write.get(name, [1])), 1) * 1024 * (w_fac or 1.0)
        key = kernel_key(name)
        lines.append("%-48s %16.2f %16.2f" % (key[:48], fr / 1e6, wr / 1e6))
        traffic[key] = {"read_bytes": fr, "write_bytes": wr}
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    # one record per workload (the summary's name kernels_<workload>.txt): the
    # same kernel instantiation runs at other sizes in other workloads
    base = os.path.basename(out_txt)
    workload = base[len("kernels_"):-len(".txt")] if base.startswith("kernels_") and base.endswith(".txt") else base
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    rec = {}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
    if rec.get("source_hash") != source_hash() or "workloads" not in rec:
        rec = {"source_hash": source_hash(), "workloads": {}}
    rec["note"] = ("bytes that leave the L2 per launch (reads that miss it, writes sent on): requests to the "
                   "memory side, served by the Infinity Cache or HBM; an upper bound on HBM bytes")
    rec["workloads"][workload] = {
        "copy_mib": copy_mib, "fetch_factor": f_fac, "write_factor": w_fac,
        "kernels": {k: {"hbm_bytes_per_launch": v["read_bytes"] + v["write_bytes"], **v} for k, v in traffic.items()}}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))


def sq_main(argv):
    sq_dir, out_txt = argv[2:4]
    cmds = open(argv[4]).read().strip().splitlines() if len(argv) > 4 else []
    path = _find(sq_dir, "*counter_collection.csv")
    vals = defaultdict(lambda: defaultdict(list))
    regs = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            key = kernel_key(row["Kernel_Name"])
            if not key.startswith("gemm_"):
                continue
            vals[key][row["Counter_Name"]].append(float(row["Counter_Value"]))
            regs[key] = (row.get("VGPR_Count"), row.get("Accum_VGPR_Count"), row.get("SGPR_Count"),
                         row.get("LDS_Block_Size"), row.get("Scratch_Size"))
    lines = ["# rocprofv3 SQ counters of bench.py's GEMM kernels (averages per dispatch)", ""]
    lines += ["# " + c for c in cmds] + [""] if cmds else []
    lines.append("source hash of fp4_diffusion_transformer_amd/csrc: " + source_hash())
    lines.append("")
    lines.append("%-28s %9s %11s %9s %11s %11s %11s %5s %7s %7s" % (
        "kernel", "mfma_util", "fp4_gflop", "lds_conf", "mfma_insts", "valu_insts", "lds_insts",
        "sgpr", "lds_B", "scratch"))
    for key in sorted(vals):
        d = {c: sum(v) / len(v) for c, v in vals[key].items()}
        busy = d.get("SQ_BUSY_CU_CYCLES", 0.0)
        util = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * busy) if busy else float("nan")
        lds = d.get("SQ_LDS_IDX_ACTIVE", 0.0)
        conf = d.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds if lds else 0.0
        _, _, sg, ldsb, scr = regs[key]
        lines.append("%-28s %9.3f %11.1f %9.4f %11.0f %11.0f %11.0f %5s %7s %7s" % (
            key[:28], util, d.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0) * 512 / 1e9, conf,
            d.get("SQ_INSTS_MFMA", 0.0), d.get("SQ_INSTS_VALU", 0.0), d.get("SQ_INSTS_LDS", 0.0), sg, ldsb, scr))
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--sq":
        sq_main(sys.argv)
    else:
        main(sys.argv)
