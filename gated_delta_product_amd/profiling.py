"""Turn rocprofv3 CSV output into the short text summaries kept with the
benchmark: per-kernel launch statistics and measured HBM traffic per launch.

    python -m gated_delta_product_amd.profiling stats  STATS_CSV OUT.md  --command "..."
    python -m gated_delta_product_amd.profiling traffic FETCH_CSV WRITE_CSV OUT.json \
        --copy-mib 512 --command "..."
    python -m gated_delta_product_amd.profiling mfma PMC_CSV OUT.md --command "..."

Traffic: FETCH_SIZE and WRITE_SIZE are read per dispatch (KiB).  The same run
contains one plain device copy of a known size, which fixes how many bytes
one counted KiB stands for (the raw counts need not equal the bytes moved: on
MI355X the fetch count of a copy reads half of the bytes it copies).  Each
kernel's bytes per launch = mean over its dispatches of FETCH_SIZE * fetch_factor + WRITE_SIZE * write_factor, with
fetch_factor = copy bytes / copy FETCH_SIZE and likewise for writes.  The
JSON records the kernel-source digest it was taken on, so a reader can tell
when the figure no longer describes the built kernel.
"""
import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_product_amd", "csrc")

# host-visible operation -> (device symbol substring, sources that define it)
KERNELS = {
    "gdp_decode_prepare": ("gdp_decode_prepare_k", ["prepare.hip"]),
    "gdp_decode_update": ("gdp_decode_k", ["decode.hip"]),
    "gdp_prefill_prepare": ("gdp_prepare_k", ["prepare.hip"]),
    "gdp_recompute_w_u": ("gdp_wy_k", ["wy.hip"]),
    "gdp_chunk_h": ("gdp_chunk_h_k", ["chunk_h.hip"]),
    "gdp_chunk_o": ("gdp_chunk_o_k", ["chunk_o.hip"]),
    "gdp_chunk_ho": ("gdp_chunk_ho_k", ["chunk_ho.hip"]),
    "gdp_seg_map": ("gdp_seg_map_k", ["scan.hip"]),
    "gdp_seg_scan": ("gdp_seg_scan_k", ["scan.hip"]),
}
COPY_SYMBOL = "copyBuffer"


def src_digest(op):
    """Digest of the sources a kernel is built from (its file + the shared header)."""
    h = hashlib.sha256()
    for f in KERNELS[op][1] + ["gdp_common.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _op_of(name):
    for op, (sym, _) in KERNELS.items():
        if sym in name:
            return op
    if COPY_SYMBOL in name:
        return "copy"
    return None


def read_counter(path, counter):
    """{op: [value per dispatch]} for one counter of a counter-collection CSV."""
    out = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            op = _op_of(r["Kernel_Name"])
            if op:
                out[op].append(float(r["Counter_Value"]))
    return out


def traffic(fetch_csv, write_csv, copy_mib):
    fe = read_counter(fetch_csv, "FETCH_SIZE")
    wr = read_counter(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * 1024 * 1024
    # the calibration copy is the largest copy dispatch in the run
    cf, cw = max(fe.get("copy", [0.0])), max(wr.get("copy", [0.0]))
    if cf <= 0 or cw <= 0:
        raise SystemExit("no calibration copy found in the counter CSVs")
    ff, wf = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    res = {"_calibration": {"copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
                            "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}}
    for op in KERNELS:
        if not fe.get(op) or not wr.get(op):
            continue
        f_kib = sum(fe[op]) / len(fe[op])
        w_kib = sum(wr[op]) / len(wr[op])
        res[op] = {"fetch_kib": round(f_kib, 1), "write_kib": round(w_kib, 1),
                   "bytes_per_launch": int(round(f_kib * 1024 * ff + w_kib * 1024 * wf)),
                   "dispatches": [len(fe[op]), len(wr[op])], "src_digest": src_digest(op)}
    return res


MFMA_PEAK = {"MfmaFlopsBF16": 2.5e15, "MfmaFlopsF16": 2.5e15, "MfmaFlopsF32": 157.3e12}  # MI355X dense peaks (flop/s)


def mfma_table(pmc_csv):
    """Per kernel: matrix-core flops per launch (rocprofv3's MfmaFlopsBF16,
    MfmaFlopsF16 and MfmaFlopsF32, i.e. MOPS x 512; a counter the run did not
    take reads as zero), the MfmaUtil busy percentage, and the rate over the
    profiled launch duration against each dtype's dense peak."""
    acc = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(list)
    with open(pmc_csv) as f:
        for r in csv.DictReader(f):
            op = _op_of(r["Kernel_Name"])
            if not op or op == "copy":
                continue
            acc[op][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "MfmaUtil":
                dur[op].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    lines = ["| kernel | launches | bf16 MFMA GFLOP | f16 MFMA GFLOP | f32 MFMA GFLOP | profiled us | MFMA TFLOP/s "
             "| fraction of dense peak | MfmaUtil % |",
             "|---|---|---|---|---|---|---|---|---|"]
    for op in KERNELS:
        if op not in acc:
            continue
        d = acc[op]
        mean = lambda k: sum(d.get(k, [0.0])) / max(1, len(d.get(k, [0.0])))
        fl = {k: mean(k) for k in MFMA_PEAK}
        util = mean("MfmaUtil")
        t = sum(dur[op]) / max(1, len(dur[op]))
        rate = sum(fl.values()) / t if t > 0 else 0.0
        frac = sum(fl[k] / t / MFMA_PEAK[k] for k in MFMA_PEAK) if t > 0 else 0.0
        lines.append("| %s | %d | %.2f | %.2f | %.2f | %.1f | %.1f | %.3f | %.1f |" % (
            op, len(d.get("MfmaUtil", [])), fl["MfmaFlopsBF16"] / 1e9, fl["MfmaFlopsF16"] / 1e9,
            fl["MfmaFlopsF32"] / 1e9, t * 1e6, rate / 1e12, frac, util))
    return "\n".join(lines)


def stats_table(stats_csv):
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                         float(r["MaxNs"]), float(r["Percentage"])))
    lines = ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in rows:
        op = _op_of(name) or name[:60]
        lines.append("| %s | %d | %.1f | %.1f | %.1f | %.1f |" % (op, calls, avg / 1e3, mn / 1e3, mx / 1e3, pct))
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="Kernel launch statistics")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--segments", type=int, default=None,
                   help="segments of the profiled run: the per-launch bytes of the chunk "
                        "stages hold for that split only")
    t.add_argument("--path", default=None, help="chunk forward of the profiled run (pipelined or scan)")
    m = sub.add_parser("mfma")
    m.add_argument("pmc_csv")
    m.add_argument("out")
    m.add_argument("--command", required=True)
    m.add_argument("--title", default="Matrix-core work per kernel")
    a = ap.parse_args(argv)
    if a.cmd == "mfma":
        digests = ", ".join("%s %s" % (op, src_digest(op)) for op in KERNELS)
        text = ("# %s\n\nCommand (run from the repository root on one MI355X):\n\n    %s\n\n%s\n\n"
                "MFMA flops are rocprofv3's MfmaFlopsBF16 / MfmaFlopsF16 / MfmaFlopsF32 (matrix-core "
                "operations x 512, dense tiles as issued); the fraction sums each dtype's rate over its "
                "dense peak (bf16 and f16 2.5 PFLOP/s, f32 157.3 TFLOP/s); durations are the profiled "
                "launches.\n\n"
                "Kernel source digests: %s\n" % (a.title, a.command, mfma_table(a.pmc_csv), digests))
        with open(a.out, "w") as f:
            f.write(text)
    elif a.cmd == "stats":
        digests = ", ".join("%s %s" % (op, src_digest(op)) for op in KERNELS)
        text = "# %s\n\nCommand (run from the repository root on one MI355X):\n\n    %s\n\n%s\n\n" \
               "Kernel source digests: %s\n" % (a.title, a.command, stats_table(a.stats_csv), digests)
        with open(a.out, "w") as f:
            f.write(text)
    else:
        res = traffic(a.fetch_csv, a.write_csv, a.copy_mib)
        res["_command"] = a.command
        if a.segments is not None:
            res["_segments"] = a.segments
        if a.path is not None:
            res["_path"] = a.path
        with open(a.out, "w") as f:
            json.dump(res, f, indent=1, sort_keys=True)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
