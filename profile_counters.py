"""HBM traffic of one kernel from rocprofv3 counter runs, for bench.py.

Reads four rocprofv3 output databases (rocpd SQLite, `counters_collection`
view): a FETCH_SIZE run and a WRITE_SIZE run of the kernel's workload, and
the same two counters over a plain device-to-device copy of known size
(`bench.py --only copy`).  Each counter of the kernel (median over its
dispatches, KiB per dispatch summed over all counter instances) is scaled by
copy_bytes / (the same counter's reading for the copy), which turns the raw
counter into bytes.  Writes the result into profiles/traffic.json under the
kernel's name, with the SHA-256 of the kernel's source file (bench.py reports
the figure only while that source is unchanged), and prints a summary.

usage: python profile_counters.py --kernel k_decode_mixed \\
           --source bit_quantized_linear_int8_amd/csrc/k_decode.hip \\
           --fetch F.db --write W.db --copy-fetch CF.db --copy-write CW.db \\
           [--copy-bytes 1073741824] [--workload decode_mixed] [--command "..."]

       python profile_counters.py --mfma RUN.db [RUN.db ...]
           matrix-core use per GEMM kernel from runs of SQ_VALU_MFMA_BUSY_CYCLES,
           GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_I8, SQ_LDS_BANK_CONFLICT and
           SQ_LDS_IDX_ACTIVE (median over dispatches); prints a table, writes nothing

       python profile_counters.py --waves RUN.db [RUN.db ...]
           VALU use and s_waitcnt share per kernel from runs of SQ_WAVE_CYCLES, SQ_BUSY_CYCLES,
           SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_VALU, SQ_ACTIVE_INST_ANY, GRBM_GUI_ACTIVE

       python profile_counters.py --stats RUN.db
           kernel durations of a --kernel-trace run (the table the profiles/ summaries hold)

       python profile_counters.py --kernel-times RUN.db WORKLOAD "COMMAND"
           call counts and average durations of the library's kernels in one
           workload's run (bench.py --only WORKLOAD) into profiles/kernel_times.json
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import sqlite3
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))


def per_dispatch(db_path, counter):
    """{kernel name: [counter value per dispatch]} from one rocpd database."""
    db = sqlite3.connect(db_path)
    cur = db.cursor()
    cols = [d[1] for d in cur.execute("pragma table_info(counters_collection)")]
    ci = {c: i for i, c in enumerate(cols)}
    name_col = "kernel_name" if "kernel_name" in ci else "name"
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in cur.execute("select * from counters_collection"):
        if r[ci["counter_name"]] != counter:
            continue
        acc[r[ci[name_col]]][r[ci["dispatch_id"]]] += float(r[ci["value"]])
    return {k: list(v.values()) for k, v in acc.items()}


def kernel_value(db_path, counter, kernel):
    rows = per_dispatch(db_path, counter)
    hits = {k: v for k, v in rows.items() if kernel in k}
    if not hits:
        raise SystemExit("no dispatch of %r with %s in %s" % (kernel, counter, db_path))
    vals = [x for v in hits.values() for x in v]
    return statistics.median(vals), len(vals)


def copy_value(db_path, counter):
    """Reading of the largest dispatch (the 1 GiB copy) in the copy run."""
    rows = per_dispatch(db_path, counter)
    return max(max(v) for v in rows.values())


# MI355X: 8 XCDs of 32 CUs x 4 SIMDs.  GRBM_GUI_ACTIVE, summed over its
# instances, counts the kernel's active cycles once per XCD.
XCDS, SIMDS = 8, 1024


def mfma_table(paths):
    counters = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_I8",
                "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")
    print("%-58s %6s %10s %9s %12s %9s" % ("kernel", "disp", "cycles", "mfma_busy", "int8_ops", "lds_confl"))
    for path in paths:
        med = {c: per_dispatch(path, c) for c in counters}
        for k in sorted(med["SQ_VALU_MFMA_BUSY_CYCLES"]):
            v = {c: statistics.median(med[c][k]) for c in counters if k in med[c]}
            if len(v) < len(counters) or v["SQ_INSTS_VALU_MFMA_MOPS_I8"] == 0:
                continue
            cycles = v["GRBM_GUI_ACTIVE"] / XCDS
            busy = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMDS)
            ops = v["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512
            conf = v["SQ_LDS_BANK_CONFLICT"] / max(v["SQ_LDS_IDX_ACTIVE"], 1.0)
            name = k.split("(")[0].replace("void ", "")
            print("%-58s %6d %10.0f %8.1f%% %12.4g %8.1f%%" % (name[:58], len(med["GRBM_GUI_ACTIVE"][k]), cycles,
                                                          100 * busy, ops, 100 * conf))


def waves_table(paths):
    """VALU use and waiting of each library kernel from runs of SQ_WAVE_CYCLES,
    SQ_BUSY_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_VALU,
    SQ_ACTIVE_INST_ANY and GRBM_GUI_ACTIVE (median over dispatches):
    valu_busy = SQ_ACTIVE_INST_VALU x 4 / (SIMDs x cycles), the share of SIMD
    cycles issuing VALU work (a wave64 VALU instruction occupies a SIMD for 4
    cycles); wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES, the share of wave-cycles
    spent in s_waitcnt; inst_wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, waiting
    for an instruction to issue."""
    counters = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
                "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE")
    print("%-58s %6s %10s %9s %7s %9s" % ("kernel", "disp", "cycles", "valu_busy", "wait", "inst_wait"))
    for path in paths:
        med = {c: per_dispatch(path, c) for c in counters}
        for k in sorted(med["SQ_WAVE_CYCLES"]):
            if "qa::" not in k:
                continue
            v = {c: statistics.median(med[c][k]) for c in counters if k in med[c]}
            if len(v) < len(counters) or v["SQ_WAVE_CYCLES"] == 0:
                continue
            cycles = v["GRBM_GUI_ACTIVE"] / XCDS
            valu = v["SQ_ACTIVE_INST_VALU"] * 4 / (cycles * SIMDS)
            name = k.split("(")[0].replace("void ", "")
            print("%-58s %6d %10.0f %8.1f%% %6.1f%% %8.1f%%" % (name[:58], len(med["GRBM_GUI_ACTIVE"][k]), cycles,
                                                          100 * valu, 100 * v["SQ_WAIT_ANY"] / v["SQ_WAVE_CYCLES"],
                                                          100 * v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"]))


def kernel_durations(db_path):
    """{kernel name: [duration in us per dispatch]} from a --kernel-trace run."""
    db = sqlite3.connect(db_path)
    cur = db.cursor()
    cols = [d[1] for d in cur.execute("pragma table_info(kernels)")]
    ci = {c: i for i, c in enumerate(cols)}
    name_col = "kernel_name" if "kernel_name" in ci else "name"
    out = collections.OrderedDict()
    for r in cur.execute("select * from kernels order by start"):
        out.setdefault(r[ci[name_col]], []).append((r[ci["end"]] - r[ci["start"]]) / 1000.0)
    return out


def stats_table(db_path):
    """Kernel duration table (calls, avg, median, min, max in us, share of the
    summed time) of one rocprofv3 --kernel-trace database."""
    d = kernel_durations(db_path)
    total = sum(sum(v) for v in d.values()) or 1.0
    print("%-70s %6s %9s %9s %9s %9s %6s" % ("kernel", "calls", "avg_us", "med_us", "min_us", "max_us", "pct"))
    for k, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        print("%-70s %6d %9.2f %9.2f %9.2f %9.2f %6.2f" % (k.split("(")[0].replace("void ", "")[:70], len(v),
                                                            statistics.mean(v), statistics.median(v), min(v), max(v),
                                                            100.0 * sum(v) / total))


def record_kernel_times(db_path, workload, command):
    """Every library kernel's call count and average duration in one
    workload's --kernel-trace run, into profiles/kernel_times.json under the
    workload's name, with the SHA-256 of every kernel source file (bench.py
    uses a record only while all of them are unchanged)."""
    d = kernel_durations(db_path)
    csrc = os.path.join(ROOT, "bit_quantized_linear_int8_amd", "csrc")
    shas = {}
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            shas[f] = hashlib.sha256(fh.read()).hexdigest()
    rec = {"command": command, "sources_sha256": shas, "kernels": {}}
    for k, v in d.items():
        if not k.startswith("void qa::") and not k.startswith("qa::"):
            continue
        rec["kernels"][k.split("(")[0].replace("void ", "")] = {
            "calls": len(v), "avg_us": round(statistics.mean(v), 3), "median_us": round(statistics.median(v), 3)}
    if not rec["kernels"]:
        raise SystemExit("no library kernel in %s" % db_path)
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[workload] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({workload: rec["kernels"]}, indent=1))


def main():
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "--mfma":
        mfma_table(sys.argv[2:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--waves":
        waves_table(sys.argv[2:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--stats":
        stats_table(sys.argv[2])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--kernel-times":
        # --kernel-times RUN.db WORKLOAD "COMMAND"
        record_kernel_times(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    p = argparse.ArgumentParser()
    p.add_argument("--kernel", required=True)
    p.add_argument("--source", required=True, help="kernel source, relative to the repository root")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--copy-fetch", required=True)
    p.add_argument("--copy-write", required=True)
    p.add_argument("--copy-bytes", type=int, default=1 << 30)
    p.add_argument("--workload", default="")
    p.add_argument("--command", default="")
    a = p.parse_args()

    f_kib, nf = kernel_value(a.fetch, "FETCH_SIZE", a.kernel)
    w_kib, nw = kernel_value(a.write, "WRITE_SIZE", a.kernel)
    cf_kib = copy_value(a.copy_fetch, "FETCH_SIZE")
    cw_kib = copy_value(a.copy_write, "WRITE_SIZE")
    ff = a.copy_bytes / (cf_kib * 1024.0)
    fw = a.copy_bytes / (cw_kib * 1024.0)
    fetch_b = f_kib * 1024.0 * ff
    write_b = w_kib * 1024.0 * fw
    with open(os.path.join(ROOT, a.source), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    rec = {
        "workload": a.workload, "source": a.source, "source_sha256": sha,
        "fetch_size_kib_per_dispatch": round(f_kib, 1), "write_size_kib_per_dispatch": round(w_kib, 1),
        "dispatches": [nf, nw],
        "copy_bytes": a.copy_bytes, "copy_fetch_size_kib": round(cf_kib, 1), "copy_write_size_kib": round(cw_kib, 1),
        "fetch_scale": round(ff, 4), "write_scale": round(fw, 4),
        "hbm_bytes_per_launch": int(round(fetch_b + write_b)),
        "fetch_bytes_per_launch": int(round(fetch_b)), "write_bytes_per_launch": int(round(write_b)),
        "command": a.command,
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[a.kernel] = rec
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({a.kernel: rec}, indent=1))


if __name__ == "__main__":
    main()
