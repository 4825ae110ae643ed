"""Short text summaries of rocprofv3 output for this library's kernels.

    python -m int4_quantized_moe_amd.profsum trace DIR OUT --command "..."
        kernel table (calls, average and total time) from DIR/run_kernel_stats.csv

    python -m int4_quantized_moe_amd.profsum traffic FETCH_DIR WRITE_DIR OUT --kernel NAME
            --phase PHASE --workload NAME --copy-mib N --command "..."
        HBM bytes per dispatch of one kernel from a FETCH_SIZE run and a
        WRITE_SIZE run, each scaled by what the same counter reads for the
        plain elementwise copy bench.py --copy-mib N runs (N MiB read, N MiB
        written), tagged with the hash of the library sources so that a stale
        figure is recognised.

    python -m int4_quantized_moe_amd.profsum counters OUT --workload NAME --command "..." DIR [DIR ...]
        per-kernel compute counters from one or more --pmc runs (each DIR one
        pass): MFMA busy share of SIMD cycles, instructions per MFMA, LDS bank
        conflicts and waits, the clock during the kernel, registers and LDS.

bench.py reads the traffic summary of its dominant kernel and reports it only
while the sources hash the same.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def source_hash() -> str:
    """sha256 over the library's kernel sources, public header and build settings."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*"))) + sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    files.append(os.path.join(HERE, "build.py"))
    for path in files:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _find(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def _counter_per_dispatch(path: str):
    """{kernel name: {counter: [value summed over the dispatch's rows, per dispatch]}}"""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = r["Dispatch_Id"]
            names[key] = r["Kernel_Name"]
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for key, counters in per.items():
        for c, v in counters.items():
            out[names[key]][c].append(v)
    return out


def trace(directory: str, out: str, command: str) -> None:
    rows = list(csv.DictReader(open(_find(directory, "kernel_stats.csv"))))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# rocprofv3 kernel summary (--kernel-trace --stats)", f"# command: {command}",
             f"# library sources sha256: {source_hash()}", "",
             f"{'kernel':64s} {'calls':>6s} {'avg_us':>11s} {'total_ms':>10s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{r['Name'][:64]:64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:11.1f} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}")
    # every dispatch of the expert GEMMs in launch order: the first of each is the
    # warm-up step's, the rest are the timed steps' (what bench.py's events measure)
    per = collections.defaultdict(list)
    for r in sorted(csv.DictReader(open(_find(directory, "kernel_trace.csv"))), key=lambda r: int(r["Start_Timestamp"])):
        if "k_gemm<" in r["Kernel_Name"]:
            per[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if per:
        lines += ["", "per-dispatch durations (us) of the expert GEMMs, in launch order:"]
        for name, ds in sorted(per.items()):
            timed = ds[1:] if len(ds) > 1 else ds
            lines.append(f"{name[:64]:64s} " + " ".join(f"{d:.1f}" for d in ds) +
                         f"   avg after the first: {sum(timed) / len(timed):.1f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def traffic(fetch_dir: str, write_dir: str, out: str, kernel: str, phase: str, workload: str, copy_mib: int,
            command: str) -> None:
    fetch = _counter_per_dispatch(_find(fetch_dir, "counter_collection.csv"))
    write = _counter_per_dispatch(_find(write_dir, "counter_collection.csv"))

    def pick(table, counter, needle):
        vals = [v for name, cs in table.items() if needle in name for v in cs.get(counter, [])]
        if not vals:
            raise KeyError(f"{counter}: no dispatch of a kernel matching {needle!r}")
        return sum(vals) / len(vals), len(vals)

    copy_bytes = copy_mib * (1 << 20)
    f_copy, _ = pick(fetch, "FETCH_SIZE", "neg_kernel")
    w_copy, _ = pick(write, "WRITE_SIZE", "neg_kernel")
    f_kib, nf = pick(fetch, "FETCH_SIZE", kernel)
    w_kib, nw = pick(write, "WRITE_SIZE", kernel)
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    read_b = f_kib * 1024.0 * f_scale
    write_b = w_kib * 1024.0 * w_scale
    lines = [f"# HBM traffic of {kernel} ({phase}) at workload {workload}",
             "# two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE), KiB per dispatch, each scaled by",
             f"# what the same counter reads for a plain elementwise copy of {copy_mib} MiB (bench.py --copy-mib)",
             f"# command: {command}",
             f"kernel: {kernel}", f"phase: {phase}", f"workload: {workload}", f"source_sha256: {source_hash()}",
             f"dispatches: {nf} {nw}", f"fetch_kib_per_dispatch: {f_kib:.1f}", f"write_kib_per_dispatch: {w_kib:.1f}",
             f"copy_fetch_kib: {f_copy:.1f}", f"copy_write_kib: {w_copy:.1f}",
             f"fetch_scale: {f_scale:.4f}", f"write_scale: {w_scale:.4f}",
             f"hbm_read_bytes_per_launch: {read_b:.0f}", f"hbm_write_bytes_per_launch: {write_b:.0f}",
             f"hbm_bytes_per_launch: {read_b + write_b:.0f}"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path: str):
    """Bytes per launch from a traffic summary, or None if absent or taken from other sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash():
        return None
    return {"read": float(kv["hbm_read_bytes_per_launch"]), "write": float(kv["hbm_write_bytes_per_launch"])}


SIMDS = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
XCDS = 8  # GRBM counters come summed over the 8 XCDs, each counting the whole dispatch


def _dispatch_rows(path: str):
    """{dispatch id: (kernel name, {counter: value summed over rows}, extra columns)}"""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = r["Dispatch_Id"]
            if key not in out:
                extra = {k: r.get(k) for k in ("VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size",
                                               "Start_Timestamp", "End_Timestamp", "Grid_Size")}
                out[key] = (r["Kernel_Name"], collections.defaultdict(float), extra)
            out[key][1][r["Counter_Name"]] += float(r["Counter_Value"])
    return out


def counters(dirs, out: str, workload: str, command: str) -> None:
    """Average per dispatch of every counter, per kernel, over the given passes; the
    first dispatch of each kernel (the warm-up step's) is left out when there are more."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    meta = {}
    durations = collections.defaultdict(list)
    for d in dirs:
        rows = _dispatch_rows(_find(d, "counter_collection.csv"))
        # durations from a kernel trace taken in the same run, where the counter rows carry none
        try:
            with open(_find(d, "kernel_trace.csv")) as f:
                for r in csv.DictReader(f):
                    hit = rows.get(r["Dispatch_Id"])
                    if hit and not hit[2].get("End_Timestamp"):
                        hit[2]["Start_Timestamp"], hit[2]["End_Timestamp"] = r["Start_Timestamp"], r["End_Timestamp"]
        except FileNotFoundError:
            pass
        by_kernel = collections.defaultdict(list)
        for key in sorted(rows, key=int):
            name, cs, extra = rows[key]
            by_kernel[name].append((cs, extra))
        for name, lst in by_kernel.items():
            use = lst[1:] if len(lst) > 1 else lst
            meta.setdefault(name, use[0][1])
            for cs, extra in use:
                for c, v in cs.items():
                    per[name][c].append(v)
                if extra.get("Start_Timestamp") and extra.get("End_Timestamp"):
                    durations[name].append((int(extra["End_Timestamp"]) - int(extra["Start_Timestamp"])) / 1e3)
    avg = {n: {c: sum(v) / len(v) for c, v in cs.items()} for n, cs in per.items()}
    for cs in avg.values():
        if "GRBM_GUI_ACTIVE" in cs:
            cs["GRBM_GUI_ACTIVE"] /= XCDS
    total = {n: sum(durations[n]) / len(durations[n]) if durations[n] else 0.0 for n in avg}  # us per dispatch
    names = sorted(avg, key=lambda n: -total[n])
    lines = [f"# compute counters per kernel at workload {workload} (rocprofv3 --pmc, one pass per directory;",
             "# averages per dispatch, the warm-up step's dispatch left out)", f"# command: {command}",
             f"# library sources sha256: {source_hash()}", "#",
             "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs), GRBM_GUI_ACTIVE taken per XCD (sum / 8)",
             "# valu/mfma, lds/mfma, salu/mfma, vmem/mfma = SQ_INSTS_* / SQ_INSTS_MFMA (VALU counts include the MFMAs)",
             "# bank_confl = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; lds_wait, any_wait = SQ_WAIT_INST_LDS,",
             "# SQ_WAIT_ANY (quad-cycles) x 4 / SQ_WAVE_CYCLES (share of wave time); clock_ghz = GRBM_GUI_ACTIVE /",
             "# dispatch duration; vgpr / agpr / lds_bytes as the dispatch reports them", "",
             f"{'kernel':52s} {'us':>8s} {'ghz':>5s} {'mfma_busy':>9s} {'valu/mfma':>9s} {'lds/mfma':>8s} "
             f"{'salu/mfma':>9s} {'vmem/mfma':>9s} {'bank_confl':>10s} {'lds_wait':>8s} {'any_wait':>8s} "
             f"{'vgpr':>4s} {'agpr':>4s} {'lds_bytes':>9s}"]

    def ratio(a, b):
        return a / b if b else float("nan")

    for n in names:
        cs = avg[n]
        us = sum(durations[n]) / len(durations[n]) if durations[n] else float("nan")
        ghz = ratio(cs.get("GRBM_GUI_ACTIVE", 0.0), us * 1e3) if durations[n] else float("nan")
        mfma = cs.get("SQ_INSTS_MFMA", 0.0)
        busy = ratio(cs.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), cs.get("GRBM_GUI_ACTIVE", 0.0) * SIMDS)
        wave = cs.get("SQ_WAVE_CYCLES", 0.0)
        m = meta[n]
        lines.append(
            f"{n[:52]:52s} {us:8.1f} {ghz:5.2f} {busy:9.3f} {ratio(cs.get('SQ_INSTS_VALU', 0.0), mfma):9.2f} "
            f"{ratio(cs.get('SQ_INSTS_LDS', 0.0), mfma):8.2f} {ratio(cs.get('SQ_INSTS_SALU', 0.0), mfma):9.2f} "
            f"{ratio(cs.get('SQ_INSTS_VMEM', 0.0), mfma):9.2f} "
            f"{ratio(cs.get('SQ_LDS_BANK_CONFLICT', 0.0), cs.get('SQ_LDS_IDX_ACTIVE', 0.0)):10.3f} "
            f"{ratio(4 * cs.get('SQ_WAIT_INST_LDS', 0.0), wave):8.3f} {ratio(4 * cs.get('SQ_WAIT_ANY', 0.0), wave):8.3f} "
            f"{m.get('VGPR_Count') or '-':>4s} {m.get('Accum_VGPR_Count') or '-':>4s} {m.get('LDS_Block_Size') or '-':>9s}")
    lines += ["", "raw averages per dispatch:"]
    for n in names:
        lines.append(n[:100])
        lines.append("  " + " ".join(f"{c}={v:.0f}" for c, v in sorted(avg[n].items())))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("out")
    c.add_argument("--kernel", required=True)
    c.add_argument("--phase", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--copy-mib", type=int, required=True)
    c.add_argument("--command", required=True)
    k = sub.add_parser("counters")
    k.add_argument("out")
    k.add_argument("dirs", nargs="+")
    k.add_argument("--workload", required=True)
    k.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.mode == "trace":
        trace(a.dir, a.out, a.command)
    elif a.mode == "counters":
        counters(a.dirs, a.out, a.workload, a.command)
    else:
        traffic(a.fetch_dir, a.write_dir, a.out, a.kernel, a.phase, a.workload, a.copy_mib, a.command)


if __name__ == "__main__":
    main()
