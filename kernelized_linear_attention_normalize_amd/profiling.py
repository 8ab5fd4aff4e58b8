"""Summaries of rocprofv3 output as the short text files kept under profiles/.

    python -m kernelized_linear_attention_normalize_amd.profiling kernels \\
        --stats <dir>/<prefix>_kernel_stats.csv --cmd "<the profiled command>" --out profiles/<name>.txt
    python -m kernelized_linear_attention_normalize_amd.profiling mfma \\
        --pmc <csv with SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA, GRBM_GUI_ACTIVE> --kernel <substring> \\
        --cmd "<command>" --out profiles/<name>_mfma.txt
    python -m kernelized_linear_attention_normalize_amd.profiling traffic \\
        --kernel <substring> --fetch <csv> --write <csv> --copy-fetch <csv> --copy-write <csv> \\
        --copy-bytes <bytes> --cmd "<commands>" --out profiles/<name>_traffic.txt
    python -m kernelized_linear_attention_normalize_amd.profiling counters \\
        --pmc <csv of pass A> --pmc <csv of pass B> --kernel "<label>=<substring>" ... \\
        --title "<workload>" --cmd "<commands>" --out profiles/<name>_counters.txt

The traffic summary scales the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) by
what they read for a plain device copy of known size, averages over the dispatches of the
named kernel, and records the hash of the HIP sources the counters were taken on
(bench.py reports the figure only while the sources are unchanged).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kernelized_linear_attention_normalize_amd", "csrc")


def source_hash() -> str:
    """Hash of the HIP sources (same definition as bench.py)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(path: str, counter: str, kernel: str) -> tuple[float, int]:
    """Mean value of `counter` over the dispatches whose kernel name contains `kernel`."""
    per = {}
    for r in _rows(path):
        if r.get("Counter_Name") != counter or kernel not in r.get("Kernel_Name", ""):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(per))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernel '{kernel}' in {path}")
    return statistics.mean(per.values()), len(per)


def cmd_kernels(a):
    rows = _rows(a.stats)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel-trace summary: {a.title}", f"# command: {a.cmd}", "#",
             f"{'avg_us':>10} {'calls':>6} {'total_us':>11} {'pct':>6}  kernel"]
    for r in rows[: a.top]:
        lines.append(f"{float(r['AverageNs']) / 1e3:10.2f} {int(r['Calls']):6d} "
                     f"{float(r['TotalDurationNs']) / 1e3:11.1f} {float(r['Percentage']):6.2f}  {r['Name'][:110]}")
    if a.bench_log:  # the JSON line the profiled bench.py printed (HIP-event timings, same run)
        import json
        rec = None
        for line in open(a.bench_log):
            if line.startswith('{"metric"'):
                rec = json.loads(line)
        if rec is not None:
            r = rec["roofline"]
            lines.append(f"# bench.py line of this run: ms_per_step {rec['ms_per_step']}, per-launch HIP-event "
                         f"ms {r.get('launch_ms')}, dominant kernel {r.get('kernel')} {r.get('kernel_ms')} ms, "
                         f"frac {r['frac']} (event times include the profiler's dispatch overhead)")
    lines.append(f"source_hash: {source_hash()}")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(a):
    fk, nf = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    wk, nw = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cf, _ = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw, _ = counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    sf = a.copy_bytes / (cf * 1024.0)   # true bytes per counted byte, reads
    sw = a.copy_bytes / (cw * 1024.0)   # writes
    fetch_b, write_b = fk * 1024.0 * sf, wk * 1024.0 * sw
    lines = [f"# HBM traffic per dispatch of '{a.kernel}' from rocprofv3 PMC counters" + (f" ({a.title})" if a.title else ""),
             f"# commands: {a.cmd}",
             f"# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by the ratio of the",
             f"# known bytes of a plain {a.copy_bytes}-byte device copy ('{a.copy_kernel}') to what the",
             f"# same counter reads for it.",
             f"fetch_kib_per_dispatch: {fk:.1f}   (mean over {nf} dispatches)",
             f"write_kib_per_dispatch: {wk:.1f}   (mean over {nw} dispatches)",
             f"copy_fetch_kib: {cf:.1f}",
             f"copy_write_kib: {cw:.1f}",
             f"fetch_scale: {sf:.4f}",
             f"write_scale: {sw:.4f}",
             f"fetch_bytes_per_launch: {fetch_b:.0f}",
             f"write_bytes_per_launch: {write_b:.0f}",
             f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
             f"source_hash: {source_hash()}"]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# MI355X: 256 CUs x 4 SIMDs in 8 XCDs; GRBM_GUI_ACTIVE is reported summed over the XCDs
SIMDS, XCDS = 1024, 8


def cmd_mfma(a):
    busy, n = counter_per_dispatch(a.pmc, "SQ_VALU_MFMA_BUSY_CYCLES", a.kernel)
    insts, _ = counter_per_dispatch(a.pmc, "SQ_INSTS_MFMA", a.kernel)
    gui, _ = counter_per_dispatch(a.pmc, "GRBM_GUI_ACTIVE", a.kernel)
    cycles = gui / XCDS
    frac = busy / (cycles * SIMDS)
    lines = [f"# MFMA pipe occupancy of '{a.kernel}' from rocprofv3 PMC counters" + (f" ({a.title})" if a.title else ""),
             f"# command: {a.cmd}",
             f"# busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} XCDs x {SIMDS} SIMDs);",
             f"# it counts every executed MFMA (padding and recompute included), unlike the",
             f"# algorithmic fraction bench.py reports.",
             f"mfma_insts_per_dispatch: {insts:.0f}   (mean over {n} dispatches)",
             f"mfma_busy_cycles_per_dispatch: {busy:.0f}",
             f"gpu_active_cycles_per_xcd: {cycles:.0f}",
             f"mfma_busy_fraction: {frac:.4f}",
             f"source_hash: {source_hash()}"]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_dispatch_any(paths, counter, kernel):
    for path in paths:
        try:
            return counter_per_dispatch(path, counter, kernel)[0]
        except SystemExit:
            continue
    return float("nan")


def cmd_counters(a):
    """Wait, VALU and LDS shares of the named kernels from two counter passes: fractions of
    wave cycles (SQ_WAIT_ANY, SQ_WAIT_INST_LDS, SQ_ACTIVE_INST_VALU over SQ_WAVE_CYCLES, all in
    the same quad-cycle units), LDS activity and bank conflicts over SQ_BUSY_CU_CYCLES, and
    instruction counts per dispatch (SQ_INSTS_VALU includes the MFMAs)."""
    lines = [f"# rocprofv3 counter summary: {a.title}", f"# commands (one run per pass): {a.cmd}",
             "# wait_any, wait_lds, valu_act: fractions of SQ_WAVE_CYCLES; lds_busy = SQ_LDS_IDX_ACTIVE /",
             "# SQ_BUSY_CU_CYCLES, bank_cf = SQ_LDS_BANK_CONFLICT / SQ_BUSY_CU_CYCLES; instruction counts",
             "# per dispatch (SQ_INSTS_VALU includes the MFMAs)", "#",
             f"{'kernel':28s} {'wait_any':>8s} {'wait_lds':>8s} {'valu_act':>8s} {'lds_busy':>8s} {'bank_cf':>8s} "
             f"{'valu_insts':>11s} {'mfma_insts':>11s} {'salu_insts':>11s}"]
    for spec in a.kernel:
        label, sub = spec.split("=", 1)
        g = lambda c: _per_dispatch_any(a.pmc, c, sub)
        wave = g("SQ_WAVE_CYCLES")
        busy = g("SQ_BUSY_CU_CYCLES")
        lines.append(f"{label[:28]:28s} {g('SQ_WAIT_ANY') / wave:8.2f} {g('SQ_WAIT_INST_LDS') / wave:8.2f} "
                     f"{g('SQ_ACTIVE_INST_VALU') / wave:8.2f} {g('SQ_LDS_IDX_ACTIVE') / busy:8.2f} "
                     f"{g('SQ_LDS_BANK_CONFLICT') / busy:8.3f} {g('SQ_INSTS_VALU'):11.4g} "
                     f"{g('SQ_INSTS_MFMA'):11.4g} {g('SQ_INSTS_SALU'):11.4g}")
    lines.append(f"source_hash: {source_hash()}")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("--stats", required=True)
    k.add_argument("--cmd", required=True)
    k.add_argument("--title", default="")
    k.add_argument("--top", type=int, default=8)
    k.add_argument("--bench-log", default="")
    k.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--pmc", required=True)
    m.add_argument("--kernel", required=True)
    m.add_argument("--cmd", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--title", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-kernel", default="elementwise")
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--title", default="")
    c = sub.add_parser("counters")
    c.add_argument("--pmc", action="append", required=True)
    c.add_argument("--kernel", action="append", required=True, help="label=kernel-name substring")
    c.add_argument("--title", default="")
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    {"kernels": cmd_kernels, "traffic": cmd_traffic, "mfma": cmd_mfma, "counters": cmd_counters}[a.what](a)


if __name__ == "__main__":
    main()
