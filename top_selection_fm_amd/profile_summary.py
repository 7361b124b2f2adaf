"""Text summaries of rocprofv3 CSV output, as kept under profiles/.

    python -m top_selection_fm_amd.profile_summary stats  TRACE_DIR  [--cmd "..."]
    python -m top_selection_fm_amd.profile_summary hbm    FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR [--cmd "..."]
    python -m top_selection_fm_amd.profile_summary sq     TRACE_DIR PASS_DIR [PASS_DIR ...] --kernel NAME[@GRID] [--cmd "..."]
    python -m top_selection_fm_amd.profile_summary traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR --kernel NAME[@GRID] [...] [--cmd "..."]

Each DIR is a rocprofv3 output directory written with --output-format csv (the
*_kernel_trace.csv or *_counter_collection.csv file inside it is found by suffix).

* stats: per kernel (name without its argument list, grid size): dispatches, average, median,
  minimum and maximum duration from the kernel trace.
* hbm: FETCH_SIZE and WRITE_SIZE per dispatch (KiB as counted), scaled to bytes by what the
  same counters read for a plain 1 GiB device copy (a copy reads and writes 2^30 bytes each).
* sq: SQ counters of one kernel (median over its dispatches) with the utilisations they give:
  SQ_VALU_MFMA_BUSY_CYCLES and SQ_CYCLES are per SIMD (1,024 SIMDs); the other SQ_* counters
  are summed per shader engine in quad-cycles (4 cycles), so they are normalised by
  4 / (1,024 x kernel cycles); kernel cycles = the trace's median duration x 2.4 GHz.
* traffic: the HBM bytes per launch of the named kernels (summed over them), in the
  key: value form bench.py reads, with the digest of the kernel sources they were taken on.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys
from collections import defaultdict

CLOCK_HZ = 2.4e9
SIMDS = 1024
COPY_BYTES = 1 << 30


def _csv(d: str, suffix: str) -> str:
    m = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not m:
        sys.exit(f"no *{suffix} under {d}")
    return m[0]


def short_name(n: str) -> str:
    n = n.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth, out = 0, []
    for ch in n:                      # drop the argument list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    s = "".join(out).strip()
    return s[4:] if s.startswith("fm::") else s


def kernel_sources_digest(root: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(root, "top_selection_fm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def trace(d: str):
    rows = defaultdict(list)
    for r in csv.DictReader(open(_csv(d, "kernel_trace.csv"))):
        key = (short_name(r["Kernel_Name"]), int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0))
        rows[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    return rows


def counters(d: str):
    per = defaultdict(lambda: defaultdict(float))       # (name, grid, dispatch) -> counter -> v
    for r in csv.DictReader(open(_csv(d, "counter_collection.csv"))):
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]), int(r["Dispatch_Id"]))
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
    return per


def copy_factor(d: str, counter: str) -> float:
    vals = [v[counter] for (n, g, _), v in counters(d).items() if "copyBuffer" in n or "copy" in n.lower()]
    big = max(vals)                                      # KiB counted for the 1 GiB copies
    return COPY_BYTES / 1024.0 / big


def cmd_stats(a):
    out = [f"# rocprofv3 kernel trace: duration per dispatch (us), MI355X",
           f"# command: {a.cmd}" if a.cmd else "# command: (not given)",
           f"# kernel_sources: {kernel_sources_digest(a.root)}",
           f"{'kernel':58s} {'grid':>9s} {'n':>4s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for (n, g), ds in sorted(trace(a.dirs[0]).items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{n[:58]:58s} {g:9d} {len(ds):4d} {statistics.mean(ds):9.1f} "
                   f"{statistics.median(ds):9.1f} {min(ds):9.1f} {max(ds):9.1f}")
    print("\n".join(out))


def _hbm_rows(a):
    fetch, write = counters(a.dirs[0]), counters(a.dirs[1])
    ff, wf = copy_factor(a.dirs[2], "FETCH_SIZE"), copy_factor(a.dirs[3], "WRITE_SIZE")
    agg = defaultdict(lambda: [0, 0.0, 0.0])
    for key, v in fetch.items():
        w = write.get(key, {}).get("WRITE_SIZE", 0.0)
        t = agg[key[:2]]
        t[0] += 1
        t[1] += v["FETCH_SIZE"]
        t[2] += w
    return agg, ff, wf


def cmd_hbm(a):
    agg, ff, wf = _hbm_rows(a)
    out = ["# rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch (KiB as counted, then scaled bytes), MI355X",
           f"# command: {a.cmd}" if a.cmd else "# command: (not given)",
           f"# calibration: a 1 GiB device copy counts {COPY_BYTES / 1024 / ff:.0f} KiB FETCH_SIZE and "
           f"{COPY_BYTES / 1024 / wf:.0f} KiB WRITE_SIZE -> factors {ff:.4f} / {wf:.4f}",
           f"# kernel_sources: {kernel_sources_digest(a.root)}",
           f"{'kernel':58s} {'grid':>9s} {'n':>4s} {'fetch_KiB':>11s} {'write_KiB':>11s} {'hbm_MB':>9s}"]
    for (n, g), (cnt, fk, wk) in sorted(agg.items()):
        fk, wk = fk / cnt, wk / cnt
        out.append(f"{n[:58]:58s} {g:9d} {cnt:4d} {fk:11.1f} {wk:11.1f} "
                   f"{(fk * ff + wk * wf) * 1024 / 1e6:9.2f}")
    print("\n".join(out))


def cmd_traffic(a):
    agg, ff, wf = _hbm_rows(a)
    tot, parts = 0.0, []
    want = [(k.split("@")[0], int(k.split("@")[1]) if "@" in k else None) for k in a.kernel]
    for (n, g), (cnt, fk, wk) in agg.items():
        if any(k == n and (kg is None or kg == g) for k, kg in want):
            b = (fk / cnt * ff + wk / cnt * wf) * 1024
            parts.append(f"{n} (grid {g}): {b:.0f}")
            tot += b
    if not parts:
        sys.exit("no dispatch of the named kernels")
    print("# HBM bytes per launch of the named kernels, from rocprofv3 FETCH_SIZE / WRITE_SIZE "
          "scaled by a 1 GiB device copy (factors %.4f / %.4f), MI355X" % (ff, wf))
    print(f"# command: {a.cmd}" if a.cmd else "# command: (not given)")
    for p in parts:
        print(f"# {p}")
    print(f"kernel_sources: {kernel_sources_digest(a.root)}")
    print(f"hbm_bytes_per_launch: {tot:.0f}")


def cmd_sq(a):
    # NAME or NAME@GRID: the dispatches of one kernel, or of one kernel at one grid size
    name, grid = (a.kernel[0].split("@")[0], int(a.kernel[0].split("@")[1])) if "@" in a.kernel[0] \
        else (a.kernel[0], None)
    pick = lambda n, g: n == name and (grid is None or g == grid)
    ds = [d for (n, g), v in trace(a.dirs[0]).items() if pick(n, g) for d in v]
    if not ds:
        sys.exit("kernel not in the trace")
    us = statistics.median(ds)
    cyc = us * 1e-6 * CLOCK_HZ
    vals = {}
    for d in a.dirs[1:]:
        per = counters(d)
        keys = [k for k in per if pick(k[0], k[1])]
        for c in per[keys[0]]:
            vals[c] = statistics.median(per[k][c] for k in keys)
    q = lambda c: 4 * vals[c] / (SIMDS * cyc)
    what = name + (f" (grid {grid})" if grid is not None else "")
    out = [f"# rocprofv3 SQ counters of {what}, median over its dispatches, MI355X",
           f"# command: {a.cmd}" if a.cmd else "# command: (not given)",
           f"# kernel_sources: {kernel_sources_digest(a.root)}",
           f"# kernel time: median {us:.1f} us over {len(ds)} traced dispatches = {cyc:.4g} cycles at 2.4 GHz",
           "# normalisation: per-SIMD counters / (1,024 SIMDs x cycles); per-SE quad-cycle counters x 4 / (1,024 x cycles)"]
    for c in sorted(vals):
        out.append(f"{c:32s} {vals[c]:.6g}")
    out.append("# derived")
    out.append(f"mfma_busy_fraction:        {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * cyc):.3f}")
    if "SQ_INSTS_VALU_MFMA_MOPS_F8" in vals or "SQ_INSTS_VALU_MFMA_MOPS_BF16" in vals:
        f8 = vals.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) * 512
        b16 = vals.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        if f8:
            out.append(f"mfma_fp8_pflops:            {f8 / (us * 1e-6) / 1e15:.3f} (of 5.0 dense: {f8 / (us * 1e-6) / 5e15:.3f})")
        if b16:
            out.append(f"mfma_bf16_pflops:           {b16 / (us * 1e-6) / 1e15:.3f} (of 2.5 dense: {b16 / (us * 1e-6) / 2.5e15:.3f})")
    for c, lab in (("SQ_ACTIVE_INST_VALU", "valu_busy_fraction"), ("SQ_ACTIVE_INST_LDS", "lds_inst_fraction"),
                   ("SQ_ACTIVE_INST_ANY", "any_inst_fraction"), ("SQ_WAVE_CYCLES", "resident_waves_per_simd"),
                   ("SQ_WAIT_INST_ANY", "waves_waiting_to_issue_per_simd")):
        if c in vals:
            out.append(f"{lab + ':':27s} {q(c):.3f}")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in vals:
        out.append(f"{'mfma_valu_coexec_fraction:':27s} {vals['SQ_VALU_MFMA_COEXEC_CYCLES'] / (SIMDS * cyc):.3f}")
    if "SQ_LDS_BANK_CONFLICT" in vals:
        out.append(f"{'lds_bank_conflict_per_cu_cycle:':27s} {vals['SQ_LDS_BANK_CONFLICT'] / (256 * cyc):.4f}")
    for c in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS"):
        if c in vals:
            out.append(f"{c.lower() + '_per_mfma:':27s} {vals[c] / vals['SQ_INSTS_MFMA']:.2f}")
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["stats", "hbm", "sq", "traffic"])
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--kernel", action="append", default=[])
    ap.add_argument("--cmd", default="")
    ap.add_argument("--root", default=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "hbm": cmd_hbm, "sq": cmd_sq, "traffic": cmd_traffic}[a.what](a)


if __name__ == "__main__":
    main()
