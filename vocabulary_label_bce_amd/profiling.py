"""Turns rocprofv3 CSV output into the short text summaries kept under profiles/.

  python -m vocabulary_label_bce_amd.profiling stats --csv <dir>/run_kernel_stats.csv --out <file.md>
      --title "..." --command "..."
  python -m vocabulary_label_bce_amd.profiling traffic --fetch <dir>/run_counter_collection.csv
      --write <dir>/run_counter_collection.csv --kernel-regex k_rows< --name rows_sweep --workload sasrec876k
      --copy-regex neg_kernel --copy-bytes N --out <file.json> --command "..."

  python -m vocabulary_label_bce_amd.profiling counters --csv <pass1>/run_counter_collection.csv [--csv ...]
      --kernel rows_sweep=k_rowsI --kernel items_sweep=k_itemsI --out <file.md> --title "..." --command "..."

`counters` averages SQ/GRBM counters per dispatch of each named kernel over the given passes and derives the
MFMA pipe's busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over SIMDs x GRBM_GUI_ACTIVE per XCD, i.e. over the
dispatch's shader-clock cycles), cycles per MFMA, VALU/MFMA co-execution and instructions per MFMA.

`traffic` reads one FETCH_SIZE pass and one WRITE_SIZE pass (KiB per dispatch). It scales each counter by
what the same counter read for a plain copy kernel that moved a known number of bytes in the same run, so the
result is in HBM bytes per launch. The JSON records a digest of the sources that define the two sweep kernels
(sweep.hip and the shared layouts in common.h), and a reader treats the figure as stale once they differ.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


SWEEP_SOURCES = ("common.h", "sweep.hip")


def _code_only(text: str) -> str:
    """Source text without comments and with runs of whitespace collapsed, so that edits to comments alone do
    not mark measured counters as stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    """sha256 over the code of the sweep kernels' sources (file names and comment-free contents)."""
    h = hashlib.sha256()
    for f in SWEEP_SOURCES:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def _counter_rows(path, counter):
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                yield row["Kernel_Name"], float(row["Counter_Value"]), int(row["Dispatch_Id"])


def _per_dispatch(path, counter, regex):
    """Counter value of each dispatch whose kernel name matches regex (summed over duplicate records)."""
    pat = re.compile(regex)
    acc = {}
    for name, val, disp in _counter_rows(path, counter):
        if pat.search(name):
            acc[disp] = acc.get(disp, 0.0) + val
    return [acc[k] for k in sorted(acc)]


def traffic(fetch_csv, write_csv, kernel_regex, copy_regex, copy_bytes):
    fk = _per_dispatch(fetch_csv, "FETCH_SIZE", kernel_regex)
    wk = _per_dispatch(write_csv, "WRITE_SIZE", kernel_regex)
    fc = _per_dispatch(fetch_csv, "FETCH_SIZE", copy_regex)
    wc = _per_dispatch(write_csv, "WRITE_SIZE", copy_regex)
    if not (fk and wk and fc and wc):
        raise SystemExit(f"missing dispatches: kernel fetch {len(fk)} write {len(wk)}, copy fetch {len(fc)} "
                         f"write {len(wc)}")
    # copy kernel: reads copy_bytes and writes copy_bytes
    f_fetch = copy_bytes / (statistics.median(fc) * 1024.0)
    f_write = copy_bytes / (statistics.median(wc) * 1024.0)
    fetch_b = statistics.median(fk) * 1024.0 * f_fetch
    write_b = statistics.median(wk) * 1024.0 * f_write
    return {
        "fetch_kib_per_dispatch": [round(x, 1) for x in fk],
        "write_kib_per_dispatch": [round(x, 1) for x in wk],
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": [round(x, 1) for x in fc],
        "copy_write_kib": [round(x, 1) for x in wc],
        "scale_fetch": f_fetch,
        "scale_write": f_write,
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b,
    }


def counter_means(paths, regex):
    """{counter: mean per dispatch} for dispatches whose kernel name matches regex, and {counter: mean duration
    in ns of the dispatches that carried it} (each pass times its own dispatches). Records of one dispatch and
    counter are summed first."""
    pat = re.compile(regex)
    per, dur = {}, {}
    for path in paths:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if not pat.search(row["Kernel_Name"]):
                    continue
                key = (path, int(row["Dispatch_Id"]))
                c = row["Counter_Name"]
                per.setdefault(c, {}).setdefault(key, 0.0)
                per[c][key] += float(row["Counter_Value"])
                dur.setdefault(c, {})[key] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    means = {c: statistics.mean(v.values()) for c, v in per.items()}
    durs = {c: statistics.mean(v.values()) for c, v in dur.items()}
    return means, durs


def counter_report(means, durs, simds=1024, xcds=8):
    """Derived figures from counter_means (figures whose counters are missing are left out). The shader clock
    comes from GRBM_GUI_ACTIVE (cycles summed over the XCDs) and its own dispatches' durations; the MFMA busy
    fraction divides SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) by SIMDs x that clock x its own dispatches'
    duration."""
    g = means.get
    busy, mfma, gui = g("SQ_VALU_MFMA_BUSY_CYCLES"), g("SQ_INSTS_MFMA"), g("GRBM_GUI_ACTIVE")
    d = {}
    clock = gui / xcds / durs["GRBM_GUI_ACTIVE"] if gui else None  # cycles per ns = GHz
    if clock:
        d["shader clock during the dispatch, GHz (GRBM_GUI_ACTIVE per XCD / duration)"] = clock
    if busy and clock:
        d["MFMA pipe busy fraction (SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x clock x duration))"] = \
            busy / (simds * clock * durs["SQ_VALU_MFMA_BUSY_CYCLES"])
    if busy:
        d["dispatch duration under counter collection, ms"] = durs["SQ_VALU_MFMA_BUSY_CYCLES"] / 1e6
    if busy and mfma:
        d["MFMA busy cycles per MFMA instruction"] = busy / mfma
    if busy and g("SQ_VALU_MFMA_COEXEC_CYCLES"):
        d["fraction of MFMA busy cycles co-executing with VALU"] = g("SQ_VALU_MFMA_COEXEC_CYCLES") / busy
    if mfma:
        if g("SQ_INSTS_VALU") is not None:
            d["VALU instructions per MFMA (SQ_INSTS_VALU counts MFMA too; excluded)"] = (g("SQ_INSTS_VALU") - mfma) / mfma
        for c in ("SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_BRANCH"):
            if g(c) is not None:
                d[f"{c} per MFMA"] = g(c) / mfma
    if g("SQ_WAVE_CYCLES"):
        for c in ("SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"):
            if g(c) is not None:
                d[f"{c} / SQ_WAVE_CYCLES"] = g(c) / g("SQ_WAVE_CYCLES")
    if g("SQ_LDS_BANK_CONFLICT") is not None and g("SQ_INSTS_LDS"):
        d["LDS bank-conflict cycles per LDS instruction"] = g("SQ_LDS_BANK_CONFLICT") / g("SQ_INSTS_LDS")
    return d


def stats_table(path, top=16):
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[3])
    out = ["| kernel | calls | avg us | % of GPU time |", "|---|---|---|---|"]
    for name, calls, avg, pct in rows[:top]:
        out.append(f"| `{name[:80]}` | {calls} | {avg:.1f} | {pct:.2f} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    c = sub.add_parser("counters")
    c.add_argument("--csv", action="append", required=True)
    c.add_argument("--kernel", action="append", required=True, help="name=regex")
    c.add_argument("--out", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel-regex", required=True)
    t.add_argument("--name", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-regex", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", action="append", default=[])
    a = ap.parse_args()
    if a.cmd == "counters":
        kernels = [k.split("=", 1) for k in a.kernel]
        md = {name: counter_means(a.csv, rx) for name, rx in kernels}
        means = {n: m for n, (m, _) in md.items()}
        names = [n for n, _ in kernels]
        txt = [f"# {a.title}", "", "Commands (repo root, on the MI355X box; one counter pass each):", "", "```"]
        txt += a.command + ["```", "", "Mean per dispatch of each kernel:", "",
                            "| counter | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
        counters = sorted({c for m in means.values() for c in m})
        for cn in counters:
            txt.append(f"| {cn} | " + " | ".join(f"{means[n].get(cn, float('nan')):.4g}" for n in names) + " |")
        reps = {n: counter_report(*md[n]) for n in names}
        keys = list(dict.fromkeys(k for r in reps.values() for k in r))
        txt += ["", "Derived:", "", "| figure | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
        for k in keys:
            txt.append(f"| {k} | " + " | ".join(f"{reps[n][k]:.3f}" if k in reps[n] else "" for n in names) + " |")
        txt.append("")
        if a.note:
            txt += [a.note, ""]
        with open(a.out, "w") as f:
            f.write("\n".join(txt))
    elif a.cmd == "stats":
        txt = [f"# {a.title}", "", "Command (repo root, on the MI355X box):", "", "```", a.command, "```", "",
               f"Source: `{os.path.basename(a.csv)}`.", "", stats_table(a.csv), ""]
        if a.note:
            txt += [a.note, ""]
        with open(a.out, "w") as f:
            f.write("\n".join(txt))
    else:
        d = traffic(a.fetch, a.write, a.kernel_regex, a.copy_regex, a.copy_bytes)
        d.update({"kernel": a.name, "kernel_regex": a.kernel_regex, "workload": a.workload,
                  "source_digest": source_digest(), "commands": a.command})
        with open(a.out, "w") as f:
            json.dump(d, f, indent=1)
        print(json.dumps({k: d[k] for k in ("kernel", "bytes_per_launch", "scale_fetch", "scale_write")}))


if __name__ == "__main__":
    main()
