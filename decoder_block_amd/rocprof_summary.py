"""Per-kernel summaries of rocprofv3 CSV output, as the tables in profiles/ give them.

    python -m decoder_block_amd.rocprof_summary trace <kernel_trace.csv> [--skip N] [--regex R] [--merge-grids R]
    python -m decoder_block_amd.rocprof_summary pmc <counter_collection.csv> [--skip N] [--regex R] [--merge-grids R]

``--skip N`` drops the first N dispatches of every kernel (the warm-up
launches), so the averages cover the same launches a timed run averages.

``trace``: dispatches, mean and median duration per kernel.

``pmc``: per kernel, the mean of every counter over the kept dispatches, and
where the counters are present:

* clock = GRBM_GUI_ACTIVE / 8 / duration (GRBM_GUI_ACTIVE adds one count per
  XCD per busy cycle, 8 XCDs);
* MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024): the
  counter adds one per busy matrix core per cycle, 256 CUs x 4 SIMDs;
* FETCH_SIZE and WRITE_SIZE in KiB per dispatch, as the counters read.
"""
from __future__ import annotations

import argparse
import collections
import csv
import re
import statistics

SIMDS = 256 * 4
XCDS = 8


_MANGLED_ARGS = {"DF16b": "bf16", "f": "float"}


def short_name(k: str) -> str:
    """Kernel name without namespaces and argument list, template arguments kept."""
    k = k.replace("llk::(anonymous namespace)::", "")
    k = re.sub(r"^void ", "", k)
    m = re.match(r"_ZN3llk12_GLOBAL__N_1(\d+)(\w+)", k)
    if m:  # mangled: length-prefixed name, then I<args>E
        n = int(m.group(1))
        name, tail = m.group(2)[:n], m.group(2)[n:]
        args = []
        if tail.startswith("I"):
            body = tail[1:tail.find("EE") + 1] if "EE" in tail else tail[1:]
            for t in re.finditer(r"DF16b|Li(\d+)E|f", body):
                args.append(t.group(1) if t.group(1) else _MANGLED_ARGS[t.group(0)])
        return name + (f"<{', '.join(args)}>" if args else "")
    return re.sub(r"\((?!anonymous).*$", "", k)


def _keep(rows, skip, regex, merge):
    """Group rows by kernel and grid size in dispatch order (the same kernel at
    prefill and decode sizes are separate entries; kernels matching `merge`,
    whose grid follows the data, by name alone); drop the first `skip`
    dispatches of each."""
    by = collections.OrderedDict()
    for r in rows:
        name = r["Kernel_Name"]
        if regex and not re.search(regex, name):
            continue
        grid = r.get("Grid_Size") or r.get("Grid_Size_X")
        key = short_name(name) if merge and re.search(merge, name) else f"{short_name(name)} grid={grid}"
        by.setdefault(key, collections.OrderedDict()).setdefault(int(r["Dispatch_Id"]), []).append(r)
    return {k: list(d.values())[skip:] for k, d in by.items()}


def trace(path: str, skip: int, regex: str | None, merge: str | None) -> None:
    rows = list(csv.DictReader(open(path)))
    print("| kernel | dispatches kept | mean us | median us |")
    print("|---|---|---|---|")
    for name, ds in _keep(rows, skip, regex, merge).items():
        if not ds:
            continue
        us = [(int(d[0]["End_Timestamp"]) - int(d[0]["Start_Timestamp"])) * 1e-3 for d in ds]
        print(f"| {name} | {len(us)} | {statistics.mean(us):.1f} | {statistics.median(us):.1f} |")


def pmc(path: str, skip: int, regex: str | None, merge: str | None) -> None:
    rows = list(csv.DictReader(open(path)))
    for name, ds in _keep(rows, skip, regex, merge).items():
        if not ds:
            continue
        counters = collections.defaultdict(list)
        durs = []
        for d in ds:
            durs.append((int(d[0]["End_Timestamp"]) - int(d[0]["Start_Timestamp"])) * 1e-9)
            for r in d:
                counters[r["Counter_Name"]].append(float(r["Counter_Value"]))
        avg = {c: statistics.mean(v) for c, v in counters.items()}
        dur = statistics.mean(durs)
        out = [f"{name}: n={len(ds)} mean {dur * 1e6:.1f} us"]
        if "GRBM_GUI_ACTIVE" in avg:
            cyc = avg["GRBM_GUI_ACTIVE"] / XCDS
            out.append(f"clock {cyc / dur / 1e9:.2f} GHz")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                out.append(f"MFMA busy {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * SIMDS) * 100:.1f}%")
        for c in sorted(avg):
            if c != "GRBM_GUI_ACTIVE":
                out.append(f"{c} {avg[c]:.6g}")
        print("; ".join(out))


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=("trace", "pmc"))
    ap.add_argument("csv")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--regex", default=None, help="keep only kernels whose names match")
    ap.add_argument("--merge-grids", default=None, help="kernels whose names match are grouped by name alone")
    a = ap.parse_args()
    (trace if a.mode == "trace" else pmc)(a.csv, a.skip, a.regex, a.merge_grids)


if __name__ == "__main__":
    main()
