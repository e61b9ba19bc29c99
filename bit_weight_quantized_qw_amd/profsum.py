"""Summaries of rocprofv3 output for the profile notes.

    python -m bit_weight_quantized_qw_amd.profsum kt DIR [FILTER ...]
        kernel-trace statistics of the kernels whose name contains one of
        the FILTER strings, per kernel and grid size (from
        run_kernel_trace.csv under DIR), as a table (calls, average / min /
        max microseconds, resources).
    python -m bit_weight_quantized_qw_amd.profsum pmc DIR [DIR ...] --kernel SUB [--grid G]
        per-dispatch counter values (run_counter_collection.csv under each
        DIR, one counter pass per DIR) of the kernels whose name contains SUB
        (and whose grid size in threads is G, when given), averaged over the
        dispatches, one line per counter.

Reads rocprofv3's CSV files only; no GPU is touched.
"""

import csv
import collections
import os
import statistics
import sys


def _strip_args(name):
    """Kernel name without its trailing parameter list."""
    if not name.endswith(")"):
        return name
    depth = 0
    for i in range(len(name) - 1, -1, -1):
        depth += name[i] == ")"
        depth -= name[i] == "("
        if depth == 0:
            return name[:i]
    return name


def _find(root, fname):
    for d, _, files in os.walk(root):
        if fname in files:
            return os.path.join(d, fname)
    raise FileNotFoundError(f"{fname} under {root}")


def kernel_stats(root, filters=()):
    """[(name, grid threads, workgroup threads, LDS bytes, VGPRs, AGPRs,
    scratch, calls, avg us, min us, max us)] from the dispatch trace."""
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(_find(root, "run_kernel_trace.csv"))):
        name = _strip_args(r["Kernel_Name"])
        if filters and not any(f in name for f in filters):
            continue
        key = (name, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]), int(r["LDS_Block_Size"]),
               int(r["VGPR_Count"]), int(r["Accum_VGPR_Count"]), int(r["Scratch_Size"]))
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return [k + (len(v), statistics.mean(v), min(v), max(v)) for k, v in sorted(groups.items())]


def counters(roots, sub, grid=None):
    vals = collections.defaultdict(list)
    for root in roots:
        for r in csv.DictReader(open(_find(root, "run_counter_collection.csv"))):
            if sub not in r["Kernel_Name"]:
                continue
            if grid is not None and int(r["Grid_Size"]) != grid:
                continue
            vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: (statistics.mean(v), len(v)) for k, v in vals.items()}


def main(argv):
    if len(argv) >= 2 and argv[0] == "kt":
        print("| kernel | grid | wg | LDS B | VGPR | AGPR | scratch | calls | avg us | min us | max us |")
        print("|---|---|---|---|---|---|---|---|---|---|---|")
        for n, g, wg, lds, v, av, sc, c, a, lo, hi in kernel_stats(argv[1], argv[2:]):
            print(f"| `{n}` | {g} | {wg} | {lds} | {v} | {av} | {sc} | {c} | {a:.3f} | {lo:.3f} | {hi:.3f} |")
        return 0
    if len(argv) >= 2 and argv[0] == "pmc":
        roots, sub, grid = [], None, None
        it = iter(argv[1:])
        for a in it:
            if a == "--kernel":
                sub = next(it)
            elif a == "--grid":
                grid = int(next(it))
            else:
                roots.append(a)
        for k, (v, n) in sorted(counters(roots, sub, grid).items()):
            print(f"{k}: {v:.6g} (mean of {n} dispatches)")
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
