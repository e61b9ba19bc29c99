"""Summaries of rocprofv3 output for the profile notes.

    python -m bit_weight_quantized_qw_amd.profsum kt DIR [FILTER ...]
        kernel-trace statistics of the kernels whose name contains one of
        the FILTER strings, per kernel and grid size (from
        run_kernel_trace.csv under DIR), as a table (calls, average / min /
        max microseconds, resources).
    python -m bit_weight_quantized_qw_amd.profsum compact DIR OUT.json
        the counter values of one --pmc run (run_counter_collection.csv under
        DIR) summed per kernel, grid size and counter, with the number of
        dispatches: a few KB in place of one CSV row per dispatch.
    python -m bit_weight_quantized_qw_amd.profsum pmc SRC [SRC ...] --kernel SUB [--grid G]
        per-dispatch counter values (SRC: a --pmc output directory or a
        compacted file, one counter pass each) of the kernels whose name
        contains SUB (and whose grid size in threads is G, when given),
        averaged over the dispatches, one line per counter.
    python -m bit_weight_quantized_qw_amd.profsum traffic DIR [--out FILE]
        HBM bytes per call of each kernel that bench.py times, from compacted
        FETCH_SIZE and WRITE_SIZE passes, into FILE (profiles/traffic.json by
        default). DIR holds, per workload W of the table below, W.json (the
        bench.py line of a plain run on the same box: the algorithmic bytes
        per call, or of flops and bytes for the GEMM), W_FETCH_SIZE.json and
        W_WRITE_SIZE.json, and the same two
        for the copy_calib workload: each counter is scaled by what it reads
        for that plain 1 GiB read + 1 GiB write, so a byte counted is a byte
        moved.

Reads rocprofv3's CSV files (or the compacted files) only; no GPU is touched.
"""

import collections
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_C = "bit_weight_quantized_qw_amd/csrc/"
_MC = [_C + "gemv2_mfma.hip", _C + "gemv2.hip", _C + "qw_internal.h"]
_VALU = [_C + "gemv2_kernel.h", _C + "gemv2_b1.hip", _C + "gemv2.hip", _C + "qw_internal.h"]
_NF4 = [_C + "gemv_nf4.hip", _C + "qw_internal.h"]
_INT4 = [_C + "gemv2_mfma.hip", _C + "gemv_int4.hip", _C + "qw_internal.h"]
_PF = [_C + "prefill.hip", _C + "qw_internal.h"]

# workload -> bench kernel -> (dispatches of one call: [(name substring, grid
# in threads or None)], dispatches per call, sources hashed). The grids tell
# apart the 32B stack's stages on a 256-CU part (q/k/v: 384 workgroups of
# 512, o: 256, the merged gate/up: 512).
TRAFFIC = {
    "llama7b_mlp_up_gemv": {"qgemv_nf4": ([("gemv_nf4_kernel", None)], 1, _NF4),
                            "qgemv_2bit": ([("gemv2m::kernel", None)], 1, _MC)},
    "decode14b_b1": {"qgemv_2bit": ([("gemv2m::kernel", None)], 1, _MC)},
    "decode14b_b8": {"qgemv_2bit": ([("gemv2m::kernel", None)], 1, _MC)},
    "down70b_b1": {"qgemv_2bit": ([("gemv2m::kernel", None)], 1, _MC)},
    # seven K parts: two grouped launches of the part kernel and the reduction
    "down70b_b8": {"qgemv_2bit": ([("gemv2m::kernel", None), ("split_reduce_kernel", None)], 3, _MC)},
    "decode32b_stack": {"qkv": ([("gemv2m::kernel", 196608)], 1, _MC),
                        "o": ([("gemv2m::kernel", 131072)], 1, _MC),
                        "gateup": ([("gemv2m::kernel", 262144)], 1, _MC),
                        "down": ([("gemv2::kernel", None)], 1, _VALU)},
    # the matrix-core INT4 kernel (K a multiple of 512)
    "decode14b_int4_b1": {"qgemv_int4": ([("gemv2m::kernel_int4", None)], 1, _INT4)},
    "decode14b_int4_b8": {"qgemv_int4": ([("gemv2m::kernel_int4", None)], 1, _INT4)},
    # 256-wide column tiles, then 128-wide ones for the last columns
    "prefill70b_2bit": {"qgemm_prefill": ([("prefill_w_kernel", None)], 2, _PF)},
    "prefill70b_nf4": {"qgemm_prefill": ([("prefill_w_kernel", None)], 2, _PF)},
    "prefill70b_int4": {"qgemm_prefill": ([("prefill_w_kernel", None)], 2, _PF)},
}
CALIB_KERNEL = "AUnaryFunctor"  # torch's elementwise kernel of copy_calib
CALIB_BYTES = 1 << 30


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


def compact(root):
    """{"rows": [{kernel, grid, counter, n, sum}]} of one --pmc run."""
    acc = collections.defaultdict(lambda: [0, 0.0])
    for r in csv.DictReader(open(_find(root, "run_counter_collection.csv"))):
        k = (_strip_args(r["Kernel_Name"]), int(r["Grid_Size"]), r["Counter_Name"])
        acc[k][0] += 1
        acc[k][1] += float(r["Counter_Value"])
    return {"rows": [{"kernel": k, "grid": g, "counter": c, "n": n, "sum": s}
                     for (k, g, c), (n, s) in sorted(acc.items())]}


def _rows(src):
    if os.path.isdir(src):
        return compact(src)["rows"]
    return json.load(open(src))["rows"]


def counters(srcs, sub, grid=None):
    """{counter: (mean per dispatch, dispatches)} of the matching kernels."""
    tot = collections.defaultdict(lambda: [0, 0.0])
    for src in srcs:
        for r in _rows(src):
            if sub in r["kernel"] and (grid is None or r["grid"] == grid):
                tot[r["counter"]][0] += r["n"]
                tot[r["counter"]][1] += r["sum"]
    return {c: (s / n, n) for c, (n, s) in tot.items() if n}


def _per_call(rows, counter, parts, per_call):
    """Counter total of one call: the matching dispatches' sum divided by
    the number of calls they make up."""
    n, s, names = 0, 0.0, set()
    for r in rows:
        if r["counter"] == counter and any(p in r["kernel"] and (g is None or r["grid"] == g) for p, g in parts):
            n += r["n"]
            s += r["sum"]
            names.add(r["kernel"])
    if n == 0 or n % per_call:
        raise ValueError(f"{counter}: {n} dispatches of {parts} is not a whole number of calls")
    return s / (n // per_call), n // per_call, sorted(names)


def traffic(d, out):
    def load(name):
        return _rows(os.path.join(d, name))
    kib = CALIB_BYTES / 1024
    cf = counters([os.path.join(d, "copy_calib_FETCH_SIZE.json")], CALIB_KERNEL)["FETCH_SIZE"][0]
    cw = counters([os.path.join(d, "copy_calib_WRITE_SIZE.json")], CALIB_KERNEL)["WRITE_SIZE"][0]
    fetch_scale, write_scale = kib / cf, kib / cw
    t = {"_about": "HBM bytes per call from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (one counter per run, "
                   "KiB per dispatch), each scaled by what the same counter reads for a plain 1 GiB read + "
                   "1 GiB write elementwise kernel (bench.py --workload copy_calib); made by "
                   "`python -m bit_weight_quantized_qw_amd.profsum traffic`. 'sha256' covers the kernel's "
                   "sources when the counters were taken; bench.py reports null traffic when they differ.",
         "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5)}
    for wl, kernels in TRAFFIC.items():
        fn = os.path.join(d, f"{wl}_FETCH_SIZE.json")
        if not os.path.exists(fn):
            continue
        fr, wr = load(f"{wl}_FETCH_SIZE.json"), load(f"{wl}_WRITE_SIZE.json")
        bench = json.load(open(os.path.join(d, f"{wl}.json")))
        for bk, (parts, per_call, srcs) in kernels.items():
            fk, calls, names = _per_call(fr, "FETCH_SIZE", parts, per_call)
            wk, _, _ = _per_call(wr, "WRITE_SIZE", parts, per_call)
            fb, wb = fk * 1024 * fetch_scale, wk * 1024 * write_scale
            kb = bench["kernels"][bk]
            alg = kb.get("bytes", kb["amount"])
            h = hashlib.sha256()
            for f in srcs:
                h.update(open(os.path.join(ROOT, f), "rb").read())
            t.setdefault(wl, {})[bk] = {
                "bytes": int(round(fb + wb)), "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
                "fetch_kib_raw": round(fk, 2), "write_kib_raw": round(wk, 2), "calls": calls,
                "algorithmic_bytes": alg, "ratio": round((fb + wb) / alg, 4),
                "kernel": " + ".join(names), "sources": srcs, "sha256": h.hexdigest()}
    with open(out, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    return t


def main(argv):
    if len(argv) >= 2 and argv[0] == "kt":
        print("| kernel | grid | wg | LDS B | VGPR | AGPR | scratch | calls | avg us | min us | max us |")
        print("|---|---|---|---|---|---|---|---|---|---|---|")
        for n, g, wg, lds, v, av, sc, c, a, lo, hi in kernel_stats(argv[1], argv[2:]):
            print(f"| `{n}` | {g} | {wg} | {lds} | {v} | {av} | {sc} | {c} | {a:.3f} | {lo:.3f} | {hi:.3f} |")
        return 0
    if len(argv) == 3 and argv[0] == "compact":
        with open(argv[2], "w") as f:
            json.dump(compact(argv[1]), f, indent=0)
        return 0
    if len(argv) >= 2 and argv[0] == "pmc":
        srcs, sub, grid = [], None, None
        it = iter(argv[1:])
        for a in it:
            if a == "--kernel":
                sub = next(it)
            elif a == "--grid":
                grid = int(next(it))
            else:
                srcs.append(a)
        for k, (v, n) in sorted(counters(srcs, sub or "", grid).items()):
            print(f"{k}: {v:.6g} (mean of {n} dispatches)")
        return 0
    if len(argv) >= 2 and argv[0] == "traffic":
        out = os.path.join(ROOT, "profiles", "traffic.json")
        if "--out" in argv:
            out = argv[argv.index("--out") + 1]
        t = traffic(argv[1], out)
        for wl, ks in t.items():
            if isinstance(ks, dict):
                for bk, e in ks.items():
                    print(f"{wl} {bk}: {e['bytes']} B per call, {e['ratio']} x algorithmic")
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
