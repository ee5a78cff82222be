"""Summaries of rocprofv3 CSV output for the library's kernels.

    python -m speculative_decoding_verification_06_amd.profile_summary trace DIR
        per-kernel call counts and durations from DIR/*kernel_trace.csv
    python -m speculative_decoding_verification_06_amd.profile_summary counters DIR [SUBSTRING]
        per-dispatch averages of every counter of a --pmc run, per kernel
        (kernels whose name contains SUBSTRING)
    python -m speculative_decoding_verification_06_amd.profile_summary traffic \\
        WORKLOAD FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR COPY_MIB OUT_JSON
        HBM bytes per weight-streaming GEMM launch from FETCH_SIZE and
        WRITE_SIZE runs (KiB per dispatch), each scaled by what the same
        counter reads for `bench.py --copy-probe COPY_MIB` (a kernel that
        reads and writes COPY_MIB MiB), written as the JSON record bench.py
        reads (tied to the hash of the GEMM kernels' sources)

Only the parsing and arithmetic live here; the counters come from
rocprofv3 runs of bench.py on the device.
"""

import collections
import csv
import glob
import json
import os
import sys

GEMM_PREFIXES = ("void sv::k_gemm_mfma", "void sv::k_gemm_wide", "void sv::k_gemm_fma")


def _rows(directory, suffix):
    out = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path) as f:
            out.extend(csv.DictReader(f))
    return out


def kernel_trace(directory):
    """{kernel name: [durations in us]} from a --kernel-trace run."""
    d = collections.defaultdict(list)
    for r in _rows(directory, "kernel_trace.csv"):
        d[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return d


def trace_table(directory, prefix="sv::"):
    d = kernel_trace(directory)
    total = sum(sum(v) for v in d.values())
    lines = ["| kernel | calls | avg us | median us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for name, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        if prefix not in name:
            continue
        short = name if len(name) <= 90 else name[:87] + "..."
        med = sorted(v)[len(v) // 2]
        lines.append(f"| `{short}` | {len(v)} | {sum(v) / len(v):.1f} | {med:.1f} | {min(v):.1f} | "
                     f"{max(v):.1f} | {100 * sum(v) / total:.2f} |")
    return "\n".join(lines)


def counter_per_dispatch(directory, counter):
    """{kernel name: [value per dispatch]} of one counter (summed over its
    instances within a dispatch)."""
    per = collections.defaultdict(float)
    names = {}
    for r in _rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        key = r["Dispatch_Id"]
        per[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key, v in per.items():
        out[names[key]].append(v)
    return out


def counter_table(directory, substring="sv::"):
    """{kernel: {counter: per-dispatch average}} and the dispatch counts."""
    names = set()
    for r in _rows(directory, "counter_collection.csv"):
        names.add(r["Counter_Name"])
    out, counts = {}, {}
    for cname in sorted(names):
        for kern, vals in counter_per_dispatch(directory, cname).items():
            if substring not in kern:
                continue
            out.setdefault(kern, {})[cname] = sum(vals) / len(vals)
            counts[kern] = len(vals)
    return out, counts


def _copy_scale(directory, counter, mib):
    vals = [v for name, vs in counter_per_dispatch(directory, counter).items()
            if "elementwise" in name or "mul" in name.lower() for v in vs]
    vals = [v for v in vals if v > 0.25 * mib * 1024]
    if not vals:
        raise SystemExit(f"no copy-probe dispatch in {directory}")
    return mib * 1024.0 / (sum(vals) / len(vals))


def traffic(workload, fetch_dir, write_dir, copy_fetch, copy_write, copy_mib, out_json):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from bench import source_hash
    fs = _copy_scale(copy_fetch, "FETCH_SIZE", copy_mib)
    ws = _copy_scale(copy_write, "WRITE_SIZE", copy_mib)
    fetch = counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = counter_per_dispatch(write_dir, "WRITE_SIZE")
    per_kernel, tot_bytes, tot_launch = {}, 0.0, 0
    for name in sorted(set(fetch) | set(write)):
        if not name.startswith(GEMM_PREFIXES):
            continue
        fr, wr = fetch.get(name, [0.0]), write.get(name, [0.0])
        rb = sum(fr) / len(fr) * 1024 * fs
        wb = sum(wr) / len(wr) * 1024 * ws
        n = len(fr)
        per_kernel[name] = {"read_bytes": rb, "write_bytes": wb, "launches": n,
                            "fetch_kib_raw": sum(fr) / len(fr), "write_kib_raw": sum(wr) / len(wr)}
        tot_bytes += (rb + wb) * n
        tot_launch += n
    rec = {"workload": workload, "source_hash": source_hash(),
           "hbm_bytes_per_launch": tot_bytes / tot_launch, "fetch_scale": fs, "write_scale": ws,
           "per_kernel": per_kernel}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "trace":
        print(trace_table(sys.argv[2]))
    elif len(sys.argv) in (3, 4) and sys.argv[1] == "counters":
        tab, counts = counter_table(sys.argv[2], sys.argv[3] if len(sys.argv) == 4 else "sv::")
        for kern, cs in tab.items():
            print(f"{kern} ({counts[kern]} dispatches)")
            for cname, v in cs.items():
                print(f"  {cname}: {v:.6g}")
    elif len(sys.argv) == 9 and sys.argv[1] == "traffic":
        rec = traffic(sys.argv[2], *sys.argv[3:7], float(sys.argv[7]), sys.argv[8])
        print(json.dumps({k: v for k, v in rec.items() if k != "per_kernel"}))
        for k, v in rec["per_kernel"].items():
            print(k, {kk: round(vv, 1) for kk, vv in v.items()})
    else:
        print(__doc__)
        sys.exit(2)
