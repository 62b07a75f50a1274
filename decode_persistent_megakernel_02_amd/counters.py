"""HBM bytes per launch from rocprofv3 counter runs.

rocprofv3 --pmc FETCH_SIZE (then, in a run of its own, WRITE_SIZE) reports
KiB per dispatch.  Each counter is scaled by what it reads for a plain
device-to-device copy of known size (`bench.py --copy-probe MIB`), so the
result is in bytes that moved, whatever the counter's own unit convention.

    python -m decode_persistent_megakernel_02_amd.counters \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-mib 1024 \\
        --kernel mk_op_gu_x --workload llama8b --source-hash HASH --out profiles/traffic_llama8b.json

Each DIR is a rocprofv3 output directory holding run_counter_collection.csv.
Prints a per-kernel table (markdown) of every kernel in the --fetch run.
--last N keeps only the kernel's last N dispatches for --out: a megakernel
counter run starts with one launch that runs the whole prefill (one step
per prompt position), then launches one decode step each.
"""
import argparse
import csv
import json
import os
import statistics
from collections import defaultdict


def per_kernel(run_dir, counter):
    """{kernel name: [counter value (KiB) per dispatch, in dispatch order]} of one rocprofv3 run."""
    rows = defaultdict(list)
    with open(os.path.join(run_dir, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: [v for _, v in sorted(xs)] for k, xs in rows.items()}


def copy_scale(run_dir, counter, nbytes):
    """Bytes per counter unit: the copy kernel's known bytes over its reading
    (the median over its dispatches)."""
    v = per_kernel(run_dir, counter)
    copies = [x for k, xs in v.items() if "copyBuffer" in k for x in xs]
    if not copies:
        raise SystemExit(f"{run_dir}: no copy kernel dispatches with {counter}")
    return nbytes / statistics.median(copies)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--kernel", required=True, help="kernel whose bytes per launch go to --out")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--source-hash", required=True)
    ap.add_argument("--out")
    ap.add_argument("--last", type=int, default=0, metavar="N",
                    help="--out: average only the kernel's last N dispatches")
    a = ap.parse_args()
    n = a.copy_mib << 20
    fs = copy_scale(a.copy_fetch, "FETCH_SIZE", n)
    ws = copy_scale(a.copy_write, "WRITE_SIZE", n)
    fetch = per_kernel(a.fetch, "FETCH_SIZE")
    write = per_kernel(a.write, "WRITE_SIZE")
    print(f"copy probe: {a.copy_mib} MiB read and written; bytes per FETCH_SIZE unit {fs:.1f}, "
          f"per WRITE_SIZE unit {ws:.1f}\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | written MB |")
    print("|---|---|---|---|---|---|")
    for k in sorted(fetch, key=lambda k: -statistics.mean(fetch[k])):
        f = statistics.mean(fetch[k])
        w = statistics.mean(write[k]) if write.get(k) else 0.0
        print(f"| {k[:48]} | {len(fetch[k])} | {f:.0f} | {w:.0f} | {f * fs / 1e6:.2f} | {w * ws / 1e6:.3f} |")
    if a.out:
        if a.kernel not in fetch or a.kernel not in write:
            raise SystemExit(f"kernel {a.kernel} missing from the counter runs")
        fk, wk = fetch[a.kernel], write[a.kernel]
        if a.last:
            fk, wk = fk[-a.last:], wk[-a.last:]
        f = statistics.mean(fk)
        w = statistics.mean(wk)
        rec = {"workload": a.workload, "kernel": a.kernel, "kernel_source_hash": a.source_hash,
               "fetch_size_kib_per_dispatch": f, "write_size_kib_per_dispatch": w,
               "bytes_per_fetch_unit": fs, "bytes_per_write_unit": ws,
               "read_bytes_per_launch": f * fs, "written_bytes_per_launch": w * ws,
               "bytes_per_launch": f * fs + w * ws, "dispatches": len(fk)}
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")


if __name__ == "__main__":
    main()
