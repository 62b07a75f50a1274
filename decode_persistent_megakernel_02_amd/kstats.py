"""Per-kernel dispatch durations from a rocprofv3 --kernel-trace run.

    python -m decode_persistent_megakernel_02_amd.kstats DIR [--one-step KERNEL]

DIR is a rocprofv3 output directory holding run_kernel_trace.csv.  Prints a
markdown table (calls, average / min / max microseconds, share of GPU time)
of every kernel.  A megakernel dispatch runs one decode step, or several:
mk_prefill runs one step per prompt position in one launch and mk_generate
all of its steps.  --one-step KERNEL adds a row for that kernel's one-step
dispatches alone: those no longer than twice the kernel's median dispatch
(one-step launches are the large majority of bench.py's profiled command,
and a launch of two or more steps takes at least twice as long).
"""
import argparse
import csv
import os
import statistics
from collections import defaultdict


def durations(run_dir):
    """{kernel name: [duration (ns) per dispatch]}."""
    d = defaultdict(list)
    with open(os.path.join(run_dir, "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            d[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return d


def row(name, xs, total):
    return (f"| {name[:48]} | {len(xs)} | {statistics.mean(xs) / 1e3:.2f} | {min(xs) / 1e3:.2f} | "
            f"{max(xs) / 1e3:.2f} | {100.0 * sum(xs) / total:.1f} |")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("run_dir")
    ap.add_argument("--one-step", metavar="KERNEL", help="also list this kernel's one-step dispatches")
    a = ap.parse_args()
    d = durations(a.run_dir)
    total = sum(sum(xs) for xs in d.values())
    print("| kernel | calls | avg us | min us | max us | % of GPU time |")
    print("|---|---|---|---|---|---|")
    for k in sorted(d, key=lambda k: -sum(d[k])):
        print(row(k, d[k], total))
        if k == a.one_step:
            med = statistics.median(d[k])
            one = [x for x in d[k] if x <= 2 * med]
            print(row(k + " (one-step)", one, total))


if __name__ == "__main__":
    main()
