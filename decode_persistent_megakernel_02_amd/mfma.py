"""Matrix-core use per kernel from one rocprofv3 counter run.

    rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d DIR -o run -- python3 bench.py ...
    python -m decode_persistent_megakernel_02_amd.mfma DIR [--match mk_b_]

MfmaUtil is rocprofv3's derived counter: the cycles the SIMDs' matrix cores
were busy over the cycles the GPU was active times the SIMD count, in percent
(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMD_NUM) * 100), per
dispatch.  MfmaFlopsBF16 is the bf16 matrix-core work the dispatch issued,
in FLOP (SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512).  Prints one markdown row per
kernel: dispatches, mean utilisation, mean bf16 work per dispatch.
"""
import argparse
import statistics

from decode_persistent_megakernel_02_amd.counters import per_kernel


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("run_dir")
    ap.add_argument("--match", default="", help="only kernels whose name contains this")
    a = ap.parse_args()
    util = per_kernel(a.run_dir, "MfmaUtil")
    flops = per_kernel(a.run_dir, "MfmaFlopsBF16")
    print("| kernel | dispatches | matrix cores busy (MfmaUtil, mean %) | bf16 matrix work per dispatch (GFLOP) |")
    print("|---|---|---|---|")
    names = [k for k in util if a.match in k]
    for k in sorted(names, key=lambda k: -statistics.mean(flops.get(k, [0.0]))):
        f = statistics.mean(flops[k]) / 1e9 if flops.get(k) else 0.0
        print(f"| {k[:48]} | {len(util[k])} | {statistics.mean(util[k]):.1f} | {f:.2f} |")


if __name__ == "__main__":
    main()
