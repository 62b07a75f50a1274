"""Host-side checks of the benchmark's bookkeeping: the algorithmic byte count
behind the roofline, the hardware-counter scaling, and the one-GPU contract.
Nothing here touches a GPU.
"""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from decode_persistent_megakernel_02_amd import counters  # noqa: E402
from synth import presets  # noqa: E402

# Llama-3-8B: 8,030,261,248 parameters in all, of which the input embedding
# table is 128256 x 4096 = 525,336,576 (the LM head is a separate matrix).
LLAMA3_8B_PARAMS = 8_030_261_248
LLAMA3_8B_EMBED = 128256 * 4096


def test_step_bytes_counts_every_weight_once():
    """Weights = every parameter except the embedding table, in bf16; plus one
    embedding row, and K/V read over T positions and written once per layer."""
    s = presets.WORKLOADS["llama8b"].shape
    kd = s.n_kv_heads * s.head_dim
    for T, kvb in ((1, 2), (295, 2), (551, 4)):
        expect = (2 * (LLAMA3_8B_PARAMS - LLAMA3_8B_EMBED) + 2 * s.hidden
                  + 2 * kvb * s.n_layers * kd * T + 2 * kvb * s.n_layers * kd)
        assert bench.step_bytes(s, T, 1, kvb) == expect


def test_step_bytes_scales_the_per_sequence_terms_with_the_batch():
    s = presets.WORKLOADS["llama8b"].shape
    one, eight = bench.step_bytes(s, 4096, 1, 2), bench.step_bytes(s, 4096, 8, 2)
    weights = 2 * (LLAMA3_8B_PARAMS - LLAMA3_8B_EMBED)
    assert eight - weights == 8 * (one - weights)


def test_gate_up_bytes_per_launch():
    """Both 14336 x 4096 bf16 matrices, the bf16 norm gain, the fp32 input and
    the fp32 SwiGLU output of one sequence."""
    s = presets.WORKLOADS["llama8b"].shape
    assert bench.gu_bytes(s) == 2 * 14336 * 4096 * 2 + 4096 * 2 + 4096 * 4 + 14336 * 4 == 234962944


def _counter_dir(tmp_path, name, counter, rows):
    d = tmp_path / name
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})
    return str(d)


def test_counter_scaling_uses_the_copy_probe(tmp_path):
    """A copy of 1 MiB that reads 512 FETCH_SIZE units means 2048 B per unit;
    a kernel reading 1000 units then moved 2,048,000 bytes."""
    mib = 1 << 20
    cf = _counter_dir(tmp_path, "cf", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 512)] * 3)
    cw = _counter_dir(tmp_path, "cw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1024)] * 3)
    f = _counter_dir(tmp_path, "f", "FETCH_SIZE", [("mk_op_gu_x", 1000), ("mk_op_gu_x", 1002)])
    w = _counter_dir(tmp_path, "w", "WRITE_SIZE", [("mk_op_gu_x", 10)])
    assert counters.copy_scale(cf, "FETCH_SIZE", mib) == 2048.0
    assert counters.copy_scale(cw, "WRITE_SIZE", mib) == 1024.0
    out = tmp_path / "t.json"
    subprocess.run([sys.executable, "-m", "decode_persistent_megakernel_02_amd.counters", "--fetch", f, "--write", w,
                    "--copy-fetch", cf, "--copy-write", cw, "--copy-mib", "1", "--kernel", "mk_op_gu_x",
                    "--workload", "llama8b", "--source-hash", "x", "--out", str(out)],
                   check=True, cwd=ROOT, capture_output=True)
    import json
    rec = json.load(open(out))
    assert rec["read_bytes_per_launch"] == pytest.approx(1001 * 2048)
    assert rec["written_bytes_per_launch"] == pytest.approx(10 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(1001 * 2048 + 10 * 1024)


def test_counter_scaling_needs_a_copy_kernel(tmp_path):
    cf = _counter_dir(tmp_path, "cf", "FETCH_SIZE", [("mk_op_gu_x", 512)])
    with pytest.raises(SystemExit):
        counters.copy_scale(cf, "FETCH_SIZE", 1 << 20)


def test_matrix_core_summary_averages_each_kernel(tmp_path):
    """mfma.py: one row per kernel, mean MfmaUtil and mean bf16 work per
    dispatch, heaviest first; kernels outside --match are left out."""
    d = tmp_path / "m"
    d.mkdir()
    rows = [("mk_b_gu_b4_t_g2", "MfmaUtil", 30.0), ("mk_b_gu_b4_t_g2", "MfmaFlopsBF16", 120e9),
            ("mk_b_gu_b4_t_g2", "MfmaUtil", 28.0), ("mk_b_gu_b4_t_g2", "MfmaFlopsBF16", 120e9),
            ("mk_b_o_b4_t", "MfmaUtil", 19.0), ("mk_b_o_b4_t", "MfmaFlopsBF16", 17e9),
            ("other_kernel", "MfmaUtil", 1.0), ("other_kernel", "MfmaFlopsBF16", 1e9)]
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i // 2 + 1, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})
    r = subprocess.run([sys.executable, "-m", "decode_persistent_megakernel_02_amd.mfma", str(d), "--match", "mk_b_"],
                       check=True, cwd=ROOT, capture_output=True, text=True)
    lines = [l for l in r.stdout.splitlines() if l.startswith("| mk_")]
    assert lines == ["| mk_b_gu_b4_t_g2 | 2 | 29.0 | 120.00 |", "| mk_b_o_b4_t | 1 | 19.0 | 17.00 |"]


def test_counter_last_dispatches_skip_the_prefill_launch(tmp_path):
    """A megakernel counter run: one launch of the whole prefill (40 steps'
    bytes), then one launch per decode step; --last 3 keeps the decode steps."""
    cf = _counter_dir(tmp_path, "cf", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 512)])
    cw = _counter_dir(tmp_path, "cw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1024)])
    k = "mk_mega_x_128_f32_g4"
    f = _counter_dir(tmp_path, "f", "FETCH_SIZE", [(k, 40000), (k, 1000), (k, 1001), (k, 1002)])
    w = _counter_dir(tmp_path, "w", "WRITE_SIZE", [(k, 400), (k, 10), (k, 10), (k, 10)])
    out = tmp_path / "t.json"
    subprocess.run([sys.executable, "-m", "decode_persistent_megakernel_02_amd.counters", "--fetch", f, "--write", w,
                    "--copy-fetch", cf, "--copy-write", cw, "--copy-mib", "1", "--kernel", k, "--last", "3",
                    "--workload", "llama8b_mega", "--source-hash", "x", "--out", str(out)],
                   check=True, cwd=ROOT, capture_output=True)
    import json
    rec = json.load(open(out))
    assert rec["dispatches"] == 3
    assert rec["read_bytes_per_launch"] == pytest.approx(1001 * 2048)
    assert rec["written_bytes_per_launch"] == pytest.approx(10 * 1024)


def test_kernel_stats_keep_one_step_dispatches_apart(tmp_path):
    """kstats: dispatches longer than twice the kernel's median (multi-step
    launches) are left out of the one-step row."""
    from decode_persistent_megakernel_02_amd import kstats
    d = tmp_path / "k"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for dur in [3000, 3100, 3050, 120000, 3020, 200000]:
            w.writerow({"Kernel_Name": "mk_mega_x", "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 10
    r = subprocess.run([sys.executable, "-m", "decode_persistent_megakernel_02_amd.kstats", str(d),
                        "--one-step", "mk_mega_x"], check=True, cwd=ROOT, capture_output=True, text=True)
    one = [l for l in r.stdout.splitlines() if "(one-step)" in l][0].split("|")
    assert int(one[2]) == 4 and float(one[3]) == pytest.approx(3042.5 / 1e3, abs=0.006)  # printed to 0.01 us
    assert kstats.durations(str(d))["mk_mega_x"][3] == 120000


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
