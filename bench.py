"""Decode benchmark: ms/token of one greedy decode step on one MI355X, with
achieved HBM bandwidth against the 8 TB/s peak.

Default workload: the Llama-3-8B shape (32 layers, hidden 4096, 32 q / 8 KV
heads of 128, FFN 14336, vocab 128256), random bf16 weights, batch 1, a 39-token
seeded prompt and 512 greedy decode steps -- the 39/512 workload of the MPK
write-up, on synthetic inputs.  Prints ONE JSON line.

Protocol: W untimed warm-up decode steps, reset + prefill, then exactly K
decode steps with device-side token feedback, bracketed by synchronize.  The
step runs in kernel-per-operator mode, one HIP graph per step (the persistent
single-launch mode is refused by the library on this device).  The dominant
kernel's duration (gate/up projection + SwiGLU, the roofline figure) comes
from back-to-back replays of its launches for every layer between two HIP
events on the decode stream; an eager pass with an event pair around each
launch, a per-operator breakdown and replays of the other operators are
reported beside it.  The oracle's time on a bounded sample is reported as
cpu_baseline.

`--workload llama8b_b8_kv4096` (8 sequences, 4096-token prompts, 128 steps)
and `--workload llama70b_b64` (the 70B shape, 64 sequences, 512-token prompts,
64 steps) time the batched path the same way; their unit is ms per step (one
token for every sequence) and they carry no cpu_baseline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/token decode (8B shape, batch 1) + achieved HBM GB/s vs peak, 1 MI355X"
PEAK_GBPS = 8000.0


def step_bytes(shape, T, batch=1, kv_bytes=4):
    """Algorithmic HBM bytes of one decode step with T cached positions (incl. the new one).

    Every weight matrix once, one embedding row per sequence, the norm gains,
    K and V of T positions read per layer and sequence, the new K/V written
    (kv_bytes per cached element: 4 for the fp32 cache of batch-1 decode).
    """
    s = shape
    qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    per_layer = s.hidden * (qd + 2 * kd) + s.hidden * qd + 3 * s.hidden * s.ffn + 2 * s.hidden
    weights = 2 * (s.n_layers * per_layer + s.vocab * s.hidden + s.hidden)
    emb = 2 * s.hidden * batch
    kv_read = 2 * kv_bytes * s.n_layers * kd * T * batch
    kv_write = 2 * kv_bytes * s.n_layers * kd * batch
    return weights + emb + kv_read + kv_write


def kernel_source_hash():
    """Hash of the sources the batch-1 operator kernels are compiled from
    (kernels.hip, device.h, mk_internal.h): a counter summary taken on other
    kernel sources is not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_persistent_megakernel_02_amd", "csrc")
    for f in ("device.h", "kernels.hip", "mk_internal.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """Measured HBM bytes per launch from a committed counter summary, if it was
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def gu_bytes(shape, batch=1):
    """Algorithmic bytes of one gate/up + SwiGLU launch.  Batch 1: both weight
    matrices, the norm gain, the fp32 input vector read once, the output
    written once.  Batched: both weight matrices, the bf16 normalised inputs
    [B, H] read once, the outputs written once (fp32 and the bf16 operand of
    the down-projection)."""
    w = 2 * shape.ffn * shape.hidden * 2
    if batch == 1:
        return w + 2 * shape.hidden + 4 * shape.hidden + 4 * shape.ffn
    return w + 2 * batch * shape.hidden + 6 * batch * shape.ffn


def run_steps(abi, h, toks, first, steps):
    """Decode steps with device-side feedback: row s of toks feeds step s, whose
    greedy tokens land in row s + 1."""
    for s in range(first, first + steps):
        abi.mk_decode_step(h, toks[s], toks[s + 1])


def timed_pass(abi, h, prompt_t, toks, steps, torch, time_types=()):
    """reset + prefill, then exactly `steps` decode steps between two events."""
    abi.mk_reset(h)
    abi.mk_prefill(h, prompt_t, toks[0])
    abi.mk_synchronize(h)
    if time_types:
        abi.mk_time_ops(h, time_types, steps * 64 + 64)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    run_steps(abi, h, toks, 0, steps)
    t1.record()
    torch.cuda.synchronize()
    abi.mk_synchronize(h)
    times = abi.mk_read_op_times(h) if time_types else {}
    return t0.elapsed_time(t1), times


def time_decode(abi, h, prompt_t, steps, warmup, shape, torch, log=lambda *a: None):
    """Headline pass (graph-replayed steps), then an eager pass whose gate/up
    launches are bracketed by HIP events, then an untimed per-operator breakdown."""
    B = prompt_t.shape[0]
    toks = torch.zeros(max(steps, warmup) + 64 + 1, B, dtype=torch.int32, device=torch.device("cuda"))
    abi.mk_prefill(h, prompt_t, toks[0])                         # warm-up generation
    run_steps(abi, h, toks, 0, warmup)
    abi.mk_synchronize(h)
    log("warm-up done; timed pass")
    total, _ = timed_pass(abi, h, prompt_t, toks, steps, torch)
    tokens = toks[:steps + 1].cpu().numpy()
    log(f"timed pass: {total / steps:.4f} ms/step; eager pass with gate/up events")
    eager_total, times = timed_pass(abi, h, prompt_t, toks, steps, torch, ["gu"])
    gu = times.get("gu", (0.0, 0))
    same = bool((toks[:steps + 1].cpu().numpy() == tokens).all())
    abi.mk_time_ops(h, list(abi.OP_TYPES), 32 * (12 * shape.n_layers + 4))  # every launch of 32 steps
    run_steps(abi, h, toks, steps, 32)
    breakdown = abi.mk_read_op_times(h)
    return total, eager_total, gu, same, breakdown


def cpu_baseline(shape, weights, prompt):
    """The oracle as it stands on the host: one fp64 decode step (position 0)."""
    from oracle import decoder as D
    threads = os.cpu_count()
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        if info:
            threads = max(i.get("num_threads", 0) for i in info) or threads
    except Exception:
        pass
    dec = D.Decoder(shape, weights, prompt.shape[0], 4, cache_weights=False)
    n = 2
    t = time.perf_counter()
    for i in range(n):
        dec.step(prompt[:, i])
    ms = (time.perf_counter() - t) * 1000.0 / n
    return {"value": ms, "unit": "ms/token", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} fp64 decode steps of the {shape.name} shape at positions 0 and 1 "
                      "(weights widened per use), averaged"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--fused-merge", action="store_true",
                    help="merge attention splits in the last split workgroup instead of a separate launch")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB five times (the known-size reference "
                         "for scaling hardware byte counters) and exit")
    ap.add_argument("--row-major", action="store_true",
                    help="batched workloads: keep the projection weights row-major instead of tiled")
    ap.add_argument("--attn-split", type=int, default=0, metavar="POSITIONS",
                    help="positions per split-KV attention workgroup (0: the library's choice)")
    ap.add_argument("--counters", type=int, default=0, metavar="STEPS",
                    help="only run prefill and STEPS eager decode steps (no graph, no timing) so that a "
                         "hardware-counter profiler sees each launch, and exit")
    ap.add_argument("--counters-prompt", type=int, default=0, metavar="TOKENS",
                    help="with --counters: use only the first TOKENS prompt positions (a short prefill, so a "
                         "kernel trace stays small; attention then sees a shorter context)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(it measures one GPU's share of the work).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from synth import gen, presets
    from decode_persistent_megakernel_02_amd import abi, runtime

    log = (lambda *a: None) if args.quiet else (lambda *a: print(*a, file=sys.stderr, flush=True))
    wl = presets.WORKLOADS[args.workload]
    shape, B = wl.shape, wl.batch
    steps, warmup = args.steps, args.warmup
    max_seq = wl.prompt_len + max(steps, warmup)
    t = time.time()
    # the batched path reads its projection weights in the tiled layout
    tiled = B > 1 and not args.row_major
    if B == 1:
        weights = gen.gen_weights(shape, wl.weight_seed)
        dw = runtime.upload_weights(weights)
    else:  # one tensor at a time through host memory (the 70B shape is 141 GB)
        weights = None
        last = [time.time()]

        def progress(i, n):
            if time.time() - last[0] > 20 or i == n:
                last[0] = time.time()
                log(f"weights: {i}/{n} tensors on the device")
        dw = runtime.generate_device_weights(shape, wl.weight_seed, progress=progress, tiled=tiled)
    torch.cuda.synchronize()
    log(f"weights generated and uploaded in {time.time() - t:.1f}s")
    prompt = gen.gen_prompt(wl)
    prompt_t = torch.from_numpy(prompt).cuda()

    # batch 1 keeps an fp32 KV cache; the batched workloads state a bf16 cache
    kv_fp32 = B == 1
    flags = (abi.MK_FLAG_FUSED_MERGE if args.fused_merge else 0) | (abi.MK_FLAG_TILED_WEIGHTS if tiled else 0)
    if args.counters:
        if args.counters_prompt:
            prompt_t = prompt_t[:, :args.counters_prompt].contiguous()
        h = runtime.create(shape, dw, prompt_t.shape[1] + args.counters + 1, B, abi.MK_MODE_PER_OP,
                           flags | abi.MK_FLAG_NO_GRAPH, attn_split=args.attn_split, kv_fp32=kv_fp32)
        toks = torch.zeros(args.counters + 1, B, dtype=torch.int32, device="cuda")
        abi.mk_prefill(h, prompt_t, toks[0])
        for s in range(args.counters):
            abi.mk_decode_step(h, toks[s], toks[s + 1])
            abi.mk_synchronize(h)
            log(f"counter pass: decode step {s + 1}/{args.counters} done")
        abi.mk_destroy(h)
        print(json.dumps({"counter_pass_steps": args.counters, "workload": wl.name}))
        return
    h = runtime.create(shape, dw, max_seq + 64, B, abi.MK_MODE_PER_OP, flags, attn_split=args.attn_split,
                       kv_fp32=kv_fp32)
    total, eager_total, (gu_ms, gu_n), same_tokens, breakdown = time_decode(abi, h, prompt_t, steps, warmup, shape,
                                                                             torch, log)
    view = abi.mk_get_debug_view(h)
    gu_exact = bool(view.exact_ops & (1 << abi.TASK_TYPES["gu"]))
    op_grid = {k: view.op_grid[v] for k, v in abi.TASK_TYPES.items() if view.op_grid[v]}
    # The gate/up launches of every layer replayed back to back between two
    # events: per-launch time without the cost of an event pair around each
    # launch (cycling through the layers keeps the weights out of the caches).
    reps = 64 if B == 1 else 8
    rep_ms, rep_launches = abi.mk_time_op_replay(h, "gu", reps)
    log(f"gate/up replay: {rep_launches} launches in {rep_ms:.2f} ms")
    # every operator that can be replayed, the same way: us per layer
    replay_us = {}
    for name in (["norm"] if B > 1 else []) + ["qkv", "attn", "merge", "o", "gu", "down"]:
        if B > 1 and name == "qkv":
            continue  # appends to the KV cache; not replayable on the batched path
        ms_r, n_r = abi.mk_time_op_replay(h, name, 8)
        if n_r:
            replay_us[name] = {"us_per_layer": 1e3 * ms_r / (8 * shape.n_layers),
                               "launches_per_layer": n_r / (8 * shape.n_layers)}
    log("replayed operators (us per layer): " +
        ", ".join(f"{k} {v['us_per_layer']:.1f}" for k, v in replay_us.items()))
    abi.mk_destroy(h)
    ms = total / steps
    kern_ms = rep_ms / (reps * shape.n_layers)  # one layer's gate/up operator
    per_layer = rep_launches // (reps * shape.n_layers)  # 2 when a split-K finishing launch follows
    eager_kern_ms = gu_ms * per_layer / max(gu_n, 1)
    bytes_steps = [step_bytes(shape, wl.prompt_len + s + 1, B, 4 if kv_fp32 else 2) for s in range(steps)]
    alg_bytes = float(np.mean(bytes_steps))
    bound_ms = alg_bytes / (PEAK_GBPS * 1e9) * 1e3
    kb = gu_bytes(shape, B)
    achieved = kb / (kern_ms * 1e-3) / 1e9
    unit = "ms/token" if B == 1 else "ms/step"
    log(f"per-op: {ms:.4f} {unit}, bound {bound_ms:.4f} ms, step {alg_bytes / (ms * 1e-3) / 1e9:.0f} GB/s; "
        f"gate/up kernel {kern_ms * 1e3:.1f} us = {achieved:.0f} GB/s")
    op_breakdown = {k: {"ms_per_step": v[0] / 32.0, "launches_per_step": v[1] / 32.0} for k, v in breakdown.items()}
    log("breakdown (ms/step): " + ", ".join(f"{k} {v['ms_per_step']:.3f}" for k, v in op_breakdown.items()))
    traffic = load_traffic(wl.name)
    if B == 1:
        gu_kernel = "mk_op_gu_x" if gu_exact else "mk_op_gu"
    else:
        bt = 1 if B <= 16 else 2 if B <= 32 else 4
        # the library gives a wave two row groups at four batch tiles when the
        # operator has at least half a CU's worth of groups per CU
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        gpw2 = bt == 4 and -(-shape.ffn // 16) // 8 >= ncu // 2
        gu_kernel = (f"mk_b_gu_b{bt}" + ("_t" if tiled else "") + ("_g2" if gpw2 else "")
                     + (" + mk_b_fin_gu" if per_layer > 1 else ""))
    res = {
        "metric": METRIC if wl.name == "llama8b" else f"ms/step decode ({wl.name}, batch {B}), 1 MI355X",
        "value": ms,
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: batch {B}, prompt {wl.prompt_len}, {steps} greedy decode steps",
                   "batch": B, "prompt_len": wl.prompt_len, "decode_steps": steps,
                   "mode": "per_op (HIP graph per step)" + (", fused merge" if args.fused_merge else ""),
                   "kv_cache": "fp32" if kv_fp32 else "bf16",
                   "attn_split": args.attn_split or "library default",
                   "weights": "tiled" if tiled else "row-major",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": 1000.0 * B / ms,
        "achieved_gbps": alg_bytes / (ms * 1e-3) / 1e9,
        "bound_ms_per_token": bound_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBPS, "traffic": traffic,
                     "kernel": gu_kernel, "kernel_avg_ms": kern_ms, "algorithmic_bytes_per_launch": kb,
                     "timing": f"{reps} back-to-back replays of the {shape.n_layers} layers' gate/up launches "
                               "between two HIP events on the decode stream",
                     "kernel_avg_ms_event_pair_per_launch": eager_kern_ms},
        "step_frac_of_hbm_bound": bound_ms / ms,
        "eager_ms_per_step": eager_total / steps,
        "graph_and_eager_tokens_equal": same_tokens,
        "op_breakdown": op_breakdown,
        "op_replay_us_per_layer": replay_us,
        "op_grid": op_grid,
        "megakernel": {"status": "disabled", "reason": "cooperative persistent launch did not complete on MI355X"},
        "cpu_baseline": None,
    }
    if B > 1:
        gu_flop = 2.0 * B * 2 * shape.ffn * shape.hidden
        res["gu_matrix_core_tflops"] = gu_flop / (kern_ms * 1e-3) / 1e12
        res["gu_matrix_core_frac_of_bf16_peak"] = res["gu_matrix_core_tflops"] / 2500.0
    if not args.no_cpu_baseline and weights is not None:
        log("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(shape, weights, prompt)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
