"""Decode benchmark: ms/token of one greedy decode step on one MI355X, with
achieved HBM bandwidth against the 8 TB/s peak.

Default workload: the Llama-3-8B shape (32 layers, hidden 4096, 32 q / 8 KV
heads of 128, FFN 14336, vocab 128256), random bf16 weights, batch 1, a 39-token
seeded prompt and 512 greedy decode steps -- the 39/512 workload of the MPK
write-up, on synthetic inputs.  Prints ONE JSON line.

Headline: the persistent megakernel, one launch per decode step.  Protocol,
for the megakernel and for the kernel-per-operator build of the same task
bodies (one HIP graph per step) alike: one warm-up generation (prefill + W
decode steps), then five runs of reset + prefill + exactly K decode steps with
device-side token feedback between two HIP events on the decode stream; the
value is the median run.  A sixth run brackets every step with events for the
per-step p50/p99.  The roofline entry is the megakernel dispatch itself:
whole-step algorithmic bytes over its duration.  A traced megakernel run gives
the time the compute waves wait between operators; a streaming-read probe
gives the measured HBM ceiling; the oracle's host time on a bounded sample is
reported as cpu_baseline.

`--workload llama8b_b8_kv4096` (8 sequences, 4096-token prompts, 128 steps)
and `--workload llama70b_b64` (the 70B shape, 64 sequences, 512-token prompts,
64 steps) time the batched path (per-operator launches, matrix cores); their
unit is ms per step (one token for every sequence) and they carry no
cpu_baseline.
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
    (kernels.hip, mega.hip, device.h, mk_internal.h): a counter summary taken on other
    kernel sources is not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_persistent_megakernel_02_amd", "csrc")
    for f in ("device.h", "kernels.hip", "mega.hip", "mk_internal.h"):
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


def protocol(abi, h, prompt_t, steps, warmup, torch, runs=5, log=lambda *a: None, name=""):
    """Warm-up generation, then `runs` timed runs (reset + prefill + `steps`
    decode steps between two events) and one run with an event pair around
    every step.  Returns (median ms/step, run totals, per-step ms, tokens)."""
    B = prompt_t.shape[0]
    toks = torch.zeros(max(steps, warmup) + 1, B, dtype=torch.int32, device="cuda")
    abi.mk_prefill(h, prompt_t, toks[0])
    run_steps(abi, h, toks, 0, warmup)
    abi.mk_synchronize(h)
    totals = []
    for r in range(runs):
        total, _ = timed_pass(abi, h, prompt_t, toks, steps, torch)
        totals.append(total)
        log(f"{name} run {r + 1}/{runs}: {total / steps:.4f} ms/step")
    tokens = toks[:steps + 1].cpu().numpy()
    abi.mk_reset(h)
    abi.mk_prefill(h, prompt_t, toks[0])
    abi.mk_synchronize(h)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for s in range(steps):
        abi.mk_decode_step(h, toks[s], toks[s + 1])
        ev[s + 1].record()
    torch.cuda.synchronize()
    abi.mk_synchronize(h)
    per = [ev[s].elapsed_time(ev[s + 1]) for s in range(steps)]
    totals.sort()
    return totals[len(totals) // 2] / steps, totals, per, tokens


def one_launch(abi, h, prompt_t, steps, torch, log=lambda *a: None, runs=5):
    """Megakernel: reset + prefill, then all `steps` decode steps in ONE launch
    (mk_generate) between two events; median of `runs`.  Returns (median
    ms/step, run totals, tokens [steps + 1, 1])."""
    toks = torch.zeros(steps + 1, 1, dtype=torch.int32, device="cuda")
    totals = []
    for r in range(runs):
        abi.mk_reset(h)
        abi.mk_prefill(h, prompt_t, toks[0])
        abi.mk_synchronize(h)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        abi.mk_generate(h, toks[0], steps, toks[1:].view(-1))
        t1.record()
        torch.cuda.synchronize()
        abi.mk_synchronize(h)
        totals.append(t0.elapsed_time(t1))
        log(f"megakernel one-launch run {r + 1}/{runs}: {totals[-1] / steps:.4f} ms/step")
    srt = sorted(totals)
    return srt[len(srt) // 2] / steps, totals, toks.cpu().numpy()


def prefill_flops(shape, B, P):
    """Flops of a prefill of B prompts of P positions, each product counted once
    (the second pass over the low parts of the split operands is not counted):
    every projection for the B P rows, the LM head for the B last rows, and the
    causal attention (q.k and p.v for every row over positions 0 .. p)."""
    H, F, V, L = shape.hidden, shape.ffn, shape.vocab, shape.n_layers
    qd, kd = shape.n_q_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim
    per_row = L * (H * (qd + 2 * kd) + qd * H + 2 * H * F + F * H)
    attn = L * qd * 2 * (P * (P + 1) // 2)
    return 2.0 * (B * P * per_row + B * V * H + B * attn)


def prefill_leg(abi, runtime, shape, dw, prompt_t, kv_fp32, torch, log, stepwise_mode=None, runs=5):
    """The batched prefill (MK_FLAG_BATCHED_PREFILL) of the workload's prompts:
    reset + prefill between two HIP events, median of `runs`; beside it, with
    `stepwise_mode`, the step-by-step prefill of that mode timed the same way."""
    B, P = prompt_t.shape

    def time_it(h, name):
        out = torch.zeros(B, dtype=torch.int32, device="cuda")
        ts = []
        for r in range(runs):
            abi.mk_reset(h)
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record()
            abi.mk_prefill(h, prompt_t, out)
            t1.record()
            torch.cuda.synchronize()
            abi.mk_synchronize(h)
            ts.append(t0.elapsed_time(t1))
            log(f"{name} prefill run {r + 1}/{runs}: {ts[-1]:.2f} ms")
        return sorted(ts)[len(ts) // 2], ts, out.cpu().numpy()

    h = runtime.create(shape, dw, P + 1, B, abi.MK_MODE_PER_OP, abi.MK_FLAG_BATCHED_PREFILL, kv_fp32=kv_fp32)
    ms, ts, ids = time_it(h, "batched")
    abi.mk_destroy(h)
    fl = prefill_flops(shape, B, P)
    res = {"ms": ms, "runs_ms": ts, "sequences": B, "positions": P, "tokens_per_s": B * P / (ms * 1e-3),
           "tflops_products_once": fl / (ms * 1e-3) / 1e12,
           "frac_of_bf16_matrix_peak": fl / (ms * 1e-3) / 1e12 / 2500.0,
           "timing": f"reset + mk_prefill of {B} x {P} positions between two HIP events, median of {runs}"}
    if stepwise_mode is not None:
        h = runtime.create(shape, dw, P + 1, B, stepwise_mode, 0, kv_fp32=kv_fp32)
        sms, sts, sids = time_it(h, "step-by-step")
        abi.mk_destroy(h)
        res["step_by_step"] = {"ms": sms, "runs_ms": sts,
                               "mode": "megakernel, one launch of P steps" if stepwise_mode == abi.MK_MODE_MEGAKERNEL
                               else "per-operator, one step per position",
                               "next_ids_equal": bool((sids == ids).all())}
        res["speedup_over_step_by_step"] = sms / ms
    log(f"batched prefill {B} x {P}: {ms:.2f} ms ({res['tokens_per_s']:.0f} tokens/s, "
        f"{res['tflops_products_once']:.0f} TFLOP/s)")
    return res


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs), q))


def mega_overhead(abi, shape, dw, prompt_t, steps, torch, dump=None):
    """Traced megakernel steps (the last one is analysed), per operator k and
    workgroup w: publish time of k's input page and the end of k's tasks.
      wait: compute waves idle between finishing k-1 and k's input being
            staged (0 when it was staged first);
      skew: how much later than the median workgroup the last one finished k-1;
      latency: from the last workgroup finishing k-1 to the median workgroup
            publishing k's input (signal propagation + staging).
    In microseconds; per operator type (the input of QKV is the previous
    layer's down output, of O the attention merge, ...)."""
    import numpy as np
    h = runtime_create(shape, dw, prompt_t.shape[1] + steps + 1, abi.MK_MODE_MEGAKERNEL, abi.MK_FLAG_TRACE, abi)
    toks = torch.zeros(steps + 1, 1, dtype=torch.int32, device="cuda")
    abi.mk_prefill(h, prompt_t, toks[0])
    run_steps(abi, h, toks, 0, steps)
    abi.mk_synchronize(h)
    tr, tpu = abi.mk_mega_trace(h)
    abi.mk_destroy(h)
    if dump:
        np.save(dump, tr)
    ops, ncu, slots = tr.shape
    nc = slots - 10  # compute waves; then the stager's publish, poll-start, input-complete and attention times
    end = (tr[:, :, :nc] & np.uint64(0xFFFFFFFF)).astype(np.int64)
    dur = (tr[:, :, :nc] >> np.uint64(32)).astype(np.int64)
    pub = (tr[:, :, nc] & np.uint64(0xFFFFFFFF)).astype(np.int64)
    got = (tr[:, :, nc + 2] & np.uint64(0xFFFFFFFF)).astype(np.int64)
    base = int(pub[0].min())
    rel = lambda a: ((a - base) % (1 << 32)).astype(np.int64) / tpu   # us since the first publish
    end_us, pub_us, got_us = rel(end).max(axis=2), rel(pub), rel(got)  # [ops, ncu]
    wait = np.maximum(pub_us[1:] - end_us[:-1], 0.0)
    skew = end_us[:-1].max(axis=1) - np.median(end_us[:-1], axis=1)
    lat = np.median(pub_us[1:], axis=1) - end_us[:-1].max(axis=1)
    stage = np.median(pub_us[1:] - got_us[1:], axis=1)   # input complete -> published (norm, rendezvous)
    run = dur.max(axis=2) / tpu
    names = ("qkv", "o", "gu", "down")
    by = lambda a, i: float(np.median(a[(np.arange(1, ops) % 4) == i])) if ops > 1 else 0.0
    # attention path of each layer, from the last workgroup finishing QKV:
    # units' inputs complete, units' records written, merges' inputs complete,
    # merges' outputs written (medians over the workgroups that ran them), and
    # O's input complete (median workgroup)
    path = {n: [] for n in ("unit_inputs", "unit_record", "merge_inputs", "merge_output", "o_input")}
    for l in range(shape.n_layers):
        k = 4 * l + 1
        qe = end_us[k - 1].max()
        for j, n in zip(range(3, 7), ("unit_inputs", "unit_record", "merge_inputs", "merge_output")):
            raw = tr[k, :, nc + j]
            m = raw != 0
            if m.any():
                path[n].append(float(np.median(rel((raw[m] & np.uint64(0xFFFFFFFF)).astype(np.int64)))) - qe)
        path["o_input"].append(float(np.median(got_us[k])) - qe)
    attn_path = {n: float(np.median(v)) for n, v in path.items() if v}
    return {"wait_us_median": float(np.median(wait)), "wait_us_p90": pct(wait.reshape(-1), 90),
            "wait_us_per_step": float(wait.sum(axis=0).mean()),
            "wait_us_median_by_op": {n: by(np.median(wait, axis=1), i) for i, n in enumerate(names)},
            "skew_us_median_by_op_input": {n: by(skew, i) for i, n in enumerate(names)},
            "latency_us_median_by_op_input": {n: by(lat, i) for i, n in enumerate(names)},
            "stage_us_median_by_op": {n: by(stage, i) for i, n in enumerate(names)},
            "op_run_us_median": {n: float(np.median(run[i::4][:shape.n_layers])) for i, n in enumerate(names)},
            "lm_head_run_us_median": float(np.median(run[-1])),
            "attention_path_us_after_qkv": attn_path,
            "steps_traced": steps}


def runtime_create(shape, dw, max_seq, mode, flags, abi):
    from decode_persistent_megakernel_02_amd import runtime
    return runtime.create(shape, dw, max_seq, 1, mode, flags, kv_fp32=True)


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
    # the oracle widens each bf16 matrix to fp64 when it uses it (a 15 GB model
    # does not fit the host in fp64); that widening alone, timed the same way:
    t = time.perf_counter()
    for name in weights:
        if name != "embed" or shape.tie_embeddings:
            D.widen_bf16(weights[name])
    widen = (time.perf_counter() - t) * 1000.0
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": ms, "unit": "ms/token", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} fp64 decode steps of the {shape.name} shape at positions 0 and 1, averaged; each "
                      "step widens the bf16 weights to fp64 as it uses them",
            "widening_ms_per_step": widen, "arithmetic_ms_per_step": ms - widen,
            "host_cpu": cpu, "os_cpu_count": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--no-megakernel", action="store_true", help="time only the per-operator build")
    ap.add_argument("--no-trace", action="store_true", help="skip the traced megakernel steps")
    ap.add_argument("--trace-dump", default=None, metavar="FILE.npy", help="save the raw megakernel trace")
    ap.add_argument("--no-per-op", action="store_true", help="skip the per-operator baseline (quick runs)")
    ap.add_argument("--no-stream-probe", action="store_true", help="skip the streaming-read ceiling probe")
    ap.add_argument("--no-prefill", action="store_true", help="skip the batched-prefill timing")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the batched prefill of the workload's prompts (row-major weights) and exit")
    ap.add_argument("--counters-mode", choices=("mega", "per_op"), default="mega",
                    help="with --counters: which build's launches the counter run sees")
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
    tiled = B > 1 and not args.row_major and not args.prefill_only
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
    if args.prefill_only:
        pf = prefill_leg(abi, runtime, shape, dw, prompt_t, kv_fp32, torch, log)
        print(json.dumps({"prefill": pf, "workload": wl.name, "kv_cache": "fp32" if kv_fp32 else "bf16",
                          "weights": "row-major"}), flush=True)
        return
    flags = (abi.MK_FLAG_FUSED_MERGE if args.fused_merge else 0) | (abi.MK_FLAG_TILED_WEIGHTS if tiled else 0)
    if args.counters:
        if args.counters_prompt:
            prompt_t = prompt_t[:, :args.counters_prompt].contiguous()
        if B == 1 and args.counters_mode == "mega":
            h = runtime.create(shape, dw, prompt_t.shape[1] + args.counters + 1, 1, abi.MK_MODE_MEGAKERNEL, 0,
                               attn_split=args.attn_split, kv_fp32=True)
        else:
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
    bytes_steps = [step_bytes(shape, wl.prompt_len + s + 1, B, 4 if kv_fp32 else 2) for s in range(steps)]
    alg_bytes = float(np.mean(bytes_steps))
    bound_ms = alg_bytes / (PEAK_GBPS * 1e9) * 1e3
    unit = "ms/token" if B == 1 else "ms/step"

    mega = None
    if B == 1 and not args.no_megakernel:
        h = runtime.create(shape, dw, max_seq + 64, 1, abi.MK_MODE_MEGAKERNEL, 0, attn_split=args.attn_split,
                           kv_fp32=True)
        mega_ms, mega_runs, mega_per, mega_tokens = protocol(abi, h, prompt_t, steps, warmup, torch, log=log,
                                                             name="megakernel")
        split = abi.mk_get_debug_view(h).split
        one_ms, one_runs, one_tokens = one_launch(abi, h, prompt_t, steps, torch, log)
        abi.mk_destroy(h)
        mega = {"ms_per_token": mega_ms, "runs_ms_per_token": [t / steps for t in mega_runs],
                "step_p50_ms": pct(mega_per, 50), "step_p99_ms": pct(mega_per, 99),
                "attn_split": split, "kernel": mega_kernel_name(shape),
                "one_launch": {"ms_per_token": one_ms, "runs_ms_per_token": [t / steps for t in one_runs],
                               "tokens_equal_per_step_launches": bool((one_tokens == mega_tokens).all()),
                               "timing": f"mk_generate: all {steps} steps in one launch, median of 5 runs "
                                         "between two HIP events"}}
        log(f"megakernel: {mega_ms:.4f} ms/token (median of 5), p50 {mega['step_p50_ms']:.4f}, "
            f"p99 {mega['step_p99_ms']:.4f} ms; bound {bound_ms:.4f} ms")
        if not args.no_trace:
            mega["overhead"] = mega_overhead(abi, shape, dw, prompt_t, args.steps, torch, dump=args.trace_dump)
            log(f"megakernel operator-boundary wait: median {mega['overhead']['wait_us_median']:.2f} us, "
                f"{mega['overhead']['wait_us_per_step']:.1f} us per step")

    per_op, op_ms, op_tokens = None, None, None
    if not (args.no_per_op and mega is not None):
        per_op, op_ms, op_tokens, gu_gbps, kern_ms, kb, gu_kernel = per_op_baseline(
            abi, runtime, shape, dw, prompt_t, steps, warmup, max_seq, B, flags, args, kv_fp32, tiled, wl, torch, log)

    prefill = None
    if not tiled and not args.no_prefill:
        prefill = prefill_leg(abi, runtime, shape, dw, prompt_t, kv_fp32, torch, log,
                              stepwise_mode=abi.MK_MODE_MEGAKERNEL if B == 1 else None)

    ceiling = None
    if B == 1 and not args.no_stream_probe:
        buf = torch.empty(1 << 30, dtype=torch.int32, device="cuda").fill_(1)  # 4 GiB
        ceiling = {}
        for wgs, loads in ((256, 4), (256, 8), (512, 8), (1024, 8)):
            ms = abi.mk_t_stream_read(buf, wgs, loads, reps=5)
            ceiling[f"{wgs}x512_threads_{loads}_loads"] = buf.numel() * 4 / (ms * 1e-3) / 1e9
        del buf
        log("streaming-read ceiling (GB/s): " + ", ".join(f"{k} {v:.0f}" for k, v in ceiling.items()))

    if mega is not None:
        ms = mega["ms_per_token"]
        achieved = alg_bytes / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / PEAK_GBPS, "traffic": load_traffic(wl.name + "_mega"),
                    "kernel": mega["kernel"], "kernel_avg_ms": ms,
                    "algorithmic_bytes_per_launch": alg_bytes,
                    "timing": "one megakernel dispatch per step: median of 5 runs of the decode steps between two "
                              "HIP events on the decode stream"}
        mode = "megakernel (one persistent launch per step)"
    else:
        ms = op_ms
        roofline = {"bound": "hbm", "achieved": gu_gbps, "peak": PEAK_GBPS, "unit": "GB/s",
                    "frac": gu_gbps / PEAK_GBPS, "traffic": load_traffic(wl.name), "kernel": gu_kernel,
                    "kernel_avg_ms": kern_ms, "algorithmic_bytes_per_launch": kb}
        mode = per_op["mode"]
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
                   "batch": B, "prompt_len": wl.prompt_len, "decode_steps": steps, "mode": mode,
                   "kv_cache": "fp32" if kv_fp32 else "bf16",
                   "attn_split": args.attn_split or "library default",
                   "weights": "tiled" if tiled else "row-major",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": 1000.0 * B / ms,
        "achieved_gbps": alg_bytes / (ms * 1e-3) / 1e9,
        "bound_ms_per_token": bound_ms,
        "step_frac_of_hbm_bound": bound_ms / ms,
        "roofline": roofline,
        "megakernel": mega,
        "per_op_baseline": per_op,
        "megakernel_speedup_over_per_op": (op_ms / mega["ms_per_token"]) if mega and op_ms else None,
        "streaming_read_ceiling_gbps": ceiling,
        "prefill": prefill,
        "tokens_equal_megakernel_per_op": bool((mega_tokens == op_tokens).all()) if mega and op_ms else None,
        "cpu_baseline": None,
    }
    if B > 1 and per_op:
        gu_flop = 2.0 * B * 2 * shape.ffn * shape.hidden
        res["gu_matrix_core_tflops"] = gu_flop / (kern_ms * 1e-3) / 1e12
        res["gu_matrix_core_frac_of_bf16_peak"] = res["gu_matrix_core_tflops"] / 2500.0
    if not args.no_cpu_baseline and weights is not None:
        log("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(shape, weights, prompt)
    print(json.dumps(res), flush=True)


def per_op_baseline(abi, runtime, shape, dw, prompt_t, steps, warmup, max_seq, B, flags, args, kv_fp32, tiled, wl, torch, log):
    """The kernel-per-operator build, same protocol; plus its gate/up kernel roofline, replays and breakdown."""
    h = runtime.create(shape, dw, max_seq + 64, B, abi.MK_MODE_PER_OP, flags, attn_split=args.attn_split,
                       kv_fp32=kv_fp32)
    op_ms, op_runs, op_per, op_tokens = protocol(abi, h, prompt_t, steps, warmup, torch, log=log, name="per-op")
    # per-operator breakdown (eager launches bracketed by events) of 32 more steps
    toks = torch.zeros(33, B, dtype=torch.int32, device="cuda")
    toks[0] = torch.from_numpy(op_tokens[-1]).cuda()
    abi.mk_time_ops(h, list(abi.OP_TYPES), 32 * (12 * shape.n_layers + 4))
    run_steps(abi, h, toks, 0, 32)
    breakdown = abi.mk_read_op_times(h)
    view = abi.mk_get_debug_view(h)
    gu_exact = bool(view.exact_ops & (1 << abi.TASK_TYPES["gu"]))
    op_grid = {k: view.op_grid[v] for k, v in abi.TASK_TYPES.items() if view.op_grid[v]}
    # The gate/up launches of every layer replayed back to back between two
    # events: per-launch time without the cost of an event pair around each
    # launch (cycling through the layers keeps the weights out of the caches).
    reps = 64 if B == 1 else 8
    rep_ms, rep_launches = abi.mk_time_op_replay(h, "gu", reps)
    log(f"gate/up replay: {rep_launches} launches in {rep_ms:.2f} ms")
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
    kern_ms = rep_ms / (reps * shape.n_layers)  # one layer's gate/up operator
    kb = gu_bytes(shape, B)
    gu_gbps = kb / (kern_ms * 1e-3) / 1e9
    unit = "ms/token" if B == 1 else "ms/step"
    log(f"per-op: {op_ms:.4f} {unit} (median of 5), gate/up kernel {kern_ms * 1e3:.1f} us = {gu_gbps:.0f} GB/s")
    op_breakdown = {k: {"ms_per_step": v[0] / 32.0, "launches_per_step": v[1] / 32.0} for k, v in breakdown.items()}
    per_layer = rep_launches // (reps * shape.n_layers)  # 2 when a split-K finishing launch follows
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
    per_op = {"ms_per_step": op_ms, "runs_ms_per_step": [t / steps for t in op_runs],
              "step_p50_ms": pct(op_per, 50), "step_p99_ms": pct(op_per, 99),
              "mode": "one HIP graph of per-operator launches per step" + (", fused merge" if args.fused_merge else ""),
              "gu_kernel": {"kernel": gu_kernel, "avg_ms": kern_ms, "algorithmic_bytes_per_launch": kb,
                            "achieved_gbps": gu_gbps, "frac_of_peak": gu_gbps / PEAK_GBPS,
                            "traffic_bytes_per_launch": load_traffic(wl.name),
                            "timing": f"{reps} back-to-back replays of the {shape.n_layers} layers' gate/up launches "
                                      "between two HIP events on the decode stream"},
              "op_breakdown_eager": op_breakdown, "op_replay_us_per_layer": replay_us, "op_grid": op_grid}

    return per_op, op_ms, op_tokens, gu_gbps, kern_ms, kb, gu_kernel


def mega_kernel_name(shape):
    """The megakernel instance the library launches for a batch-1 shape with an fp32 cache."""
    qd = shape.n_q_heads * shape.head_dim
    G = shape.n_q_heads // shape.n_kv_heads
    exact = shape.hidden % 2048 == 0 and qd % 2048 == 0 and shape.ffn % 2048 == 0 and G == 4
    return f"mk_mega_{'x' if exact else 'n'}_{shape.head_dim}_f32_g{G}"


if __name__ == "__main__":
    main()
