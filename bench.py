"""Decode benchmark: ms/token of one greedy decode step (one persistent-kernel
launch) on one MI355X, with achieved HBM bandwidth against the 8 TB/s peak.

Default workload: the Llama-3-8B shape (32 layers, hidden 4096, 32 q / 8 KV
heads of 128, FFN 14336, vocab 128256), random bf16 weights, batch 1, a 39-token
seeded prompt and 512 greedy decode steps -- the 39/512 workload of the MPK
write-up, on synthetic inputs.  Prints ONE JSON line.

Protocol: W untimed warm-up decode steps, reset + prefill, then exactly K
decode steps with device-side token feedback, bracketed by synchronize.  Every
launch is also bracketed by HIP events on the stream it runs on, which gives
the average kernel duration used for the roofline figure.  The same protocol
times the kernel-per-operator build of the same task bodies.  The oracle's
time on a bounded sample is reported as cpu_baseline.
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


def step_bytes(shape, T, batch=1):
    """Algorithmic HBM bytes of one decode step with T cached positions (incl. the new one).

    Every weight matrix once, one embedding row per sequence, the norm gains,
    K and V of T positions read per layer and sequence, the new K/V written.
    """
    s = shape
    qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    per_layer = s.hidden * (qd + 2 * kd) + s.hidden * qd + 3 * s.hidden * s.ffn + 2 * s.hidden
    weights = 2 * (s.n_layers * per_layer + s.vocab * s.hidden + s.hidden)
    emb = 2 * s.hidden * batch
    kv_read = 2 * 2 * s.n_layers * kd * T * batch
    kv_write = 2 * 2 * s.n_layers * kd * batch
    return weights + emb + kv_read + kv_write


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_persistent_megakernel_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
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


def time_decode(abi, h, prompt_t, steps, warmup, torch):
    """Returns (total ms, per-launch kernel ms list)."""
    dev = torch.device("cuda")
    toks = torch.zeros(max(steps, warmup) + 1, dtype=torch.int32, device=dev)
    # warm-up generation
    abi.mk_prefill(h, prompt_t, toks[0:1])
    for s in range(warmup):
        abi.mk_decode_step(h, toks[s:s + 1], toks[s + 1:s + 2])
    abi.mk_synchronize(h)
    abi.mk_reset(h)
    abi.mk_prefill(h, prompt_t, toks[0:1])
    abi.mk_synchronize(h)
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        ev_s[s].record()
        abi.mk_decode_step(h, toks[s:s + 1], toks[s + 1:s + 2])
        ev_e[s].record()
    t1.record()
    torch.cuda.synchronize()
    abi.mk_synchronize(h)
    total = t0.elapsed_time(t1)
    per = [ev_s[i].elapsed_time(ev_e[i]) for i in range(steps)]
    return total, per, toks.cpu().numpy()


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
    dec = D.Decoder(shape, weights, 1, 4, cache_weights=False)
    t = time.perf_counter()
    dec.step(prompt[:, 0])
    ms = (time.perf_counter() - t) * 1000.0
    return {"value": ms, "unit": "ms/token", "cores": int(threads), "kind": "oracle",
            "sample": f"one fp64 decode step of the {shape.name} shape at position 0 (weights widened per use)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-op", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from synth import gen, presets
    from decode_persistent_megakernel_02_amd import abi, runtime

    log = (lambda *a: None) if args.quiet else (lambda *a: print(*a, file=sys.stderr, flush=True))
    wl = presets.WORKLOADS[args.workload]
    shape = wl.shape
    if wl.batch != 1:
        print(f"bench.py: workload {wl.name} (batch {wl.batch}) is not supported yet", file=sys.stderr)
        sys.exit(2)
    steps, warmup = args.steps, args.warmup
    max_seq = wl.prompt_len + max(steps, warmup)
    t = time.time()
    weights = gen.gen_weights(shape, wl.weight_seed)
    log(f"weights generated in {time.time() - t:.1f}s")
    t = time.time()
    dw = runtime.upload_weights(weights)
    torch.cuda.synchronize()
    log(f"weights uploaded in {time.time() - t:.1f}s")
    prompt = gen.gen_prompt(wl)
    prompt_t = torch.from_numpy(prompt).cuda()

    h = runtime.create(shape, dw, max_seq, 1, abi.MK_MODE_MEGAKERNEL)
    total, per, toks = time_decode(abi, h, prompt_t, steps, warmup, torch)
    abi.mk_destroy(h)
    ms = total / steps
    kern_ms = float(np.mean(per))
    bytes_steps = [step_bytes(shape, wl.prompt_len + s + 1) for s in range(steps)]
    alg_bytes = float(np.mean(bytes_steps))
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    bound_ms = alg_bytes / (PEAK_GBPS * 1e9) * 1e3
    log(f"megakernel: {ms:.4f} ms/token (kernel avg {kern_ms:.4f} ms), bound {bound_ms:.4f} ms, "
        f"{achieved:.0f} GB/s")

    per_op = None
    if not args.no_per_op:
        h2 = runtime.create(shape, dw, max_seq, 1, abi.MK_MODE_PER_OP)
        total2, _, toks2 = time_decode(abi, h2, prompt_t, steps, warmup, torch)
        abi.mk_destroy(h2)
        per_op = {"ms_per_step": total2 / steps, "megakernel_speedup": (total2 / steps) / ms,
                  "same_tokens": bool(np.array_equal(toks, toks2))}
        log(f"per-op baseline: {total2 / steps:.4f} ms/token")

    traffic = load_traffic(wl.name)
    res = {
        "metric": METRIC,
        "value": ms,
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: batch 1, prompt {wl.prompt_len}, {steps} greedy decode steps",
                   "batch": 1, "prompt_len": wl.prompt_len, "decode_steps": steps, "mode": "megakernel",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": 1000.0 / ms,
        "achieved_gbps": alg_bytes / (ms * 1e-3) / 1e9,
        "bound_ms_per_token": bound_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBPS, "traffic": traffic, "kernel": "mk_persistent",
                     "kernel_avg_ms": kern_ms, "algorithmic_bytes_per_launch": alg_bytes},
        "per_op_baseline": per_op,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(shape, weights, prompt)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
