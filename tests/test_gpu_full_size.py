"""Full-size parity: the Llama-3.2-1B and Llama-3-8B shapes in the launch
configurations the benchmark times (the persistent megakernel, one launch per
step, and the kernel-per-operator build; every CU).

The oracle cannot afford hundreds of fp64 decode steps at these sizes, so the
GPU decodes seeded random tokens after the seeded 39-token prompt (teacher
forcing with inputs that come from the generator, never from the GPU), and the
oracle's cache-free causal forward over the same sequence gives the expected
logits at every compared position.
"""
import os

import numpy as np
import pytest
import torch

from oracle import decoder as D
from synth import gen, presets
from tests.gpu_util import d2h, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl_name,kv_fp32,mode", [("llama1b", True, "per_op"), ("llama1b", False, "per_op"),
                                                   ("llama8b", True, "per_op"), ("llama1b", True, "megakernel"),
                                                   ("llama8b", True, "megakernel")])
def test_full_size_logits_and_tokens(wl_name, kv_fp32, mode):
    """fp32 KV cache: compared with the fp64 oracle.  bf16 KV cache: compared
    with the oracle that rounds its cached K/V to bf16 (the storage format)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi, runtime
    wl = presets.WORKLOADS[wl_name]
    shape = wl.shape
    n_dec = 3
    prompt = gen.gen_prompt(wl)[0]
    extra = gen.tokens(77, presets.TID_PROMPT, 0, n_dec, shape.vocab)
    seq = np.concatenate([prompt, extra]).astype(np.int32)
    print(f"[{wl_name}] generating weights", flush=True)
    w = gen.gen_weights(shape, wl.weight_seed)
    dw = runtime.upload_weights(w)
    m = abi.MK_MODE_MEGAKERNEL if mode == "megakernel" else abi.MK_MODE_PER_OP
    h = runtime.create(shape, dw, wl.max_seq, mode=m, kv_fp32=kv_fp32)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")
    got_logits, got_tok = [], []
    abi.mk_prefill(h, torch.from_numpy(prompt.reshape(1, -1)).cuda(), out, lg)
    abi.mk_synchronize(h)
    got_logits.append(lg.cpu().numpy()[0])
    got_tok.append(int(out.item()))
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t in extra:
        tok.fill_(int(t))
        abi.mk_decode_step(h, tok, out, lg)
        abi.mk_synchronize(h)
        got_logits.append(lg.cpu().numpy()[0])
        got_tok.append(int(out.item()))
    abi.mk_destroy(h)
    del dw
    print(f"[{wl_name}] oracle forward", flush=True)
    ref = D.forward_full(shape, w, seq[None, :])[0]         # [T, V]
    ref = ref[len(prompt) - 1:]                              # positions compared
    ref_kv = D.forward_full(shape, w, seq[None, :], kv_bf16=True)[0][len(prompt) - 1:]
    errs = rel_err(np.stack(got_logits), ref)
    errs_kv = rel_err(np.stack(got_logits), ref_kv)
    kv_only = rel_err(ref_kv, ref)
    print(f"[{wl_name} kv_fp32={kv_fp32} {mode}] max rel err vs fp64 oracle {errs.max():.3e}; vs bf16-KV oracle "
          f"{errs_kv.max():.3e}; bf16-KV oracle vs fp64 oracle {kv_only.max():.3e}", flush=True)
    mine = errs if kv_fp32 else errs_kv
    assert np.all(mine <= 2e-2)   # the contract
    assert np.all(mine <= 5e-3)   # fp32 accumulation-order level
    for s in range(n_dec + 1):
        r = ref[s] if kv_fp32 else ref_kv[s]
        if D.top2_margin(r) > 5e-2:
            assert got_tok[s] == int(D.greedy(r))


def test_batched_workload_long_cache_full_depth():
    """The 8B-shape batched workload at full depth and context: 8 sequences
    prefilled with their 4096-token seeded prompts on the GPU (tiled weights,
    bf16 cache, the bench's launch configuration), then one seeded decode
    step.  The oracle imports the GPU's bf16 cache through mk_kv_read and
    runs the same step in fp64 from it, so the comparison covers every layer
    of the decode step at a 4097-position context (the prefill itself is
    covered by the other tests)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi, runtime
    wl = presets.WORKLOADS["llama8b_b8_kv4096"]
    shape, B, P = wl.shape, wl.batch, wl.prompt_len
    max_seq = P + 1
    prompt = gen.gen_prompt(wl)
    step_tok = gen.tokens(78, presets.TID_PROMPT, 0, B, shape.vocab).astype(np.int32)
    print(f"[c4 full depth] generating weights", flush=True)
    w = gen.gen_weights(shape, wl.weight_seed)
    dw = runtime.upload_weights(w, tiled=True)
    h = runtime.create(shape, dw, max_seq, B, abi.MK_MODE_PER_OP, abi.MK_FLAG_TILED_WEIGHTS, kv_fp32=False)
    out = torch.zeros(B, dtype=torch.int32, device="cuda")
    lg = torch.zeros(B, shape.vocab, dtype=torch.float32, device="cuda")
    print(f"[c4 full depth] prefill {B} x {P} on the GPU", flush=True)
    abi.mk_prefill(h, torch.from_numpy(prompt).cuda(), out, lg)
    abi.mk_synchronize(h)
    L, nkv, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
    kb = np.empty((L, B, nkv, max_seq, hd), dtype=np.uint16)
    vb = np.empty_like(kb)
    abi.mk_kv_read(h, kb, vb)
    tok = torch.from_numpy(step_tok).cuda()
    abi.mk_decode_step(h, tok, out, lg)
    abi.mk_synchronize(h)
    got = lg.cpu().numpy()
    got_tok = out.cpu().numpy()
    abi.mk_destroy(h)
    del dw
    print(f"[c4 full depth] oracle step from the imported cache", flush=True)
    ora = D.Decoder(shape, w, B, max_seq, cache_weights=False, kv_bf16=True)
    ora.K[:, :, :, :P] = D.widen_bf16(kb[:, :, :, :P])
    ora.V[:, :, :, :P] = D.widen_bf16(vb[:, :, :, :P])
    del kb, vb
    ora.length = P
    ref = ora.step(step_tok)
    errs = rel_err(got, ref)
    print(f"[c4 full depth] max rel err vs the bf16-KV oracle {errs.max():.3e}", flush=True)
    assert np.all(errs <= 2e-2)   # the contract
    assert np.all(errs <= 5e-3)   # fp32 accumulation order and the hi/lo operand split
    for b in range(B):
        if D.top2_margin(ref[b]) > 5e-2:
            assert got_tok[b] == int(D.greedy(ref[b]))


def test_megakernel_8b_bench_workload_layers_at_longest_context_against_oracle():
    """The benchmark's own run, checked where its context is longest: the 8B
    shape in megakernel mode (fp32 cache, the library's attention split: 18
    live splits at 551 positions), the seeded 39-token prompt, 511 greedy steps
    in one launch, then one step more at position 550.  The oracle takes the
    GPU's residual stream entering layers 0 (the embedding row), 1, 16, 30 and
    31 (the hand-over words of that step, every one carrying its epoch) and
    those layers' GPU cache (mk_kv_read), runs each layer in fp64, and
    compares the residual stream leaving it with the GPU's; then the final
    norm and LM head on the GPU's last residual stream against the GPU's
    logits.  fp32 arithmetic and cache against fp64: 1e-4."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi, runtime
    wl = presets.WORKLOADS["llama8b"]
    shape, P, S = wl.shape, wl.prompt_len, wl.decode_steps
    max_seq, layers, tag = P + S, (0, 1, 16, 30, 31), "8b mega longest context"
    L, nkv, hd, H = shape.n_layers, shape.n_kv_heads, shape.head_dim, shape.hidden
    print(f"[{tag}] generating weights", flush=True)
    w = gen.gen_weights(shape, wl.weight_seed)
    dw = runtime.upload_weights(w)
    h = runtime.create(shape, dw, max_seq, mode=abi.MK_MODE_MEGAKERNEL)
    toks = torch.zeros(S + 1, dtype=torch.int32, device="cuda")
    lg = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")
    print(f"[{tag}] prefill {P}, {S - 1} steps in one launch, one step more", flush=True)
    abi.mk_prefill(h, torch.from_numpy(gen.gen_prompt(wl)).cuda(), toks[0:1])
    abi.mk_generate(h, toks[0:1], S - 1, toks[1:S])
    abi.mk_decode_step(h, toks[S - 1:S], toks[S:S + 1], lg)
    abi.mk_synchronize(h)
    last_tok = int(toks[S - 1].item())
    kf = np.empty((L, 1, nkv, max_seq, hd), dtype=np.float32)
    vf = np.empty_like(kf)
    abi.mk_kv_read(h, kf, vf)
    v = abi.mk_get_mega_view(h)
    xw = np.empty((L + 1) * H, dtype=np.uint64)
    d2h(xw.ctypes.data, v.x, xw.nbytes)
    assert np.all((xw[H:] >> np.uint64(32)) == v.epoch), "a word without the last step's epoch"
    xs = (xw & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).astype(np.float64).reshape(L + 1, 1, H)
    got = lg.cpu().numpy()
    abi.mk_destroy(h)
    del dw
    p = max_seq - 1
    ora = D.Decoder(shape, w, 1, max_seq, cache_weights=False)
    for l in layers:
        ora.K[l, :, :, :p] = kf[l, :, :, :p]
        ora.V[l, :, :, :p] = vf[l, :, :, :p]
    for l in layers:
        x_in = D.widen_bf16(w["embed"][[last_tok]]) if l == 0 else xs[l]
        err = rel_err(xs[l + 1], ora.layer(l, x_in, p))
        print(f"[{tag}] layer {l}: residual stream after it, max rel err {err.max():.3e}", flush=True)
        assert np.all(err <= 1e-4), (l, err)
    errs = rel_err(got, ora.head(xs[L]))
    print(f"[{tag}] LM head on the last residual stream: max rel logit err {errs.max():.3e}", flush=True)
    assert np.all(errs <= 1e-4)


class _RegeneratedWeights:
    """The oracle's weight table for a shape too large to hold: every access
    regenerates the tensor from the seeded generator (the bits the GPU was
    given); the oracle widens it, uses it and drops it."""

    def __init__(self, shape, seed, tag):
        self.shape, self.seed, self.tag = shape, seed, tag

    def __getitem__(self, name):
        print(f"[{self.tag}] oracle: {name}", flush=True)
        return gen.gen_weight(self.shape, name, self.seed)


def test_batched_70b_workload_layers_at_full_depth_against_oracle():
    """The 70B-shape batched workload at full depth and context: 64 sequences
    prefilled with their 512-token seeded prompts (batched prefill, bf16
    cache), then one seeded decode step for all of them.  A full fp64 oracle
    step at this shape widens 141 GB of weights on the host (most of an hour),
    so the oracle checks the step layer by layer instead: for two sequences it
    takes the GPU's residual stream entering layers 0 (the embedding row), 1,
    39, 78 and 79 and the GPU's cache of those layers (mk_kv_read), runs each layer
    in fp64 with its weights regenerated from the seeded generator, and
    compares the residual stream the layer leaves with the GPU's; then the
    final norm and LM head on the GPU's last residual stream against the
    GPU's logits.  Every compared layer sees the 513-position context
    (measured: 1.1e-5 at layer 0, below 1e-6 at layers 39 and 79, 2.6e-6 on
    the logits; about 40 s on the GPU machine)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi, runtime
    wl = presets.WORKLOADS["llama70b_b64"]
    shape, B, P = wl.shape, wl.batch, wl.prompt_len
    max_seq, rows, layers = P + 1, 2, (0, 1, 39, 78, 79)
    tag = "c5 layers"
    step_tok = gen.tokens(79, presets.TID_PROMPT, 0, B, shape.vocab).astype(np.int32)
    print(f"[{tag}] generating weights on the device", flush=True)
    dw = runtime.generate_device_weights(shape, wl.weight_seed)
    h = runtime.create(shape, dw, max_seq, B, abi.MK_MODE_PER_OP, abi.MK_FLAG_BATCHED_PREFILL, kv_fp32=False)
    out = torch.zeros(B, dtype=torch.int32, device="cuda")
    lg = torch.zeros(B, shape.vocab, dtype=torch.float32, device="cuda")
    print(f"[{tag}] prefill {B} x {P}, then one decode step", flush=True)
    abi.mk_prefill(h, torch.from_numpy(gen.gen_prompt(wl)).cuda(), out, lg)
    abi.mk_synchronize(h)
    L, nkv, hd, H = shape.n_layers, shape.n_kv_heads, shape.head_dim, shape.hidden
    kb = np.empty((L, B, nkv, max_seq, hd), dtype=np.uint16)
    vb = np.empty_like(kb)
    abi.mk_kv_read(h, kb, vb)
    abi.mk_decode_step(h, torch.from_numpy(step_tok).cuda(), out, lg)
    abi.mk_synchronize(h)
    xs = np.empty((L + 1) * B * H, dtype=np.float32)
    d2h(xs.ctypes.data, abi.mk_get_debug_view(h).xs, xs.nbytes)
    xs = xs.reshape(L + 1, B, H)[:, :rows].astype(np.float64)
    got = lg.cpu().numpy()[:rows]
    abi.mk_destroy(h)
    del dw
    torch.cuda.empty_cache()
    ora = D.Decoder(shape, _RegeneratedWeights(shape, wl.weight_seed, tag), rows, max_seq, cache_weights=False,
                    kv_bf16=True)
    tid = presets.tensor_id("embed")
    for l in layers:
        ora.K[l, :, :, :P] = D.widen_bf16(kb[l, :rows, :, :P])
        ora.V[l, :, :, :P] = D.widen_bf16(vb[l, :rows, :, :P])
    del kb, vb
    for l in layers:
        if l == 0:  # the embedding rows of the step's tokens
            x_in = np.stack([D.widen_bf16(gen.bf16_normal(wl.weight_seed, tid, int(t) * H, H)) for t in step_tok[:rows]])
        else:
            x_in = xs[l]
        x_out = ora.layer(l, x_in, P)
        err = rel_err(xs[l + 1], x_out)
        print(f"[{tag}] layer {l}: residual stream after it, max rel err {err.max():.3e}", flush=True)
        assert np.all(err <= 1e-3), (l, err)
    ref = ora.head(xs[L])
    errs = rel_err(got, ref)
    print(f"[{tag}] LM head on the last residual stream: max rel logit err {errs.max():.3e}", flush=True)
    assert np.all(errs <= 1e-3)


_W8X2 = {}


def _weights_8b_two_layers(shape):
    if "w" not in _W8X2:
        _W8X2["w"] = gen.gen_weights(shape, 1002)
    return _W8X2["w"]


@pytest.mark.parametrize("mode,batched_prefill", [("megakernel", False), ("per_op", False), ("megakernel", True),
                                                   ("per_op", True)],
                         ids=["megakernel", "per_op", "megakernel_batched_prefill", "per_op_batched_prefill"])
def test_8b_shape_two_layers_multi_split_attention(mode, batched_prefill):
    """The 8B production attention instance (fp32 cache, 4 query heads per KV
    head, head_dim 128) with several splits live: two layers of the 8B shape,
    a 140-token seeded prompt and 3 seeded decode steps (context up to 143:
    3 live splits at the per-operator default of 64 positions, 5 at the
    megakernel's 32), each mode with the library's default split and every
    CU.  Logits at the last prompt position and every decode step against the
    oracle's cache-free forward at 5e-3.  With the batched prefill the 140
    prompt positions run as one chunk of matrix-core GEMMs and the decode
    steps read the cache it wrote."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi, runtime
    shape = presets.with_layers(presets.LLAMA8B, 2)
    P, n_dec = 140, 3
    seq = gen.tokens(2024, presets.TID_PROMPT, 0, P + n_dec, shape.vocab).astype(np.int32)
    print(f"[8b x2 {mode}] generating weights", flush=True)
    w = _weights_8b_two_layers(shape)
    dw = runtime.upload_weights(w)
    m = abi.MK_MODE_MEGAKERNEL if mode == "megakernel" else abi.MK_MODE_PER_OP
    h = runtime.create(shape, dw, P + n_dec + 1, mode=m, flags=abi.MK_FLAG_BATCHED_PREFILL if batched_prefill else 0,
                       kv_fp32=True)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")
    got = []
    abi.mk_prefill(h, torch.from_numpy(seq[:P].reshape(1, -1)).cuda(), out, lg)
    abi.mk_synchronize(h)
    got.append(lg.cpu().numpy()[0])
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t in seq[P:]:
        tok.fill_(int(t))
        abi.mk_decode_step(h, tok, out, lg)
        abi.mk_synchronize(h)
        got.append(lg.cpu().numpy()[0])
    split = abi.mk_get_debug_view(h).split
    abi.mk_destroy(h)
    del dw
    live = (P + n_dec + split - 1) // split
    print(f"[8b x2 {mode}] split {split}: {live} splits live at the last step; oracle forward", flush=True)
    assert live >= 3
    ref = D.forward_full(shape, w, seq[None, :P + n_dec], positions=range(P - 1, P + n_dec))[0]
    errs = rel_err(np.stack(got), ref)
    print(f"[8b x2 {mode}] max rel err {errs.max():.3e}", flush=True)
    assert np.all(errs <= 5e-3)


@pytest.mark.timeout(1100)
@pytest.mark.parametrize("name", [
    "llama8b_b8_kv4096",
    pytest.param("llama70b_b64", marks=pytest.mark.skipif(
        os.environ.get("MK_LONG_TESTS") != "1",
        reason="about 5 minutes (141 GB of weights generated on the host, 512 step-by-step decode steps); "
               "run with MK_LONG_TESTS=1"))])
def test_batched_prefill_full_depth_agrees_with_step_by_step(name):
    """A batched workload at full depth: its seeded prompts (8 x 4096 at the
    8B shape, 64 x 512 at the 70B shape) prefilled both ways on the GPU
    (row-major weights, bf16 cache): batched (chunks of 4096 rows, matrix-core
    GEMMs and attention) and one decode step per position.  The two differ by
    the bf16 rounding of cache values that their fp32 summation orders leave
    slightly apart, and that difference grows with depth: at the 8B shape (32
    layers) the caches agree layer by layer within 1e-2 (norm of the
    difference over the norm) and the last-position logits within 5e-3; at
    the 70B shape (80 layers; 1.0e-2 measured) the logits are held to the
    scope's 2e-2 contract, which each path meets against the oracle, and the
    caches to 2e-2.  Greedy ids agree at clear margins.  The fp64
    oracle cannot recompute these prompts on the host (one oracle step of the
    70B shape widens 141 GB of weights); the step-by-step path is held against
    it at every other size."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi, runtime
    wl = presets.WORKLOADS[name]
    shape, B, P = wl.shape, wl.batch, wl.prompt_len
    prompt = torch.from_numpy(gen.gen_prompt(wl)).cuda()
    print(f"[prefill full depth {name}] generating weights", flush=True)
    dw = runtime.generate_device_weights(shape, wl.weight_seed)
    L, nkv, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
    got = []
    for flags in (abi.MK_FLAG_BATCHED_PREFILL, 0):
        print(f"[prefill full depth {name}] prefill {B} x {P}, flags {flags}", flush=True)
        h = runtime.create(shape, dw, P, B, abi.MK_MODE_PER_OP, flags, kv_fp32=False)
        out = torch.zeros(B, dtype=torch.int32, device="cuda")
        lg = torch.zeros(B, shape.vocab, dtype=torch.float32, device="cuda")
        abi.mk_prefill(h, prompt, out, lg)
        abi.mk_synchronize(h)
        kb = np.empty((L, B, nkv, P, hd), dtype=np.uint16)
        vb = np.empty_like(kb)
        abi.mk_kv_read(h, kb, vb)
        abi.mk_destroy(h)
        got.append((kb, vb, lg.cpu().numpy(), out.cpu().numpy()))
    del dw
    (ka, va, la, ia), (kb, vb, lb, ib) = got
    cache_bar, logit_bar = (1e-2, 5e-3) if shape.n_layers <= 32 else (2e-2, 2e-2)
    worst = 0.0
    for l in range(L):
        for nm, a, b in (("K", ka[l], kb[l]), ("V", va[l], vb[l])):
            a, b = D.widen_bf16(a), D.widen_bf16(b)
            err = np.linalg.norm(a - b) / np.linalg.norm(b)
            worst = max(worst, err)
            assert err <= cache_bar, (nm, l, err)
    errs = rel_err(la, lb)
    print(f"[prefill full depth {name}] cache: worst layer {worst:.3e}; last-position logits: "
          f"max rel diff {errs.max():.3e}", flush=True)
    assert np.all(errs <= logit_bar)
    for b in range(B):
        if D.top2_margin(lb[b].astype(np.float64)) > 5e-2:
            assert ia[b] == ib[b]
