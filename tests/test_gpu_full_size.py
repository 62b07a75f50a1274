"""Full-size parity: the Llama-3.2-1B and Llama-3-8B shapes in the launch
configuration the benchmark times (kernel-per-operator mode, every CU).

The oracle cannot afford hundreds of fp64 decode steps at these sizes, so the
GPU decodes seeded random tokens after the seeded 39-token prompt (teacher
forcing with inputs that come from the generator, never from the GPU), and the
oracle's cache-free causal forward over the same sequence gives the expected
logits at every compared position.
"""
import numpy as np
import pytest
import torch

from oracle import decoder as D
from synth import gen, presets
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl_name,kv_fp32", [("llama1b", True), ("llama1b", False), ("llama8b", True)])
def test_full_size_logits_and_tokens(wl_name, kv_fp32):
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
    h = runtime.create(shape, dw, wl.max_seq, mode=abi.MK_MODE_PER_OP, kv_fp32=kv_fp32)
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
    print(f"[{wl_name} kv_fp32={kv_fp32}] max rel err vs fp64 oracle {errs.max():.3e}; vs bf16-KV oracle "
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
