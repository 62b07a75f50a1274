"""Batched prefill (MK_FLAG_BATCHED_PREFILL): every prompt position at once,
the projections as bf16 matrix-core GEMMs on split fp32 activations, causal
attention over the cache, in chunks of rows (sequence x position).

Bars:
  * logits of the last prompt position, and of the decode steps that follow
    (they read the cache the prefill wrote), against the fp64 oracle: <= 1e-3
    relative with an fp32 cache; with a bf16 cache <= 1e-3 against the oracle
    that rounds its cache to bf16 (and <= 2e-2 against the exact one);
  * greedy tokens equal wherever the oracle's top-2 margin exceeds 5e-2;
  * the fp32 cache itself against the oracle's K and V: 1e-4 relative;
  * batched against step-by-step prefill of the same weights: logits within
    1e-4 relative, the same greedy tokens.
Small chunks make the prompt cross chunk boundaries; prompts longer than 64
positions cross the attention kernel's key blocks.
"""
import numpy as np
import pytest
import torch

from oracle import decoder as D
from synth import gen, presets
from tests.gpu_util import Case, rel_err
from tests.shapes import MINI, MINI_TIED, MINI_G8, MINI_HD128_G1, MINI_HD128_G2

pytestmark = pytest.mark.gpu

CONTRACT = 2e-2
TIGHT = 1e-3
MARGIN = 5e-2
MEGA, PER_OP = 0, 1


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi as a
    return a


def check(g, r, nxt, bar):
    e = float(rel_err(g, r))
    assert e <= bar, f"logit error {e:.3e} > {bar}"
    if D.top2_margin(r) > MARGIN:
        assert nxt == int(D.greedy(r)), "greedy token differs at a clear margin"
    return e


@pytest.mark.parametrize("mode", [PER_OP, MEGA], ids=["per_op", "megakernel"])
@pytest.mark.parametrize("kv_bf16", [False, True], ids=["kv_f32", "kv_bf16"])
@pytest.mark.parametrize("shape", [MINI, MINI_TIED, MINI_G8, MINI_HD128_G1, MINI_HD128_G2], ids=lambda s: s.name)
def test_single_sequence_then_decode(abi, shape, kv_bf16, mode):
    """70 prompt positions in chunks of 24 (3 chunks, 2 key blocks), then 6
    decode steps on the cache the prefill wrote."""
    print(f"[prefill] {shape.name} kv_bf16={kv_bf16} mode={mode}", flush=True)
    P, steps = 70, 6
    case = Case(shape, P + steps, mode, seed=11, random_norms=True, kv_bf16_oracle=kv_bf16,
                flags=abi.MK_FLAG_BATCHED_PREFILL, watchdog_ms=500 if mode == MEGA else 0)
    abi.mk_t_set_prefill_rows(case.h, 24)
    prompt = gen.tokens(21, 3, 0, P, shape.vocab)
    g, r, nxt = case.prefill(prompt)
    errs = [check(g, r, nxt, TIGHT)]
    feed = gen.tokens(22, 3, 0, steps, shape.vocab)
    for t in feed:
        g, r, nxt = case.step(int(t))
        errs.append(check(g, r, nxt, TIGHT))
    print(f"[prefill] max rel err {max(errs):.2e}", flush=True)


@pytest.mark.parametrize("P,rows", [(67, 1), (67, 5), (67, 64), (67, 4096), (1100, 600)])
def test_cache_matches_oracle(abi, P, rows):
    """The fp32 cache after a batched prefill against the oracle's rotated
    keys and values, every layer and position; chunk sizes from one position
    per chunk to the whole prompt in one.  Chunks of up to 512 rows run each
    projection as one GEMM over the stacked operand parts, larger ones as two
    (1100 positions in chunks of 600: one of each)."""
    shape = MINI_HD128_G2
    case = Case(shape, P, PER_OP, seed=12, random_norms=True, flags=abi.MK_FLAG_BATCHED_PREFILL)
    abi.mk_t_set_prefill_rows(case.h, rows)
    prompt = gen.tokens(23, 3, 0, P, shape.vocab)
    case.prefill(prompt)
    L, nkv, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
    kb = np.empty((L, 1, nkv, P, hd), dtype=np.float32)
    vb = np.empty_like(kb)
    abi.mk_kv_read(case.h, kb, vb)
    for name, got, ref in (("K", kb, case.oracle.K[..., :P, :]), ("V", vb, case.oracle.V[..., :P, :])):
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err <= 1e-4, (name, err)


def test_batched_agrees_with_step_by_step_prefill(abi):
    """The same weights and prompt through both prefills: last-position logits
    within 1e-4 relative, the same greedy token, and the decode steps after
    them too."""
    shape, P = MINI_G8, 45
    w = gen.gen_weights(shape, 13, True)
    prompt = gen.tokens(24, 3, 0, P, shape.vocab)
    outs = []
    for flags in (abi.MK_FLAG_BATCHED_PREFILL, 0):
        case = Case(shape, P + 4, PER_OP, weights=w, flags=flags)
        g, _, nxt = case.prefill(prompt)
        seq = [(g, nxt)]
        for t in (5, 17, 200):
            g, _, nxt = case.step(t)
            seq.append((g, nxt))
        outs.append(seq)
    for (ga, na), (gb, nb) in zip(*outs):
        assert float(rel_err(ga, gb)) <= 1e-4
        assert na == nb


class Batch:
    """B sequences, row-major weights, bf16 cache, batched prefill."""

    def __init__(self, abi, shape, B, max_seq, seed, rows):
        from decode_persistent_megakernel_02_amd import runtime
        self.abi, self.shape, self.B = abi, shape, B
        self.w = gen.gen_weights(shape, seed, True)
        self.dw = runtime.upload_weights(self.w)
        self.h = runtime.create(shape, self.dw, max_seq, B, abi.MK_MODE_PER_OP, abi.MK_FLAG_BATCHED_PREFILL,
                                kv_fp32=False)
        abi.mk_t_set_prefill_rows(self.h, rows)
        self.out = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.tok = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.logits = torch.zeros(B, shape.vocab, dtype=torch.float32, device="cuda")

    def prefill(self, prompt):
        self.abi.mk_prefill(self.h, torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda(), self.out,
                            self.logits)
        self.abi.mk_synchronize(self.h)
        return self.logits.cpu().numpy(), self.out.cpu().numpy()

    def step(self, tokens):
        self.tok.copy_(torch.from_numpy(np.asarray(tokens, dtype=np.int32)))
        self.abi.mk_decode_step(self.h, self.tok, self.out, self.logits)
        self.abi.mk_synchronize(self.h)
        return self.logits.cpu().numpy(), self.out.cpu().numpy()


@pytest.mark.parametrize("shape,B,rows", [(MINI, 2, 64), (MINI_TIED, 5, 16), (MINI_G8, 17, 40),
                                          (MINI_HD128_G1, 3, 4096), (presets.TINY, 8, 100)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_several_sequences_then_decode(abi, shape, B, rows):
    """B sequences of 33 positions (rows // B positions per chunk), then 4
    decode steps, against both oracles."""
    print(f"[prefill] {shape.name} B={B} rows={rows}", flush=True)
    P, steps = 33, 4
    case = Batch(abi, shape, B, P + steps, B, rows)
    prompt = gen.tokens(600 + B, presets.TID_PROMPT, 0, B * P, shape.vocab).reshape(B, P)
    ex = D.Decoder(shape, case.w, B, P + steps)
    rd = D.Decoder(shape, case.w, B, P + steps, kv_bf16=True)
    feed = gen.tokens(700 + B, presets.TID_PROMPT, 0, B * steps, shape.vocab).reshape(steps, B)
    pairs = [(case.prefill(prompt), ex.prefill(prompt), rd.prefill(prompt))]
    for s in range(steps):
        pairs.append((case.step(feed[s]), ex.step(feed[s]), rd.step(feed[s])))
    for (g, nxt), e, r in pairs:
        assert np.all(rel_err(g, e) <= CONTRACT)
        assert np.all(rel_err(g, r) <= TIGHT), rel_err(g, r)
        for b in range(B):
            if D.top2_margin(e[b]) > MARGIN:
                assert nxt[b] == int(D.greedy(e[b]))


def test_prefill_rows_setter_checks_its_range(abi):
    case = Case(MINI, 8, PER_OP, flags=abi.MK_FLAG_BATCHED_PREFILL)
    for bad in (0, 4097):
        with pytest.raises(abi.MkError) as e:
            abi.mk_t_set_prefill_rows(case.h, bad)
        assert e.value.status == abi.MK_ERR_INVALID_ARG
    plain = Case(MINI, 8, PER_OP)
    with pytest.raises(abi.MkError) as e:
        abi.mk_t_set_prefill_rows(plain.h, 16)
    assert e.value.status == abi.MK_ERR_STATE
