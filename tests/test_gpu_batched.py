"""Batched decode (several sequences per step) on the GPU against the oracle.

The batched path keeps a bf16 KV cache (the batched workloads state one) and
feeds the matrix cores activations as bf16 hi + lo pairs (16 significant
bits, relative error <= 2^-17).  Bars:
  * against the fp64 oracle: max|gpu - oracle| / max|oracle| <= 2e-2 per step
    and row (the contract);
  * against the oracle that rounds its cached K/V to bf16 the same way
    (kv_bf16): <= 1e-3 at test sizes and 5e-3 at the workloads' layer shapes,
    the bars of the batch-1 path -- what remains is fp32 accumulation order
    and the operand split;
  * greedy tokens equal wherever the oracle's top-2 margin exceeds 5e-2.
"""
import numpy as np
import pytest
import torch

from oracle import decoder as D
from synth import gen, presets
from tests.gpu_util import rel_err
from tests.shapes import (MINI, MINI_G8, MINI_HD128_G1, MINI_HD128_G2, MINI_TIED, MINI_TILE, MINI_TILE_G8,
                          MINI_TILE_TIED)

pytestmark = pytest.mark.gpu

CONTRACT = 2e-2
TIGHT = 1e-3
TIGHT_FULL = 5e-3
MARGIN = 5e-2


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi as a
    return a


def padded_rows(B):
    return 16 if B <= 16 else 32 if B <= 32 else 64


# ---- the matrix-core projection body ---------------------------------------------
BGEMM_CASES = [(16, 32, 1), (50, 264, 3), (300, 4096, 8), (64, 520, 16), (48, 2048, 17), (33, 1032, 40),
               (128, 8192, 64), (17, 28672, 5)]


@pytest.mark.parametrize("N,K,B", BGEMM_CASES)
def test_bgemm_exact(abi, N, K, B):
    """Exactly representable data (weights k/16, |k| <= 8; activations hi = a
    small integer, lo = a multiple of 1/256 below 1/2): every fp32 partial sum
    is exact, so the result is bit-exact."""
    rng = np.random.default_rng(N * 7 + K + B)
    W = (rng.integers(-8, 9, size=(N, K)) / 16.0).astype(np.float32)
    A = np.zeros((2, padded_rows(B), K), dtype=np.float32)
    A[0, :B] = rng.integers(-8, 9, size=(B, K))
    A[1, :B] = rng.integers(-127, 128, size=(B, K)) / 256.0
    ref = (A[0, :B].astype(np.float64) + A[1, :B]) @ W.astype(np.float64).T
    Wd = torch.from_numpy(W).to(torch.bfloat16).cuda()
    Ad = torch.from_numpy(A).to(torch.bfloat16).cuda()
    Y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    print(f"bgemm exact N={N} K={K} B={B}", flush=True)
    abi.mk_t_bgemm(Wd, Ad, Y, B)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("N,K,B", [(300, 4096, 8), (96, 14336, 64), (40, 8192, 33)])
def test_bgemm_random(abi, N, K, B):
    """fp32 activations split into hi + lo planes (by torch's own rounding):
    within a few fp32 accumulation ulps of the fp64 product of the fp32
    values (the split keeps 16 significant bits: <= 2^-17 relative)."""
    rng = np.random.default_rng(5 + N + K + B)
    W = torch.from_numpy(rng.normal(0, 0.02, size=(N, K)).astype(np.float32)).to(torch.bfloat16)
    a = torch.from_numpy(rng.normal(0, 1, size=(B, K)).astype(np.float32))
    A = torch.zeros(2, padded_rows(B), K, dtype=torch.bfloat16)
    A[0, :B] = a.to(torch.bfloat16)
    A[1, :B] = (a - A[0, :B].float()).to(torch.bfloat16)
    ref = a.double().numpy() @ W.double().numpy().T
    Y = torch.zeros(B, N, dtype=torch.float32, device="cuda")
    abi.mk_t_bgemm(W.cuda(), A.cuda(), Y, B)
    torch.cuda.synchronize()
    err = np.abs(Y.cpu().numpy() - ref).max() / np.abs(ref).max()
    print(f"bgemm random N={N} K={K} B={B}: {err:.2e}")
    assert err <= 2e-5, err


def tile_ref(bits):
    """The tiled layout of a row-major [N, K] array, written from its definition:
    block (i, j) at (i * K/32 + j) * 512 holds at 8 l + e the element
    W[16 i + l % 16][32 j + 8 (l // 16) + e]."""
    N, K = bits.shape
    out = np.empty(N * K, dtype=bits.dtype)
    for i in range(N // 16):
        for j in range(K // 32):
            base = (i * (K // 32) + j) * 512
            for l in range(64):
                out[base + 8 * l: base + 8 * l + 8] = bits[16 * i + l % 16, 32 * j + 8 * (l // 16): 32 * j + 8 * (l // 16) + 8]
    return out


@pytest.mark.parametrize("N,K", [(16, 32), (48, 96), (336, 128)])
def test_tile_layout_matches_its_definition(abi, N, K):
    bits = np.random.default_rng(N + K).integers(0, 1 << 16, size=(N, K), dtype=np.uint64).astype(np.uint16)
    src = torch.from_numpy(bits.view(np.int16)).cuda()
    dst = torch.empty_like(src)
    abi.mk_tile_weights(src, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint16).reshape(-1), tile_ref(bits))


@pytest.mark.parametrize("N,K,B", [(16, 32, 1), (300 - 12, 4096, 8), (64, 512, 16), (48, 2048, 17), (128, 8192, 64),
                                   (32, 28672, 5)])
def test_bgemm_tiled_equals_row_major(abi, N, K, B):
    """The same products from tiled weights: bit-identical to the row-major path
    (the matrix cores see the same operands in the same order)."""
    from decode_persistent_megakernel_02_amd import runtime
    rng = np.random.default_rng(N + 3 * K + B)
    W = torch.from_numpy(rng.normal(0, 0.02, size=(N, K)).astype(np.float32)).to(torch.bfloat16).cuda()
    a = torch.from_numpy(rng.normal(0, 1, size=(B, K)).astype(np.float32))
    A = torch.zeros(2, padded_rows(B), K, dtype=torch.bfloat16)
    A[0, :B] = a.to(torch.bfloat16)
    A[1, :B] = (a - A[0, :B].float()).to(torch.bfloat16)
    A = A.cuda()
    Y0 = torch.zeros(B, N, dtype=torch.float32, device="cuda")
    Y1 = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    abi.mk_t_bgemm(W, A, Y0, B)
    abi.mk_t_bgemm(runtime.tile(W), A, Y1, B, tiled=True)
    torch.cuda.synchronize()
    assert np.array_equal(Y0.cpu().numpy(), Y1.cpu().numpy())


# ---- end-to-end batched decode -------------------------------------------------------
class BatchCase:
    """One batched model on the GPU; the oracles run on the same seeded inputs."""

    def __init__(self, abi, shape, B, max_seq, seed=0, random_norms=True, attn_split=0, weights=None, tiled=False,
                 batched_prefill=False):
        from decode_persistent_megakernel_02_amd import runtime
        self.abi, self.shape, self.B = abi, shape, B
        self.w = weights if weights is not None else gen.gen_weights(shape, seed, random_norms)
        self.dw = runtime.upload_weights(self.w, tiled=tiled)
        flags = (abi.MK_FLAG_TILED_WEIGHTS if tiled else 0) | (abi.MK_FLAG_BATCHED_PREFILL if batched_prefill else 0)
        self.h = runtime.create(shape, self.dw, max_seq, B, abi.MK_MODE_PER_OP, flags, attn_split=attn_split,
                                kv_fp32=False)
        self.out = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.tok = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.logits = torch.zeros(B, shape.vocab, dtype=torch.float32, device="cuda")

    def prefill(self, prompt):
        p = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
        self.abi.mk_prefill(self.h, p, self.out, self.logits)
        self.abi.mk_synchronize(self.h)
        return self.logits.cpu().numpy(), self.out.cpu().numpy()

    def step(self, tokens):
        self.tok.copy_(torch.from_numpy(np.asarray(tokens, dtype=np.int32)))
        self.abi.mk_decode_step(self.h, self.tok, self.out, self.logits)
        self.abi.mk_synchronize(self.h)
        return self.logits.cpu().numpy(), self.out.cpu().numpy()

    def close(self):
        self.abi.mk_destroy(self.h)


def check(g, nxt, exact, rounded, errs, tight=TIGHT):
    e_c = rel_err(g, exact)
    e_t = rel_err(g, rounded)
    errs.append((float(e_c.max()), float(e_t.max())))
    assert np.all(e_c <= CONTRACT), e_c
    assert np.all(e_t <= tight), e_t
    for b in range(len(nxt)):
        if D.top2_margin(exact[b]) > MARGIN:
            assert nxt[b] == int(D.greedy(exact[b])), f"row {b}: greedy token differs at a clear margin"


def run_teacher_forced(case, prompt, steps, seed=99):
    """Prefill, then `steps` decode steps fed with seeded tokens; the two
    oracles (plain fp64, and with the bf16 KV cache) follow the same inputs."""
    shape, B = case.shape, case.B
    P = prompt.shape[1]
    ex = D.Decoder(shape, case.w, B, P + steps)
    rd = D.Decoder(shape, case.w, B, P + steps, kv_bf16=True)
    errs = []
    g, nxt = case.prefill(prompt)
    check(g, nxt, ex.prefill(prompt), rd.prefill(prompt), errs)
    feed = gen.tokens(seed, presets.TID_PROMPT, 0, B * steps, shape.vocab).reshape(steps, B)
    for s in range(steps):
        g, nxt = case.step(feed[s])
        check(g, nxt, ex.step(feed[s]), rd.step(feed[s]), errs)
    return errs


@pytest.mark.parametrize("shape,B", [(MINI, 2), (MINI, 8), (MINI_TIED, 17), (MINI_G8, 33), (presets.TINY, 64),
                                     (MINI_HD128_G1, 5), (MINI_HD128_G2, 3)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_batched_teacher_forced(abi, shape, B):
    prompt = gen.tokens(500 + B, presets.TID_PROMPT, 0, B * 9, shape.vocab).reshape(B, 9)
    print(f"batched {shape.name} B={B}", flush=True)
    case = BatchCase(abi, shape, B, 9 + 6, seed=B)
    errs = run_teacher_forced(case, prompt, 6)
    case.close()
    print(f"batched {shape.name} B={B}: max rel err vs fp64 {max(e[0] for e in errs):.2e}, "
          f"vs bf16-KV oracle {max(e[1] for e in errs):.2e}", flush=True)


def test_batched_many_splits(abi):
    """Context spanning many 16-position attention splits, ragged last split."""
    B, P, steps = 3, 53, 4
    prompt = gen.tokens(71, presets.TID_PROMPT, 0, B * P, MINI.vocab).reshape(B, P)
    case = BatchCase(abi, MINI, B, P + steps, seed=3, attn_split=16)
    errs = run_teacher_forced(case, prompt, steps)
    case.close()
    print(f"many splits: vs bf16-KV oracle {max(e[1] for e in errs):.2e}", flush=True)


def test_batched_many_splits_matrix_core_scores(abi):
    """The matrix-core score path (bf16 cache, head_dim 128) over many
    16-position splits: one block per split, three idle waves in each
    workgroup, a ragged last split."""
    B, P, steps = 3, 53, 4
    prompt = gen.tokens(73, presets.TID_PROMPT, 0, B * P, MINI_HD128_G2.vocab).reshape(B, P)
    case = BatchCase(abi, MINI_HD128_G2, B, P + steps, seed=5, attn_split=16)
    errs = run_teacher_forced(case, prompt, steps)
    case.close()
    print(f"many splits, matrix-core scores: vs bf16-KV oracle {max(e[1] for e in errs):.2e}", flush=True)


def test_batched_free_running_matches_oracle(abi):
    """Free-running greedy generation: the sequences agree up to the first
    step where the oracle's top-2 margin is at most 5e-2."""
    shape, B, P, steps = MINI_TIED, 4, 7, 10
    prompt = gen.tokens(31, presets.TID_PROMPT, 0, B * P, shape.vocab).reshape(B, P)
    case = BatchCase(abi, shape, B, P + steps, seed=8)
    ex = D.Decoder(shape, case.w, B, P + steps)
    g, nxt = case.prefill(prompt)
    ref = ex.prefill(prompt)
    alive = np.ones(B, dtype=bool)
    for _ in range(steps):
        want = D.greedy(ref)
        alive &= D.top2_margin(ref) > MARGIN
        assert np.all(nxt[alive] == want[alive])
        g, nxt = case.step(nxt)
        ref = ex.step(np.where(alive, want, nxt))
    case.close()


def test_batch_rows_are_independent(abi):
    """Permuting the batch rows permutes the outputs bit for bit, and two rows
    holding the same sequence give identical logits."""
    shape, B, P = MINI, 6, 5
    prompt = gen.tokens(41, presets.TID_PROMPT, 0, B * P, shape.vocab).reshape(B, P)
    prompt[4] = prompt[1]
    perm = np.array([3, 0, 5, 1, 4, 2])
    a = BatchCase(abi, shape, B, P + 2, seed=2)
    ga, _ = a.prefill(prompt)
    ga2, _ = a.step(prompt[:, 0])
    b = BatchCase(abi, shape, B, P + 2, weights=a.w)
    gb, _ = b.prefill(prompt[perm])
    gb2, _ = b.step(prompt[perm, 0])
    a.close()
    b.close()
    assert np.array_equal(ga[perm], gb) and np.array_equal(ga2[perm], gb2)
    assert np.array_equal(ga[1], ga[4]) and np.array_equal(ga2[1], ga2[4])


def test_batched_graph_replay_equals_eager(abi):
    """The captured step graph, eager launches, and the attention merge run by
    the last split workgroup instead of its own launch all give identical
    results (4-position splits)."""
    from decode_persistent_megakernel_02_amd import runtime
    shape, B, P = MINI, 5, 6
    w = gen.gen_weights(shape, 4, True)
    dw = runtime.upload_weights(w)
    prompt = torch.from_numpy(gen.tokens(3, presets.TID_PROMPT, 0, B * P, shape.vocab).reshape(B, P)).cuda()
    res = []
    for flags in (0, abi.MK_FLAG_NO_GRAPH, abi.MK_FLAG_FUSED_MERGE):
        h = runtime.create(shape, dw, P + 8, B, abi.MK_MODE_PER_OP, flags, attn_split=4, kv_fp32=False)
        out = torch.zeros(B, dtype=torch.int32, device="cuda")
        lg = torch.zeros(B, shape.vocab, dtype=torch.float32, device="cuda")
        abi.mk_prefill(h, prompt, out, lg)
        for _ in range(8):
            abi.mk_decode_step(h, out, out, lg)  # free-running, device-side feedback
        abi.mk_synchronize(h)
        res.append((out.cpu().numpy().copy(), lg.cpu().numpy().copy()))
        abi.mk_destroy(h)
    for r in res[1:]:
        assert np.array_equal(res[0][0], r[0]) and np.array_equal(res[0][1], r[1])


def test_batched_operator_replay_leaves_the_batch_unchanged(abi):
    """Replaying the norm, attention and projection launches (with their
    split-K finishing launches) between steps changes no later result bit; the
    QKV launches (they append to the KV cache), LM head and argmax are refused."""
    from decode_persistent_megakernel_02_amd import runtime
    shape, B, P = MINI, 6, 5
    w = gen.gen_weights(shape, 8, True)
    dw = runtime.upload_weights(w)
    prompt = torch.from_numpy(gen.tokens(8, presets.TID_PROMPT, 0, B * P, shape.vocab).reshape(B, P)).cuda()
    res = []
    for replay in (False, True):
        h = runtime.create(shape, dw, P + 8, B, abi.MK_MODE_PER_OP, 0, attn_split=4, kv_fp32=False)
        out = torch.zeros(B, dtype=torch.int32, device="cuda")
        lg = torch.zeros(B, shape.vocab, dtype=torch.float32, device="cuda")
        abi.mk_prefill(h, prompt, out, lg)
        steps = []
        for _ in range(6):
            if replay:
                for name in ("norm", "attn", "merge", "o", "gu", "down"):
                    ms, n = abi.mk_time_op_replay(h, name, 2)
                    assert n >= 2 * shape.n_layers and ms > 0.0, (name, n, ms)
                for name in ("qkv", "lm", "argmax"):  # KV append / argmax state
                    with pytest.raises(abi.MkError):
                        abi.mk_time_op_replay(h, name, 1)
            abi.mk_decode_step(h, out, out, lg)
            abi.mk_synchronize(h)
            steps.append(lg.cpu().numpy().copy())
        res.append(np.stack(steps))
        abi.mk_destroy(h)
    assert np.array_equal(res[0], res[1])


@pytest.mark.parametrize("shape,B", [(MINI_TILE, 5), (MINI_TILE_TIED, 20), (MINI_TILE_G8, 40)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_batched_tiled_weights_equal_row_major(abi, shape, B):
    """Decoding from tiled weights gives the same bits as from row-major ones
    (teacher-forced, prefill plus seeded steps), and both match the oracle."""
    P, steps = 7, 4
    prompt = gen.tokens(40 + B, presets.TID_PROMPT, 0, B * P, shape.vocab).reshape(B, P)
    feed = gen.tokens(41 + B, presets.TID_PROMPT, 0, B * steps, shape.vocab).reshape(steps, B)
    w = gen.gen_weights(shape, B, True)
    runs = []
    for tiled in (False, True):
        print(f"{shape.name} B={B} tiled={tiled}", flush=True)
        case = BatchCase(abi, shape, B, P + steps, weights=w, tiled=tiled)
        res = [case.prefill(prompt)[0]]
        for s in range(steps):
            res.append(case.step(feed[s])[0])
        case.close()
        runs.append(np.stack(res))
    assert np.array_equal(runs[0], runs[1])
    ex = D.Decoder(shape, w, B, P + steps)
    rd = D.Decoder(shape, w, B, P + steps, kv_bf16=True)
    errs = []
    refs = [(ex.prefill(prompt), rd.prefill(prompt))] + [(ex.step(feed[s]), rd.step(feed[s])) for s in range(steps)]
    for g, (e, r) in zip(runs[1], refs):
        e_c, e_t = rel_err(g, e), rel_err(g, r)
        errs.append((float(e_c.max()), float(e_t.max())))
    assert max(e[0] for e in errs) <= CONTRACT and max(e[1] for e in errs) <= TIGHT, errs


def layer_subset(shape, n_layers):
    from dataclasses import replace
    return replace(shape, name=f"{shape.name}_{n_layers}l", n_layers=n_layers)


@pytest.mark.parametrize("base,B,P,tiled,bp", [(presets.LLAMA8B, 8, 40, True, False),
                                               (presets.LLAMA70B, 64, 12, True, False),
                                               (presets.LLAMA8B, 8, 40, False, False),
                                               (presets.LLAMA70B, 64, 12, False, False),
                                               (presets.LLAMA8B, 8, 40, False, True),
                                               (presets.LLAMA70B, 64, 12, False, True)],
                         ids=["llama8b_b8_tiled", "llama70b_b64_tiled", "llama8b_b8_row_major",
                              "llama70b_b64_row_major", "llama8b_b8_batched_prefill",
                              "llama70b_b64_batched_prefill"])
def test_real_layer_shapes_reduced_depth(abi, base, B, P, tiled, bp):
    """The batched workloads' layer shapes (8B at batch 8, 70B at batch 64), two
    layers deep, against the oracle's cache-free forward (teacher-forced with
    seeded tokens); the workloads' tiled weights, and row-major ones; and the
    batched prefill (all prompt positions at once) followed by decode steps."""
    shape = layer_subset(base, 2)
    steps = 2
    T = P + steps
    seq = gen.tokens(900 + B, presets.TID_PROMPT, 0, B * T, shape.vocab).reshape(B, T).astype(np.int32)
    print(f"[{shape.name} B={B}] generating weights", flush=True)
    w = gen.gen_weights(shape, 0)
    case = BatchCase(abi, shape, B, T, weights=w, tiled=tiled, batched_prefill=bp)
    got = [case.prefill(seq[:, :P])]
    for s in range(steps):
        got.append(case.step(seq[:, P + s]))
    case.close()
    del case
    print(f"[{shape.name} B={B}] oracle forward", flush=True)
    pos = list(range(P - 1, T))
    ex = D.forward_full(shape, w, seq, positions=pos)
    rd = D.forward_full(shape, w, seq, kv_bf16=True, positions=pos)
    errs = []
    for i, (g, nxt) in enumerate(got):
        check(g, nxt, ex[:, i], rd[:, i], errs, TIGHT_FULL)
    print(f"[{shape.name} B={B}] max rel err vs fp64 {max(e[0] for e in errs):.2e}, "
          f"vs bf16-KV oracle {max(e[1] for e in errs):.2e}", flush=True)
