"""The persistent megakernel (one launch per decode step) against the oracle
and against the kernel-per-operator build of the same task bodies.

Bars (as in test_gpu_decode):
  * logits: max|gpu - oracle| / max|oracle| <= 2e-2 per step against the fp64
    oracle; <= 1e-3 against the oracle with the GPU's KV-cache rounding;
  * tokens: equal wherever the oracle's top-2 margin exceeds 5e-2;
  * megakernel vs per-operator build: the same arithmetic up to the order of
    fp32 sums in RMSNorm, attention and the split merge, so their logits agree
    to 1e-5 relative.
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
WATCHDOG_MS = 500  # in-kernel wait limit for these small cases


@pytest.fixture(scope="module")
def abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi as a
    return a


def check_step(g, r, nxt, errs, bar):
    e = float(rel_err(g, r))
    errs.append(e)
    assert e <= bar, f"logit error {e:.3e} > {bar}"
    if D.top2_margin(r) > MARGIN:
        assert nxt == int(D.greedy(r)), "greedy token differs at a clear margin"


def teacher_forced(case, prompt, steps, bar):
    errs = []
    g, r, nxt = case.prefill(prompt)
    check_step(g, r, nxt, errs, bar)
    tok = int(D.greedy(r))
    for _ in range(steps):
        g, r, nxt = case.step(tok)
        check_step(g, r, nxt, errs, bar)
        tok = int(D.greedy(r))
    return errs


def test_tiny_workload_teacher_forced(abi):
    wl = presets.WORKLOADS["tiny"]
    case = Case(wl.shape, wl.max_seq, MEGA, watchdog_ms=WATCHDOG_MS)
    errs = teacher_forced(case, gen.gen_prompt(wl)[0], wl.decode_steps, CONTRACT)
    print(f"tiny megakernel: max rel err {max(errs):.2e}")
    assert max(errs) <= TIGHT


def test_tiny_tight_against_bf16_kv_oracle(abi):
    wl = presets.WORKLOADS["tiny"]
    case = Case(wl.shape, wl.max_seq, MEGA, kv_bf16_oracle=True, watchdog_ms=WATCHDOG_MS)
    teacher_forced(case, gen.gen_prompt(wl)[0], wl.decode_steps, TIGHT)


@pytest.mark.parametrize("shape", [MINI, MINI_TIED, MINI_G8, MINI_HD128_G1, MINI_HD128_G2], ids=lambda s: s.name)
@pytest.mark.parametrize("kv_bf16", [False, True], ids=["kv_f32", "kv_bf16"])
def test_ragged_shapes_multi_split(abi, shape, kv_bf16):
    # 16-position attention splits, prompt 21 + 14 steps: positions span 3 splits
    case = Case(shape, 40, MEGA, seed=5, random_norms=True, attn_split=16, kv_bf16_oracle=kv_bf16,
                watchdog_ms=WATCHDOG_MS)
    prompt = gen.tokens(9, 3, 0, 21, shape.vocab)
    teacher_forced(case, prompt, 14, TIGHT)


@pytest.mark.parametrize("shape", [MINI_G8, MINI], ids=lambda s: s.name)
def test_megakernel_agrees_with_per_op(abi, shape):
    """Same weights, same tokens: the two builds differ only in the order of
    fp32 sums (norm, attention, merge)."""
    prompt = gen.tokens(4, 3, 0, 9, shape.vocab)
    w = gen.gen_weights(shape, 2, True)
    outs = []
    for mode in (MEGA, PER_OP):
        case = Case(shape, 24, mode, attn_split=8, weights=w, watchdog_ms=WATCHDOG_MS)
        outs.append(np.stack([case.prefill(prompt)[0]] + [case.step(t)[0] for t in (3, 77, 200, 5, 9, 11)]))
    err = np.abs(outs[0] - outs[1]).max() / np.abs(outs[1]).max()
    assert err <= 1e-5, err


@pytest.mark.parametrize("shape,kv_bf16", [(MINI, False), (MINI_G8, True), (MINI_HD128_G2, False)],
                         ids=["mini", "g8_bf16kv", "hd128_g2"])
def test_shuffled_task_dealing_changes_nothing(abi, shape, kv_bf16):
    """MK_FLAG_SHUFFLE rotates every GEMV operator's task list by a seeded
    amount per operator and step, so other workgroups run the tasks in
    another order.  Every task's result depends only on its rows and the
    staged input, so the logits and ids must be bit-identical to the unshuffled
    handle's, over a one-launch prefill, single steps and a multi-step launch,
    for two seeds."""
    from decode_persistent_megakernel_02_amd import runtime
    w = gen.gen_weights(shape, 6, True)
    prompt = gen.tokens(21, 3, 0, 11, shape.vocab)
    p_t = torch.from_numpy(prompt.reshape(1, -1)).cuda()
    dw = runtime.upload_weights(w)
    runs = []
    for flags, seed in ((0, 0), (abi.MK_FLAG_SHUFFLE, 1), (abi.MK_FLAG_SHUFFLE, 0xC0FFEE)):
        h = runtime.create(shape, dw, 40, mode=MEGA, flags=flags, watchdog_ms=WATCHDOG_MS, attn_split=8,
                           kv_fp32=not kv_bf16, debug_seed=seed)
        toks = torch.zeros(12, dtype=torch.int32, device="cuda")
        lg = torch.zeros(5, shape.vocab, dtype=torch.float32, device="cuda")
        abi.mk_prefill(h, p_t, toks[0:1], lg[0:1])
        for s in range(3):
            abi.mk_decode_step(h, toks[s:s + 1], toks[s + 1:s + 2], lg[s + 1:s + 2])
        abi.mk_generate(h, toks[3:4], 8, toks[4:12], lg[4:5])
        abi.mk_synchronize(h)
        runs.append((toks.cpu().numpy(), lg.cpu().numpy()))
        abi.mk_destroy(h)
    for r in runs[1:]:
        assert np.array_equal(r[0], runs[0][0])
        assert np.array_equal(r[1].view(np.uint32), runs[0][1].view(np.uint32))
    ref = D.Decoder(shape, w, 1, 40, kv_bf16=kv_bf16).prefill(prompt.reshape(1, -1))[0]
    assert rel_err(runs[0][1][0], ref) <= TIGHT


def test_free_running_matches_until_low_margin(abi):
    from decode_persistent_megakernel_02_amd import runtime
    wl = presets.WORKLOADS["tiny"]
    shape = wl.shape
    w = gen.gen_weights(shape, 0)
    dw = runtime.upload_weights(w)
    h = runtime.create(shape, dw, wl.max_seq, mode=MEGA, watchdog_ms=WATCHDOG_MS)
    prompt = gen.gen_prompt(wl)
    toks = torch.zeros(wl.decode_steps + 1, dtype=torch.int32, device="cuda")
    abi.mk_prefill(h, torch.from_numpy(prompt).cuda(), toks[0:1])
    for s in range(wl.decode_steps):  # device-side feedback, no host sync
        abi.mk_decode_step(h, toks[s:s + 1], toks[s + 1:s + 2])
    abi.mk_synchronize(h)
    gpu = toks.cpu().numpy()
    ref_tokens, ref_logits = D.Decoder(shape, w, 1, wl.max_seq).generate(prompt, wl.decode_steps)
    last = D.Decoder(shape, w, 1, wl.max_seq).prefill(prompt)[0]
    margins = [D.top2_margin(last)] + [D.top2_margin(ref_logits[0, s]) for s in range(wl.decode_steps)]
    ref_seq = [int(D.greedy(last))] + list(ref_tokens[0])
    for s in range(wl.decode_steps + 1):
        if margins[s] <= MARGIN:
            break
        assert gpu[s] == ref_seq[s], f"step {s}"


def test_llama1b_shape_two_layers(abi):
    """The exact (no clamped loads) instance at head_dim 64."""
    shape = presets.with_layers(presets.LLAMA1B, 2)
    case = Case(shape, 48, MEGA, watchdog_ms=2000)
    teacher_forced(case, gen.tokens(1001, 3, 0, 39, shape.vocab), 4, TIGHT)


def test_reset_and_capacity(abi):
    shape = MINI
    case = Case(shape, 5, MEGA, watchdog_ms=WATCHDOG_MS)
    prompt = gen.tokens(1, 3, 0, 4, shape.vocab)
    a = case.prefill(prompt)[0]
    case.step(5)
    with pytest.raises(abi.MkError) as e:
        abi.mk_decode_step(case.h, case.tok, case.out, case.logits)
    assert e.value.status == abi.MK_ERR_CAPACITY
    abi.mk_reset(case.h)
    p = torch.from_numpy(prompt.reshape(1, -1)).cuda()
    abi.mk_prefill(case.h, p, case.out, case.logits)
    abi.mk_synchronize(case.h)
    assert np.array_equal(case.logits.cpu().numpy()[0], a)


def test_batched_config_is_refused(abi):
    from decode_persistent_megakernel_02_amd import runtime
    shape = MINI
    dw = runtime.upload_weights(gen.gen_weights(shape, 0))
    with pytest.raises(abi.MkError) as e:
        runtime.create(shape, dw, 16, max_batch=2, mode=MEGA, kv_fp32=False)
    assert e.value.status == abi.MK_ERR_UNSUPPORTED


def test_watchdog_ends_a_step_with_timeout(abi):
    """MK_FLAG_SPIN_LIMIT_1 makes every in-kernel wait give up after one
    unsuccessful check (the host forces the condition; every wave still
    exits): the step returns MK_ERR_TIMEOUT and poisons the handle, and a new
    handle works."""
    shape = MINI
    w = gen.gen_weights(shape, 7)
    case = Case(shape, 16, MEGA, weights=w, flags=abi.MK_FLAG_SPIN_LIMIT_1)
    p = torch.from_numpy(gen.tokens(2, 3, 0, 3, shape.vocab).reshape(1, -1)).cuda()
    abi.mk_prefill(case.h, p, case.out, case.logits)
    with pytest.raises(abi.MkError) as e:
        abi.mk_synchronize(case.h)
    assert e.value.status == abi.MK_ERR_TIMEOUT
    with pytest.raises(abi.MkError) as e:
        abi.mk_decode_step(case.h, case.tok, case.out, case.logits)
    assert e.value.status == abi.MK_ERR_STATE
    ok = Case(shape, 16, MEGA, weights=w, watchdog_ms=WATCHDOG_MS)
    g, r, _ = ok.prefill(gen.tokens(2, 3, 0, 3, shape.vocab))
    assert rel_err(g, r) <= TIGHT


def test_intermediates_match_oracle_per_layer(abi):
    """The megakernel's hand-over buffers after one step, layer by layer,
    against the oracle's values: rotated q, k and v of the step's position,
    the attention output, the residual after attention, the SwiGLU output and
    the residual after each layer.  Every word read carries the step's epoch.
    fp32 arithmetic with an fp32 cache against fp64: 1e-4 relative."""
    from tests.gpu_util import d2h
    shape = MINI
    case = Case(shape, 24, MEGA, seed=8, random_norms=True, attn_split=4, watchdog_ms=WATCHDOG_MS)
    case.prefill(gen.tokens(1, 3, 0, 6, shape.vocab))
    p = case.oracle.length
    trace = {}
    case.step(17, trace)
    v = abi.mk_get_mega_view(case.h)
    L, H, F = shape.n_layers, shape.hidden, shape.ffn
    nq, nkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim

    def grab(ptr, n, skip=0):
        a = np.empty(n, dtype=np.uint64)
        d2h(a.ctypes.data, ptr, n * 8)
        assert np.all((a[skip:] >> np.uint64(32)) == v.epoch), "a word without the step's epoch"
        return (a & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).astype(np.float64)

    x = grab(v.x, (L + 1) * H, skip=H).reshape(L + 1, H)  # row 0: the embedding row is never handed over
    xmid = grab(v.xmid, L * H).reshape(L, H)
    qkv = grab(v.qkv, L * (nq + 2 * nkv) * hd).reshape(L, -1)
    attn = grab(v.attn, L * nq * hd).reshape(L, nq * hd)
    hh = grab(v.h, L * F).reshape(L, F)

    def close(got, ref, what):
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err < 1e-4, (what, err)

    for l in range(L):
        close(qkv[l, :nq * hd], trace[("q", l)][0], f"q{l}")
        close(qkv[l, nq * hd:(nq + nkv) * hd], case.oracle.K[l, 0, :, p].reshape(-1), f"k{l}")
        close(qkv[l, (nq + nkv) * hd:], case.oracle.V[l, 0, :, p].reshape(-1), f"v{l}")
        close(attn[l], trace[("attn", l)][0], f"attn{l}")
        close(xmid[l], trace[("xmid", l)][0], f"xmid{l}")
        close(hh[l], trace[("h", l)][0], f"h{l}")
        close(x[l + 1], trace[("x", l + 1)][0], f"x{l + 1}")


def test_generate_in_one_launch(abi):
    """mk_generate: 24 greedy steps in ONE megakernel launch, each step's
    argmax feeding the next step's embedding inside the kernel.  The same
    steps launched one at a time (ids fed back on the device) give the same
    ids and the same last logits bit for bit (the same arithmetic per step);
    the ids follow the oracle's greedy generation wherever its top-2 margin
    exceeds 5e-2; a request past the cache capacity is refused."""
    from decode_persistent_megakernel_02_amd import runtime
    shape, n = MINI_G8, 24
    w = gen.gen_weights(shape, 3, True)
    prompt = gen.tokens(43, 3, 0, 7, shape.vocab)  # the oracle's first 19 margins exceed 5e-2
    p_t = torch.from_numpy(prompt.reshape(1, -1)).cuda()
    dw = runtime.upload_weights(w)
    runs = []
    for one_launch in (True, False):
        h = runtime.create(shape, dw, 40, mode=MEGA, watchdog_ms=WATCHDOG_MS)
        toks = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
        lg = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")
        abi.mk_prefill(h, p_t, toks[0:1])
        if one_launch:
            abi.mk_generate(h, toks[0:1], n, toks[1:], lg)
        else:
            for s in range(n):
                abi.mk_decode_step(h, toks[s:s + 1], toks[s + 1:s + 2], lg if s == n - 1 else None)
        abi.mk_synchronize(h)
        runs.append((toks.cpu().numpy(), lg.cpu().numpy()[0]))
        if one_launch:
            with pytest.raises(abi.MkError) as e:  # 7 + 24 positions used of 40
                abi.mk_generate(h, toks[0:1], 10, toks[1:11])
            assert e.value.status == abi.MK_ERR_CAPACITY
    assert np.array_equal(runs[0][0], runs[1][0])
    assert np.array_equal(runs[0][1], runs[1][1])
    gpu = runs[0][0]
    ref_tokens, ref_logits = D.Decoder(shape, w, 1, 40).generate(prompt.reshape(1, -1), n)
    last = D.Decoder(shape, w, 1, 40).prefill(prompt.reshape(1, -1))[0]
    margins = [D.top2_margin(last)] + [D.top2_margin(ref_logits[0, s]) for s in range(n)]
    ref_seq = [int(D.greedy(last))] + list(ref_tokens[0])
    checked = 0
    for s in range(n + 1):
        if margins[s] <= MARGIN:
            break
        assert gpu[s] == ref_seq[s], f"step {s}"
        checked += 1
    print(f"one-launch generation: {checked} leading ids checked against the oracle")
    assert checked >= 8


def test_generate_per_operator_matches_oracle(abi):
    from decode_persistent_megakernel_02_amd import runtime
    wl = presets.WORKLOADS["tiny"]
    shape = wl.shape
    w = gen.gen_weights(shape, 0)
    dw = runtime.upload_weights(w)
    h = runtime.create(shape, dw, wl.max_seq, mode=PER_OP)
    prompt = gen.gen_prompt(wl)
    toks = torch.zeros(wl.decode_steps + 1, dtype=torch.int32, device="cuda")
    abi.mk_prefill(h, torch.from_numpy(prompt).cuda(), toks[0:1])
    abi.mk_generate(h, toks[0:1], wl.decode_steps, toks[1:])
    abi.mk_synchronize(h)
    gpu = toks.cpu().numpy()
    ref_tokens, ref_logits = D.Decoder(shape, w, 1, wl.max_seq).generate(prompt, wl.decode_steps)
    last = D.Decoder(shape, w, 1, wl.max_seq).prefill(prompt)[0]
    margins = [D.top2_margin(last)] + [D.top2_margin(ref_logits[0, s]) for s in range(wl.decode_steps)]
    ref_seq = [int(D.greedy(last))] + list(ref_tokens[0])
    for s in range(wl.decode_steps + 1):
        if margins[s] <= MARGIN:
            break
        assert gpu[s] == ref_seq[s], f"step {s}"
