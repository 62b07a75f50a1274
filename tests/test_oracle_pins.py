"""Pins of the oracle against facts that do not come from the oracle itself.

Closed forms, invariants, brute force, and independent library routines
(torch.nn.functional, transformers' LlamaForCausalLM run in float64 on the
CPU).  A planted-mistake test at the end checks that these pins catch the
plausible slips (dropped gain, eps outside the root, wrong rotation sign,
wrong head grouping, missing residual, wrong activation, transposed operand).
"""
import math

import numpy as np
import pytest
import torch

from oracle import decoder as D
from oracle.naive import NaiveModel
from synth import gen, presets
from tests.shapes import MICRO, MICRO_TIED, MICRO_MHA

RNG = np.random.default_rng(1234)


# ---- I1 RMSNorm --------------------------------------------------------------
def test_rmsnorm_unit_rms_at_eps0():
    x = RNG.normal(size=(5, 257)) * 3.0
    y = D.rmsnorm(x, np.ones(257), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-12)


def test_rmsnorm_rms_with_eps_closed_form():
    x = RNG.normal(size=(4, 64)) * 0.01
    eps = 1e-5
    y = D.rmsnorm(x, np.ones(64), eps)
    ms = np.mean(x * x, -1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), np.sqrt(ms / (ms + eps)), rtol=1e-12)


def test_rmsnorm_scale_invariant_and_gain():
    x = RNG.normal(size=64)
    g = 1.0 + 0.1 * RNG.normal(size=64)
    np.testing.assert_allclose(D.rmsnorm(7.5 * x, g, 0.0), D.rmsnorm(x, g, 0.0), rtol=1e-12)
    np.testing.assert_allclose(D.rmsnorm(x, g, 0.0), D.rmsnorm(x, np.ones(64), 0.0) * g, rtol=1e-12)


def test_rmsnorm_matches_torch():
    x = RNG.normal(size=(3, 96))
    g = 1.0 + 0.1 * RNG.normal(size=96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-5)
    np.testing.assert_allclose(D.rmsnorm(x, g, 1e-5), ref.numpy(), rtol=1e-12)


# ---- I2 RoPE -----------------------------------------------------------------
def test_rope_identity_at_zero_and_closed_form():
    v = RNG.normal(size=(3, 8))
    np.testing.assert_array_equal(D.rope(v, 0, 10000.0), v)
    # hd = 4: pair (0, 2) turns by p rad, pair (1, 3) by p / sqrt(theta)
    e0 = np.array([1.0, 0.0, 0.0, 0.0])
    out = D.rope(e0, 3, 10000.0)
    np.testing.assert_allclose(out, [math.cos(3), 0.0, math.sin(3), 0.0], atol=1e-15)
    e1 = np.array([0.0, 1.0, 0.0, 0.0])
    out = D.rope(e1, 3, 10000.0)
    np.testing.assert_allclose(out, [0.0, math.cos(0.03), 0.0, math.sin(0.03)], atol=1e-15)


def test_rope_norm_preserving_per_pair():
    v = RNG.normal(size=128)
    r = D.rope(v, 4223, 500000.0)
    half = 64
    np.testing.assert_allclose(r[:half] ** 2 + r[half:] ** 2, v[:half] ** 2 + v[half:] ** 2, rtol=1e-12)


def test_rope_relative_position():
    q, k = RNG.normal(size=64), RNG.normal(size=64)
    a = D.rope(q, 17, 10000.0) @ D.rope(k, 5, 10000.0)
    b = D.rope(q, 17 + 100, 10000.0) @ D.rope(k, 5 + 100, 10000.0)
    assert abs(a - b) < 1e-10 * max(1.0, abs(a))


# ---- I3 softmax --------------------------------------------------------------
def test_softmax_rows_and_closed_form():
    s = RNG.normal(size=(7, 33)) * 10
    p = D.softmax(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(D.softmax(s + 1000.0), p, rtol=1e-12)
    np.testing.assert_allclose(D.softmax(np.array([0.0, math.log(3.0)])), [0.25, 0.75], rtol=1e-15)


# ---- I4 / I10 attention --------------------------------------------------------
def test_attention_single_token_returns_v():
    q = RNG.normal(size=(4, 16))
    K = RNG.normal(size=(2, 1, 16))
    V = RNG.normal(size=(2, 1, 16))
    o = D.gqa_attention(q, K, V)
    np.testing.assert_array_equal(o[:2], np.repeat(V[0], 2, 0))
    np.testing.assert_array_equal(o[2:], np.repeat(V[1], 2, 0))


def test_attention_equal_scores_mean_of_v():
    q = np.zeros((2, 8))
    K = RNG.normal(size=(1, 5, 8))
    V = RNG.normal(size=(1, 5, 8))
    o = D.gqa_attention(q, K, V)
    np.testing.assert_allclose(o[0], V[0].mean(0), rtol=1e-14)


@pytest.mark.parametrize("nq,nkv", [(4, 4), (8, 2), (32, 8), (6, 3)])
def test_attention_matches_torch_sdpa(nq, nkv):
    hd, T = 16, 11
    q = RNG.normal(size=(nq, hd))
    K = RNG.normal(size=(nkv, T, hd))
    V = RNG.normal(size=(nkv, T, hd))
    o = D.gqa_attention(q, K, V)
    rep = nq // nkv
    Kt = torch.from_numpy(np.repeat(K, rep, 0))  # textbook MHA with each KV head repeated
    Vt = torch.from_numpy(np.repeat(V, rep, 0))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], Kt, Vt)[:, 0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-14)


# ---- I6 silu -------------------------------------------------------------------
def test_silu_closed_forms_and_torch():
    assert D.silu(np.array([0.0]))[0] == 0.0
    assert abs(D.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15
    assert abs(D.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(D.silu(np.array([-40.0]))[0]) < 1e-15
    u = RNG.normal(size=100) * 5
    np.testing.assert_allclose(D.silu(u), torch.nn.functional.silu(torch.from_numpy(u)).numpy(), rtol=1e-14)


# ---- I7 argmax ------------------------------------------------------------------
def test_greedy_ties_lowest_index_and_nan():
    assert D.greedy(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert list(D.greedy(np.array([[0.0, 0.0], [1.0, 2.0]]))) == [0, 1]
    lg = RNG.normal(size=(3, 1000))
    for row in lg:  # brute force
        best = max(range(1000), key=lambda i: (row[i], -i))
        assert D.greedy(row) == best
    with pytest.raises(FloatingPointError):
        D.greedy(np.array([0.0, np.nan]))


# ---- I8 / I11 cache vs full recompute --------------------------------------------
@pytest.mark.parametrize("shape", [MICRO, MICRO_TIED, presets.TINY], ids=lambda s: s.name)
def test_cached_decode_equals_full_recompute(shape):
    w = gen.gen_weights(shape, seed=0, random_norms=True)
    toks = gen.tokens(77, 3, 0, 2 * 12, shape.vocab).reshape(2, 12)
    dec = D.Decoder(shape, w, batch=2, max_seq=12)
    chain = np.stack([dec.step(toks[:, t]) for t in range(12)], 1)
    full = D.forward_full(shape, w, toks)
    scale = np.abs(full).max()
    assert np.abs(chain - full).max() <= 1e-12 * scale


def test_cached_decode_with_bf16_kv_equals_full_recompute_with_bf16_kv():
    shape = MICRO
    w = gen.gen_weights(shape, seed=4, random_norms=True)
    toks = gen.tokens(7, 3, 0, 9, shape.vocab).reshape(1, 9)
    dec = D.Decoder(shape, w, batch=1, max_seq=9, kv_bf16=True)
    chain = np.stack([dec.step(toks[:, t]) for t in range(9)], 1)
    full = D.forward_full(shape, w, toks, kv_bf16=True)
    assert np.abs(chain - full).max() <= 1e-12 * np.abs(full).max()
    assert np.abs(full - D.forward_full(shape, w, toks)).max() > 0  # the rounding is visible


def test_forward_full_positions_select_rows():
    shape = MICRO
    w = gen.gen_weights(shape, seed=6, random_norms=True)
    toks = gen.tokens(8, 3, 0, 2 * 7, shape.vocab).reshape(2, 7)
    full = D.forward_full(shape, w, toks)
    some = D.forward_full(shape, w, toks, positions=[2, 6])
    assert some.shape == (2, 2, shape.vocab)
    assert np.abs(some - full[:, [2, 6]]).max() <= 1e-12 * np.abs(full).max()


# ---- I9 naive pure-Python model ---------------------------------------------------
@pytest.mark.parametrize("shape", [MICRO, MICRO_TIED], ids=lambda s: s.name)
def test_naive_model_matches(shape):
    w = gen.gen_weights(shape, seed=3, random_norms=True)
    seq = [int(t) for t in gen.tokens(5, 3, 0, 6, shape.vocab)]
    naive = NaiveModel(shape, w)
    dec = D.Decoder(shape, w, batch=1, max_seq=6)
    for t in range(6):
        lg = dec.step([seq[t]])[0]
        ref = np.array(naive.logits(seq[:t + 1]))
        assert np.abs(lg - ref).max() <= 1e-10 * np.abs(ref).max()


def test_naive_model_matches_tiny_workload_prefix():
    shape = presets.TINY
    w = gen.gen_weights(shape, seed=0)
    prompt = gen.gen_prompt(presets.WORKLOADS["tiny"])[0]
    naive = NaiveModel(shape, w)
    dec = D.Decoder(shape, w, batch=1, max_seq=8)
    lg = dec.prefill(prompt[None, :3])[0]
    ref = np.array(naive.logits([int(t) for t in prompt[:3]]))
    assert np.abs(lg - ref).max() <= 1e-10 * np.abs(ref).max()


# ---- transformers' Llama as an independent library implementation ------------------
def hf_logits(shape, w, toks):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.hidden, intermediate_size=shape.ffn,
                      num_hidden_layers=shape.n_layers, num_attention_heads=shape.n_q_heads,
                      num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                      rms_norm_eps=shape.rms_eps, rope_theta=shape.rope_theta,
                      tie_word_embeddings=shape.tie_embeddings, max_position_embeddings=4096,
                      attention_bias=False, mlp_bias=False, attn_implementation="eager")
    torch.manual_seed(0)
    m = LlamaForCausalLM(cfg).double().eval()
    f = lambda n: torch.from_numpy(D.widen_bf16(w[n]))
    sd = {"model.embed_tokens.weight": f("embed"), "model.norm.weight": f("final_norm")[0]}
    sd["lm_head.weight"] = f("embed") if shape.tie_embeddings else f("lm_head")
    names = {"wq": "self_attn.q_proj", "wk": "self_attn.k_proj", "wv": "self_attn.v_proj",
             "wo": "self_attn.o_proj", "w_gate": "mlp.gate_proj", "w_up": "mlp.up_proj",
             "w_down": "mlp.down_proj"}
    for l in range(shape.n_layers):
        for ours, theirs in names.items():
            sd[f"model.layers.{l}.{theirs}.weight"] = f(f"layers.{l}.{ours}")
        sd[f"model.layers.{l}.input_layernorm.weight"] = f(f"layers.{l}.attn_norm")[0]
        sd[f"model.layers.{l}.post_attention_layernorm.weight"] = f(f"layers.{l}.ffn_norm")[0]
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in k for k in missing), (missing, unexpected)
    with torch.no_grad():
        return m(torch.from_numpy(np.asarray(toks, dtype=np.int64))).logits.numpy()


def oracle_chain(shape, w, toks):
    dec = D.Decoder(shape, w, batch=toks.shape[0], max_seq=toks.shape[1])
    return np.stack([dec.step(toks[:, t]) for t in range(toks.shape[1])], 1)


# transformers computes RoPE angles in fp32, so agreement is to ~1e-6 relative.
HF_RTOL = 2e-6


@pytest.mark.parametrize("shape", [MICRO, MICRO_TIED, MICRO_MHA, presets.TINY], ids=lambda s: s.name)
def test_oracle_matches_transformers_llama(shape):
    w = gen.gen_weights(shape, seed=11, random_norms=True)
    toks = gen.tokens(12, 3, 0, 2 * 10, shape.vocab).reshape(2, 10)
    ours = oracle_chain(shape, w, toks)
    ref = hf_logits(shape, w, toks)
    assert np.abs(ours - ref).max() <= HF_RTOL * np.abs(ref).max()


# ---- planted mistakes: each must be caught by the pins above ------------------------
def _eps_outside(x, g, eps):
    return x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + eps) * g


def _rope_sign(v, pos, theta):
    hd = v.shape[-1]
    half = hd // 2
    a = D.rope_angles(pos, hd, theta)
    c, s = np.cos(a), np.sin(a)
    lo, hi = v[..., :half], v[..., half:]
    return np.concatenate([lo * c + hi * s, hi * c - lo * s], -1)


def _gqa_modulo(q, K, V):
    nq, hd = q.shape
    o = np.empty_like(q)
    for h in range(nq):
        g = h % K.shape[0]
        o[h] = D.softmax(K[g] @ q[h] / np.sqrt(hd)) @ V[g]
    return o


PLANTS = {
    "dropped_gain": ("rmsnorm", lambda x, g, eps: x / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)),
    "eps_outside_sqrt": ("rmsnorm", _eps_outside),
    "rope_sign": ("rope", _rope_sign),
    "gqa_modulo": ("gqa_attention", _gqa_modulo),
    "relu_not_silu": ("silu", lambda u: np.maximum(u, 0.0)),
    "ffn_swapped_gate_up": ("swiglu", lambda r, g, u: D.silu(r @ u.T) * (r @ g.T)),
    "no_softmax_scale": ("gqa_attention",
                         lambda q, K, V: np.stack([D.softmax(K[(h * K.shape[0]) // q.shape[0]] @ q[h]) @
                                                   V[(h * K.shape[0]) // q.shape[0]] for h in range(q.shape[0])])),
}


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_planted_mistake_is_caught(plant, monkeypatch):
    fn_name, bad = PLANTS[plant]
    monkeypatch.setattr(D, fn_name, bad)
    shape = MICRO
    w = gen.gen_weights(shape, seed=11, random_norms=True)
    toks = gen.tokens(12, 3, 0, 2 * 10, shape.vocab).reshape(2, 10)
    ours = oracle_chain(shape, w, toks)
    monkeypatch.undo()
    ref = hf_logits(shape, w, toks)
    assert np.abs(ours - ref).max() > 100 * HF_RTOL * np.abs(ref).max()


def test_planted_transposed_wo_is_caught(monkeypatch):
    shape = MICRO  # wo is square here, so a transposed read still runs
    orig = D.Decoder.W

    def bad(self, name):
        m = orig(self, name)
        return m.T if name.endswith(".wo") else m

    monkeypatch.setattr(D.Decoder, "W", bad)
    w = gen.gen_weights(shape, seed=11, random_norms=True)
    toks = gen.tokens(12, 3, 0, 2 * 10, shape.vocab).reshape(2, 10)
    ours = oracle_chain(shape, w, toks)
    monkeypatch.undo()
    ref = hf_logits(shape, w, toks)
    assert np.abs(ours - ref).max() > 100 * HF_RTOL * np.abs(ref).max()


# ---- bf16 rounding, top-2 margin and greedy generation ------------------------------
def _torch_bf16(x):
    """torch's own fp32 -> bfloat16 conversion (round to nearest, ties to even), widened."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_cast():
    x = np.concatenate([RNG.normal(size=50_000) * 10.0 ** RNG.integers(-30, 30, size=50_000),
                        -RNG.random(20_000), RNG.random(20_000) * 3e38, [0.0, -0.0, 1.0, -1.0]])
    np.testing.assert_array_equal(D.round_bf16(x), _torch_bf16(x))


def test_round_bf16_ties_to_even_exact_halfway():
    # fp32 values exactly halfway between two neighbouring bf16 values: the
    # result is the neighbour with an even last mantissa bit
    cases = {0x3F808000: 0x3F80, 0x3F818000: 0x3F82, 0xBF808000: 0xBF80, 0xBF818000: 0xBF82,
             0x7F7F8000: 0x7F80, 0x00018000: 0x0002, 0x3F80C000: 0x3F81, 0x3F804000: 0x3F80}
    bits = np.array(list(cases), dtype=np.uint32)
    want = (np.array(list(cases.values()), dtype=np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(D.round_bf16(bits.view(np.float32)), want)
    np.testing.assert_array_equal(_torch_bf16(bits.view(np.float32)), want)


def test_round_bf16_rejects_truncation():
    # a value just above a halfway point must round up (truncation would not)
    x = np.array([np.float32(1.0) + np.float32(2.0 ** -8) + np.float32(2.0 ** -20)], dtype=np.float32)
    assert D.round_bf16(x)[0] == 1.0 + 2.0 ** -7


def _brute_top2(row):
    """top1 - top2 by two passes over the row (the second excludes the first index)."""
    i1 = max(range(len(row)), key=lambda i: row[i])
    v2 = max(row[i] for i in range(len(row)) if i != i1)
    return row[i1] - v2


def test_top2_margin_brute_force():
    lg = RNG.normal(size=(6, 300))
    lg[2, 10] = lg[2, 200] = lg[2].max() + 1.0       # tie at the top: margin 0
    m = D.top2_margin(lg)
    for r in range(lg.shape[0]):
        assert m[r] == _brute_top2(lg[r])
    assert m[2] == 0.0
    assert D.top2_margin(np.array([3.0, 1.0, 2.0])) == 1.0   # not top1 - top3


def test_generate_matches_greedy_recompute_without_cache():
    """Brute force: each decode step is a cache-free forward of the whole
    sequence so far, fed with the argmax of the previous step's logits."""
    shape = MICRO
    w = gen.gen_weights(shape, seed=21, random_norms=True)
    prompt = gen.tokens(31, 3, 0, 5, shape.vocab).reshape(1, 5)
    steps = 4
    dec = D.Decoder(shape, w, batch=1, max_seq=5 + steps)
    toks, logs = dec.generate(prompt, steps)
    seq = [int(t) for t in prompt[0]]
    nxt = max(range(shape.vocab), key=lambda i: (D.forward_full(shape, w, [seq])[0, -1][i], -i))
    for s in range(steps):
        seq.append(nxt)
        lg = D.forward_full(shape, w, [seq])[0, -1]
        assert np.abs(logs[0, s] - lg).max() <= 1e-12 * np.abs(lg).max()
        nxt = max(range(shape.vocab), key=lambda i: (lg[i], -i))
        assert toks[0, s] == nxt


# planted slips in the three functions above; each pin must reject its slip
def _trunc_bf16(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return ((u >> np.uint32(16)) << np.uint32(16)).view(np.float32).astype(np.float64)


def _ties_away_bf16(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return (((u + np.uint32(0x8000)) >> np.uint32(16)) << np.uint32(16)).view(np.float32).astype(np.float64)


def _top1_minus_top3(lg):
    s = np.sort(lg, axis=-1)
    return s[..., -1] - s[..., -3]


def _generate_stale_feed(self, prompt, steps):
    """Slip: each step is fed the token that was fed to the step before."""
    last = self.prefill(prompt)
    nxt = D.greedy(last)
    prev = nxt
    toks, logs = [], []
    for _ in range(steps):
        lg = self.step(prev)
        logs.append(lg)
        prev, nxt = nxt, D.greedy(lg)
        toks.append(nxt)
    return np.stack(toks, 1), np.stack(logs, 1)


@pytest.mark.parametrize("plant,test", [
    (("round_bf16", _trunc_bf16), test_round_bf16_matches_torch_cast),
    (("round_bf16", _trunc_bf16), test_round_bf16_rejects_truncation),
    (("round_bf16", _ties_away_bf16), test_round_bf16_ties_to_even_exact_halfway),
    (("top2_margin", _top1_minus_top3), test_top2_margin_brute_force),
], ids=["trunc_vs_torch", "trunc_halfway", "ties_away", "top1_minus_top3"])
def test_planted_slip_in_helpers_is_caught(plant, test, monkeypatch):
    monkeypatch.setattr(D, plant[0], plant[1])
    with pytest.raises(AssertionError):
        test()


def test_planted_stale_feed_in_generate_is_caught(monkeypatch):
    monkeypatch.setattr(D.Decoder, "generate", _generate_stale_feed)
    with pytest.raises(AssertionError):
        test_generate_matches_greedy_recompute_without_cache()
