"""Plain CPU reference for one greedy decode step of a Llama-style decoder.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the GPU path and never receives values computed on the GPU.

What is computed: the fused instruction list of the Hazy Research low-latency
and high-throughput megakernels (hakusoku summary "全てのGPUを購入したので、徹底的にそのGPUを活用します。",
section 高スループットMegakernelの設計と工夫 / 命令セットの再設計: RMS norm,
QKV matmul + RoPE, attention, O-proj matmul + residual) and
the SwiGLU feed-forward ("Cómo la fusión de kernels CUDA acelera la inferencia
de LLM", section "Sigue los datos intermedios"), run for one token at a time
against a key/value cache; then the final norm, the LM head and greedy argmax.
The MPK write-up ("Compilar LLM en un MegaKernel ...", sections Parte 1 and
Parte 2) describes the megakernel as a re-scheduling of exactly this
computation, so the oracle is the plain, unscheduled definition.

The pages name these operators but never define them.  Readings taken where
they are silent (each is the standard Llama definition):
  R-norm   RMSNorm y = x / sqrt(mean(x^2) + eps) * gamma, eps inside the sqrt.
  R-rope   rotate-half RoPE: pairs (i, i + hd/2), angle p * theta^(-2i/hd),
           0-based absolute positions, angles in float64, no frequency scaling.
  R-gqa    query head h reads KV head floor(h * n_kv / n_q) (contiguous groups).
  R-attn   scale 1/sqrt(hd), causal including the current token, softmax with
           max subtraction, no bias, no dropout.
  R-ffn    down(silu(gate(r)) * up(r)), silu(u) = u / (1 + e^-u), no biases.
  R-tied   a tied model uses the embedding table as LM head.
  R-argmax greedy token = lowest index among the maximal logits.
Arithmetic is float64 throughout; bf16 weights are widened exactly.
"""
import numpy as np


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMS norm over the last axis (reading R-norm)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def rope_angles(pos: int, head_dim: int, theta: float) -> np.ndarray:
    """Angles p * theta^(-2i/hd), i < hd/2, in float64 (reading R-rope)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(pos) * theta ** (-2.0 * i / head_dim)


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate each (i, i + hd/2) pair of the last axis by its angle (reading R-rope)."""
    hd = v.shape[-1]
    half = hd // 2
    a = rope_angles(pos, hd, theta)
    c, s = np.cos(a), np.sin(a)
    lo, hi = v[..., :half], v[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def gqa_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Decode attention of one sequence.

    q [nq, hd] (already rotated); K, V [nkv, T, hd] hold every position up to
    and including the current one.  Returns o [nq, hd] (readings R-gqa, R-attn).
    """
    nq, hd = q.shape
    nkv = K.shape[0]
    o = np.empty_like(q)
    for h in range(nq):
        g = (h * nkv) // nq
        s = K[g] @ q[h] / np.sqrt(hd)
        o[h] = softmax(s) @ V[g]
    return o


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def swiglu(r, w_gate, w_up) -> np.ndarray:
    """silu(r W_g^T) * (r W_u^T) (reading R-ffn); weights [out, in]."""
    return silu(r @ w_gate.T) * (r @ w_up.T)


def greedy(logits: np.ndarray) -> np.ndarray:
    """Lowest index of the maximum along the last axis (reading R-argmax)."""
    if not np.all(np.isfinite(logits)):
        raise FloatingPointError("non-finite logits")
    return np.argmax(logits, axis=-1).astype(np.int32)


class Decoder:
    """fp64 Llama-style decoder with a per-sequence key/value cache.

    `weights` maps the tensor names of synth.presets.weight_shapes to uint16
    bf16 bit arrays.  With `cache_weights=False` every matrix is widened when
    used (large shapes); otherwise once.  `kv_bf16=True` rounds cached K/V to
    bf16 like a bf16 cache would, to separate storage error from kernel error.
    """

    def __init__(self, shape, weights: dict, batch: int, max_seq: int,
                 cache_weights: bool = True, kv_bf16: bool = False):
        self.shape = shape
        self.w = weights
        self.B = batch
        self.max_seq = max_seq
        self.kv_bf16 = kv_bf16
        self._cache = {} if cache_weights else None
        L, nkv, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.K = np.zeros((L, batch, nkv, max_seq, hd))
        self.V = np.zeros((L, batch, nkv, max_seq, hd))
        self.length = 0

    def W(self, name: str) -> np.ndarray:
        if self._cache is None:
            return widen_bf16(self.w[name])
        if name not in self._cache:
            self._cache[name] = widen_bf16(self.w[name])
        return self._cache[name]

    def _lm_head(self) -> str:
        return "embed" if self.shape.tie_embeddings else "lm_head"

    def _store_kv(self, x: np.ndarray) -> np.ndarray:
        return round_bf16(x) if self.kv_bf16 else x

    def step(self, tokens, trace: dict = None) -> np.ndarray:
        """One decode step at position `length` for every sequence; returns logits [B, V].

        If `trace` is a dict, the per-layer intermediates are stored in it:
        ("q", l) rotated queries [B, nq*hd], ("attn", l) attention output,
        ("xmid", l) residual after attention, ("h", l) SwiGLU output, ("x", l+1)
        residual after layer l.
        """
        tokens = np.asarray(tokens, dtype=np.int64).reshape(self.B)
        p = self.length
        if p >= self.max_seq:
            raise IndexError("KV cache full")
        x = widen_bf16(self.w["embed"][tokens])                      # [B, H]
        for l in range(self.shape.n_layers):
            x = self.layer(l, x, p, trace)
        logits = self.head(x)
        self.length = p + 1
        return logits

    def layer(self, l: int, x: np.ndarray, p: int, trace: dict = None) -> np.ndarray:
        """Decoder layer l on the residual stream x [B, H] of the token at
        position p: appends its K/V at p to the cache and returns the residual
        stream after the layer (the body of `step`; see there for `trace`)."""
        sh = self.shape
        nq, nkv, hd = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
        pre = f"layers.{l}."
        r = rmsnorm(x, self.W(pre + "attn_norm")[0], sh.rms_eps)
        q = (r @ self.W(pre + "wq").T).reshape(self.B, nq, hd)
        k = (r @ self.W(pre + "wk").T).reshape(self.B, nkv, hd)
        v = (r @ self.W(pre + "wv").T).reshape(self.B, nkv, hd)
        q = rope(q, p, sh.rope_theta)
        k = rope(k, p, sh.rope_theta)
        self.K[l, :, :, p] = self._store_kv(k)
        self.V[l, :, :, p] = self._store_kv(v)
        o = np.stack([gqa_attention(q[b], self.K[l, b, :, :p + 1], self.V[l, b, :, :p + 1])
                      for b in range(self.B)])
        x = x + o.reshape(self.B, nq * hd) @ self.W(pre + "wo").T
        r = rmsnorm(x, self.W(pre + "ffn_norm")[0], sh.rms_eps)
        hh = swiglu(r, self.W(pre + "w_gate"), self.W(pre + "w_up"))
        if trace is not None:
            trace[("q", l)] = q.reshape(self.B, nq * hd)
            trace[("attn", l)] = o.reshape(self.B, nq * hd)
            trace[("xmid", l)] = x
            trace[("h", l)] = hh
        x = x + hh @ self.W(pre + "w_down").T
        if trace is not None:
            trace[("x", l + 1)] = x
        return x

    def head(self, x: np.ndarray) -> np.ndarray:
        """Final RMSNorm and LM head on the last residual stream x [B, H]: logits [B, V]."""
        r = rmsnorm(x, self.W("final_norm")[0], self.shape.rms_eps)
        return r @ self.W(self._lm_head()).T

    def prefill(self, tokens) -> np.ndarray:
        """Token-by-token decode chain over a prompt [B, P]; returns the last logits [B, V]."""
        tokens = np.asarray(tokens).reshape(self.B, -1)
        logits = None
        for t in range(tokens.shape[1]):
            logits = self.step(tokens[:, t])
        return logits

    def generate(self, prompt, steps: int):
        """Greedy generation: prefill, then `steps` decode steps fed with their own argmax.

        Returns (tokens [B, steps], logits [B, steps, V]) of the decode steps;
        the first decode step's input is the argmax of the prefill's last logits.
        """
        last = self.prefill(prompt)
        nxt = greedy(last)
        toks, logs = [], []
        for _ in range(steps):
            lg = self.step(nxt)
            logs.append(lg)
            nxt = greedy(lg)
            toks.append(nxt)
        return np.stack(toks, 1), np.stack(logs, 1)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), via fp32; returns float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    r = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (((u + r) >> np.uint32(16)) << np.uint32(16)).view(np.float32).astype(np.float64)


def forward_full(shape, weights: dict, tokens, kv_bf16: bool = False, positions=None) -> np.ndarray:
    """Causal forward of whole sequences without a cache: logits [B, T, V]
    (or [B, len(positions), V] for the listed positions only).

    Each position t attends to positions 0..t; used to check the cached decode
    chain and as a fast batched prefill for large shapes.  `kv_bf16` rounds the
    keys (after RoPE) and values to bf16, as a bf16 KV cache stores them.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    B, T = tokens.shape
    nq, nkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    W = lambda n: widen_bf16(weights[n])
    x = widen_bf16(weights["embed"][tokens])                         # [B, T, H]
    for l in range(shape.n_layers):
        pre = f"layers.{l}."
        r = rmsnorm(x, W(pre + "attn_norm")[0], shape.rms_eps)
        q = (r @ W(pre + "wq").T).reshape(B, T, nq, hd)
        k = (r @ W(pre + "wk").T).reshape(B, T, nkv, hd)
        v = (r @ W(pre + "wv").T).reshape(B, T, nkv, hd)
        for t in range(T):
            q[:, t] = rope(q[:, t], t, shape.rope_theta)
            k[:, t] = rope(k[:, t], t, shape.rope_theta)
        if kv_bf16:
            k, v = round_bf16(k), round_bf16(v)
        o = np.empty((B, T, nq, hd))
        for b in range(B):
            for t in range(T):
                o[b, t] = gqa_attention(q[b, t], k[b, :t + 1].transpose(1, 0, 2), v[b, :t + 1].transpose(1, 0, 2))
        x = x + o.reshape(B, T, nq * hd) @ W(pre + "wo").T
        r = rmsnorm(x, W(pre + "ffn_norm")[0], shape.rms_eps)
        x = x + swiglu(r, W(pre + "w_gate"), W(pre + "w_up")) @ W(pre + "w_down").T
    if positions is not None:
        x = x[:, list(positions)]
    r = rmsnorm(x, W("final_norm")[0], shape.rms_eps)
    return r @ W("embed" if shape.tie_embeddings else "lm_head").T


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """top1 - top2 of each row (last axis)."""
    s = np.sort(logits, axis=-1)
    return s[..., -1] - s[..., -2]
