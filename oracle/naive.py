"""Pure-Python (no numpy, no BLAS) decoder for tiny shapes.

TEST INFRASTRUCTURE ONLY (same rule as oracle/decoder.py).  Written with
plain loops over Python floats (IEEE double), independently of decoder.py, so
that the two can be checked against each other: this is the naive recompute
of a tiny model.  It recomputes every position's keys and values from scratch
at each step (no cache), following the same readings R-norm ... R-argmax.
"""
import math
import struct


def bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _mat(weights, name):
    a = weights[name]
    return [[bf16_to_float(v) for v in row] for row in a.tolist()]


def _matvec(W, x):
    out = []
    for row in W:
        acc = 0.0
        for w, v in zip(row, x):
            acc += w * v
        out.append(acc)
    return out


def _norm(x, g, eps):
    ms = 0.0
    for v in x:
        ms += v * v
    ms /= len(x)
    inv = 1.0 / math.sqrt(ms + eps)
    return [v * inv * gg for v, gg in zip(x, g)]


def _rot(vec, pos, theta):
    hd = len(vec)
    half = hd // 2
    out = [0.0] * hd
    for i in range(half):
        ang = pos * theta ** (-2.0 * i / hd)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i + half] * c + vec[i] * s
    return out


class NaiveModel:
    def __init__(self, shape, weights):
        self.s = shape
        self.m = {n: _mat(weights, n) for n in weights}

    def _layer_kv(self, l, xs):
        """Keys/values of layer l for inputs xs (list over positions)."""
        s = self.s
        pre = f"layers.{l}."
        ks, vs, qs = [], [], []
        for p, x in enumerate(xs):
            r = _norm(x, self.m[pre + "attn_norm"][0], s.rms_eps)
            q = _matvec(self.m[pre + "wq"], r)
            k = _matvec(self.m[pre + "wk"], r)
            v = _matvec(self.m[pre + "wv"], r)
            hd = s.head_dim
            qs.append([_rot(q[h * hd:(h + 1) * hd], p, s.rope_theta) for h in range(s.n_q_heads)])
            ks.append([_rot(k[g * hd:(g + 1) * hd], p, s.rope_theta) for g in range(s.n_kv_heads)])
            vs.append([v[g * hd:(g + 1) * hd] for g in range(s.n_kv_heads)])
        return qs, ks, vs

    def logits(self, seq):
        """Logits at the last position of a token list, recomputed from scratch."""
        s = self.s
        hd = s.head_dim
        xs = [list(self.m["embed"][int(t)]) for t in seq]
        for l in range(s.n_layers):
            pre = f"layers.{l}."
            qs, ks, vs = self._layer_kv(l, xs)
            new = []
            for p, x in enumerate(xs):
                o = []
                for h in range(s.n_q_heads):
                    g = (h * s.n_kv_heads) // s.n_q_heads
                    sc = []
                    for j in range(p + 1):
                        d = 0.0
                        for a, b in zip(qs[p][h], ks[j][g]):
                            d += a * b
                        sc.append(d / math.sqrt(hd))
                    mx = max(sc)
                    e = [math.exp(v - mx) for v in sc]
                    z = sum(e)
                    oh = [0.0] * hd
                    for j in range(p + 1):
                        w = e[j] / z
                        for i in range(hd):
                            oh[i] += w * vs[j][g][i]
                    o.extend(oh)
                y = _matvec(self.m[pre + "wo"], o)
                x2 = [a + b for a, b in zip(x, y)]
                r = _norm(x2, self.m[pre + "ffn_norm"][0], s.rms_eps)
                gt = _matvec(self.m[pre + "w_gate"], r)
                up = _matvec(self.m[pre + "w_up"], r)
                hh = [(a / (1.0 + math.exp(-a))) * b for a, b in zip(gt, up)]
                d = _matvec(self.m[pre + "w_down"], hh)
                new.append([a + b for a, b in zip(x2, d)])
            xs = new
        r = _norm(xs[-1], self.m["final_norm"][0], s.rms_eps)
        head = self.m["embed"] if s.tie_embeddings else self.m["lm_head"]
        return _matvec(head, r)
