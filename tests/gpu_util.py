"""Helpers for the GPU parity tests (device setup, oracle comparison)."""
import numpy as np
import torch

from oracle import decoder as D
from synth import gen, presets


def have_gpu():
    return torch.cuda.is_available()


def rel_err(g, r):
    """max |g - r| / max |r| over the last axis, per row (the logits bar)."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return np.max(np.abs(g - r), axis=-1) / np.max(np.abs(r), axis=-1)


class Case:
    """One model on the GPU plus its oracle, fed the same seeded inputs."""

    def __init__(self, shape, max_seq, mode, seed=0, random_norms=False, attn_split=0, flags=0, num_cus=0,
                 kv_bf16_oracle=False, weights=None, watchdog_ms=0):
        """kv_bf16_oracle: the GPU keeps a bf16 KV cache and the oracle rounds its
        cached K/V to bf16 the same way; otherwise both keep full precision."""
        from decode_persistent_megakernel_02_amd import abi, runtime
        self.abi = abi
        self.shape = shape
        self.w = weights if weights is not None else gen.gen_weights(shape, seed, random_norms)
        self.dw = runtime.upload_weights(self.w)
        self.h = runtime.create(shape, self.dw, max_seq, 1, mode, flags, watchdog_ms, num_cus, attn_split,
                                kv_fp32=not kv_bf16_oracle)
        self.oracle = D.Decoder(shape, self.w, 1, max_seq, kv_bf16=kv_bf16_oracle)
        self.V = shape.vocab
        self.tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.out = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.logits = torch.zeros(1, shape.vocab, dtype=torch.float32, device="cuda")

    def prefill(self, prompt):
        """prompt int array [P]; returns (gpu logits, oracle logits, gpu next)."""
        p = torch.from_numpy(np.asarray(prompt, dtype=np.int32).reshape(1, -1)).cuda()
        self.abi.mk_prefill(self.h, p, self.out, self.logits)
        self.abi.mk_synchronize(self.h)
        ref = self.oracle.prefill(np.asarray(prompt).reshape(1, -1))
        return self.logits.cpu().numpy()[0], ref[0], int(self.out.item())

    def step(self, token, trace=None):
        self.tok.fill_(int(token))
        self.abi.mk_decode_step(self.h, self.tok, self.out, self.logits)
        self.abi.mk_synchronize(self.h)
        ref = self.oracle.step([int(token)], trace)
        return self.logits.cpu().numpy()[0], ref[0], int(self.out.item())


def debug_arrays(abi, h, shape):
    """Host copies of the internal activation buffers (batch 1)."""
    v = abi.mk_get_debug_view(h)
    L, H, F = shape.n_layers, shape.hidden, shape.ffn
    qd = shape.n_q_heads * shape.head_dim
    torch.cuda.synchronize()

    def grab(ptr, n):
        a = np.empty(n, dtype=np.float32)
        d2h(a.ctypes.data, ptr, n * 4)
        return a

    return {
        "xs": grab(v.xs, (L + 1) * H).reshape(L + 1, H),
        "xmid": grab(v.xmid, L * H).reshape(L, H),
        "q": grab(v.q, L * qd).reshape(L, qd),
        "attn": grab(v.attn_out, L * qd).reshape(L, qd),
        "h": grab(v.h, L * F).reshape(L, F),
    }


_hip = None


def d2h(dst, src, nbytes):
    """Device-to-host copy through the HIP runtime (hipMemcpy, synchronous)."""
    import ctypes
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    rc = _hip.hipMemcpy(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, 2)  # hipMemcpyDeviceToHost
    assert rc == 0, rc
