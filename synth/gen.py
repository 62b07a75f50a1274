"""Seeded synthetic inputs: bf16 weights ~N(mean, std) and uniform token ids.

The definition (splitmix64 stream per tensor, Irwin-Hall sum of four 16-bit
uniforms, one fp32 multiply, bf16 round-to-nearest-even) is written out in
gen.c.  This module holds the slow, obviously-correct numpy version
(`*_np`) and a ctypes front end to the threaded C version in libsynth.so;
tests check that both give identical bits.  Nothing here computes any part of
the decoder.
"""
import ctypes
import math
import os

import numpy as np

from . import presets

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")


def scale_for_std(std: float) -> np.float32:
    """fp32 factor k so that fl32(c * k) has standard deviation `std`."""
    return np.float32(std / math.sqrt((65536.0 ** 2 - 1.0) / 3.0))


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def mix64(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def stream_base(seed: int, tid: int) -> int:
    return mix64(((seed << 32) + tid) & M64)


def hashes_np(seed: int, tid: int, start: int, n: int) -> np.ndarray:
    base = np.uint64(stream_base(seed, tid))
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64_np(base + i * np.uint64(GAMMA))


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    r = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_normal_np(seed, tid, start, n, std=0.02, mean=0.0) -> np.ndarray:
    h = hashes_np(seed, tid, start, n)
    m = np.uint64(0xFFFF)
    s = (h & m) + ((h >> np.uint64(16)) & m) + ((h >> np.uint64(32)) & m) + (h >> np.uint64(48))
    c = s.astype(np.int64) - 131070
    w = c.astype(np.float32) * scale_for_std(std)
    w = (w + np.float32(mean)).astype(np.float32)
    return f32_to_bf16_bits(w)


def tokens_np(seed, tid, start, n, vocab) -> np.ndarray:
    h = hashes_np(seed, tid, start, n)
    with np.errstate(over="ignore"):
        return (((h >> np.uint64(32)) * np.uint64(vocab)) >> np.uint64(32)).astype(np.int32)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            return None
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_fill_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_int]
        lib.synth_fill_bf16.restype = None
        lib.synth_fill_tokens.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        lib.synth_fill_tokens.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_normal(seed, tid, start, n, std=0.02, mean=0.0, out=None) -> np.ndarray:
    """Elements [start, start+n) of tensor (seed, tid) as bf16 bit patterns (uint16)."""
    lib = _load()
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    if lib is None:
        out[:] = bf16_normal_np(seed, tid, start, n, std, mean)
        return out
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    lib.synth_fill_bf16(seed, tid, start, n, float(scale_for_std(std)), float(np.float32(mean)),
                        out.ctypes.data, threads())
    return out


def tokens(seed, tid, start, n, vocab) -> np.ndarray:
    lib = _load()
    if lib is None:
        return tokens_np(seed, tid, start, n, vocab)
    out = np.empty(n, dtype=np.int32)
    lib.synth_fill_tokens(seed, tid, start, n, vocab, out.ctypes.data, threads())
    return out


# --- whole models ---------------------------------------------------------------
NORM_STD_FOR_TESTS = 0.1


def gen_weight(shape: presets.ModelShape, name: str, seed: int = 0, random_norms: bool = False) -> np.ndarray:
    """One weight tensor as uint16 bf16 bits, [rows, cols].

    Matrices are ~N(0, 0.02).  Norm gains are 1 (the workloads' random init
    applies to the matrices), or ~N(1, 0.1) when `random_norms` (unit tests,
    so that a dropped gain multiply is visible).
    """
    rows, cols = presets.weight_shapes(shape)[name]
    tid = presets.tensor_id(name)
    if name.endswith("norm"):
        if not random_norms:
            return np.full((rows, cols), 0x3F80, dtype=np.uint16)  # bf16(1.0)
        return bf16_normal(seed, tid, 0, rows * cols, NORM_STD_FOR_TESTS, 1.0).reshape(rows, cols)
    return bf16_normal(seed, tid, 0, rows * cols, 0.02).reshape(rows, cols)


def gen_weights(shape: presets.ModelShape, seed: int = 0, random_norms: bool = False) -> dict:
    return {n: gen_weight(shape, n, seed, random_norms) for n in presets.weight_shapes(shape)}


def gen_prompt(workload: presets.Workload) -> np.ndarray:
    """[batch, prompt_len] int32 token ids, uniform on [0, vocab)."""
    B, P = workload.batch, workload.prompt_len
    return tokens(workload.prompt_seed, presets.TID_PROMPT, 0, B * P, workload.shape.vocab).reshape(B, P)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (plain bit placement, no arithmetic)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
