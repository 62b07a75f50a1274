"""Caller-side glue around the C ABI: device weight upload and config building.

Weights arrive as uint16 bf16 bit arrays (synth.gen produces them); they are
copied to device tensors one at a time so that host memory holds at most one
tensor beyond the caller's copy.
"""
import numpy as np
import torch

from . import abi


def to_device_bits(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit array -> device tensor of the same 16-bit patterns (dtype bfloat16)."""
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16)).to(device, non_blocking=False).view(torch.bfloat16)


def upload_weights(weights: dict, device="cuda") -> dict:
    return {n: to_device_bits(a, device) for n, a in weights.items()}


def generate_device_weights(shape, seed=0, random_norms=False, device="cuda", progress=None) -> dict:
    """Generate each weight with the seeded host generator and move it to the
    device; `progress(done, total)` is called after every tensor if given."""
    from synth import gen, presets
    out = {}
    names = list(presets.weight_shapes(shape))
    for i, name in enumerate(names):
        out[name] = to_device_bits(gen.gen_weight(shape, name, seed, random_norms), device)
        if progress:
            progress(i + 1, len(names))
    return out


def create(shape, weights: dict, max_seq: int, max_batch: int = 1, mode=abi.MK_MODE_PER_OP, flags=0,
           watchdog_ms=0, num_cus=0, attn_split=0, kv_fp32=True, stream=None) -> abi.Handle:
    """KV cache in fp32 by default (the batched workloads state a bf16 cache and pass kv_fp32=False)."""
    cfg = abi.make_config(shape, max_seq, max_batch, mode, flags, watchdog_ms, num_cus, attn_split, kv_fp32)
    return abi.mk_create(cfg, weights, stream)
