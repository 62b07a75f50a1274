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


# Projection matrices that MK_FLAG_TILED_WEIGHTS stores tiled (the LM head only
# when it is its own matrix; the embedding table stays row-major).
TILED_FIELDS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def is_tiled_name(name: str) -> bool:
    return name == "lm_head" or name.split(".")[-1] in TILED_FIELDS


def tile(t: torch.Tensor) -> torch.Tensor:
    """The tiled layout of a row-major bf16 device matrix (a new tensor)."""
    out = torch.empty_like(t)
    abi.mk_tile_weights(t, out)
    return out


def upload_weights(weights: dict, device="cuda", tiled=False) -> dict:
    """tiled: store the projection matrices in the layout of MK_FLAG_TILED_WEIGHTS."""
    out = {}
    for n, a in weights.items():
        t = to_device_bits(a, device)
        out[n] = tile(t) if tiled and is_tiled_name(n) else t
    return out


def generate_device_weights(shape, seed=0, random_norms=False, device="cuda", progress=None, tiled=False) -> dict:
    """Generate each weight with the seeded host generator and move it to the
    device (tiled as in upload_weights); `progress(done, total)` is called
    after every tensor if given."""
    from synth import gen, presets
    out = {}
    names = list(presets.weight_shapes(shape))
    for i, name in enumerate(names):
        t = to_device_bits(gen.gen_weight(shape, name, seed, random_norms), device)
        out[name] = tile(t) if tiled and is_tiled_name(name) else t
        del t
        if progress:
            progress(i + 1, len(names))
    return out


def create(shape, weights: dict, max_seq: int, max_batch: int = 1, mode=abi.MK_MODE_PER_OP, flags=0,
           watchdog_ms=0, num_cus=0, attn_split=0, kv_fp32=True, stream=None, debug_seed=0) -> abi.Handle:
    """KV cache in fp32 by default (the batched workloads state a bf16 cache and pass kv_fp32=False)."""
    cfg = abi.make_config(shape, max_seq, max_batch, mode, flags, watchdog_ms, num_cus, attn_split, kv_fp32,
                          debug_seed)
    return abi.mk_create(cfg, weights, stream)
