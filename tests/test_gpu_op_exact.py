"""The shipped single-sequence GEMV operator kernels (mk_op_{qkv,o,gu,down,lm}
and their EXACT instances), in the launch configuration a decode step uses,
are bit-exact on exactly representable data: weights k/16 with |k| <= 8 and
small integer inputs make every fp32 partial sum exact (at most 19
significant bits), so any summation order gives the fp64 product bit for bit.
mk_t_op_raw runs each operator kernel with its input staged raw and its dot
products written raw."""
import numpy as np
import pytest
import torch

from synth import presets
from tests.shapes import MINI

pytestmark = pytest.mark.gpu

# the 8B shape's contraction widths (hidden 4096, 32 x 128 query dims, ffn
# 14336: every operator takes its EXACT instance) with one layer and a short
# vocabulary
WIDE = presets.ModelShape("exact_wide", 1, 4096, 32, 8, 128, 14336, 8192, 1e-5, 500000.0, False)
TYPES = {"qkv": 1, "o": 4, "gu": 5, "down": 6, "lm": 7}


def k16_weights(shape, seed):
    rng = np.random.default_rng(seed)
    w, vals = {}, {}
    for name, shp in presets.weight_shapes(shape).items():
        k = rng.integers(-8, 9, size=shp).astype(np.float32) / 16.0
        w[name] = (k.view(np.uint32) >> np.uint32(16)).astype(np.uint16)  # k/16 is exact in bf16
        vals[name] = k.astype(np.float64)
    return w, vals


@pytest.mark.parametrize("shape", [WIDE, MINI], ids=lambda s: s.name)
def test_operator_kernels_bit_exact(shape):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_persistent_megakernel_02_amd import abi, runtime
    w, vals = k16_weights(shape, 5)
    dw = runtime.upload_weights(w)
    h = runtime.create(shape, dw, 8, mode=abi.MK_MODE_PER_OP, kv_fp32=True)
    exact = abi.mk_get_debug_view(h).exact_ops
    print(f"[{shape.name}] EXACT instances bitmask {exact:#x}", flush=True)
    if shape is WIDE:
        assert all((exact >> t) & 1 for t in TYPES.values()), "the wide shape must take every EXACT instance"
    H, F, nq, nkv, hd, V = shape.hidden, shape.ffn, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.vocab
    lm = "embed" if shape.tie_embeddings else "lm_head"
    plan = {
        "qkv": (H, np.concatenate([vals["layers.0.wq"], vals["layers.0.wk"], vals["layers.0.wv"]])),
        "o": (nq * hd, vals["layers.0.wo"]),
        "gu": (H, np.concatenate([vals["layers.0.w_gate"], vals["layers.0.w_up"]])),
        "down": (F, vals["layers.0.w_down"]),
        "lm": (H, vals[lm]),
    }
    rng = np.random.default_rng(11)
    for name, (K, Wm) in plan.items():
        print(f"[{shape.name}] {name}: {Wm.shape[0]} x {K}", flush=True)
        x = rng.integers(-4, 5, size=K).astype(np.float32)
        y = torch.full((Wm.shape[0],), float("nan"), dtype=torch.float32, device="cuda")
        abi.mk_t_op_raw(h, TYPES[name], 0, torch.from_numpy(x).cuda(), y)
        abi.mk_synchronize(h)
        ref = Wm @ x.astype(np.float64)
        got = y.cpu().numpy().astype(np.float64)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, f"{name}: {bad.size} rows differ, first {bad[:5]}: {got[bad[:5]]} vs {ref[bad[:5]]}"
    abi.mk_destroy(h)
