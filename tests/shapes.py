"""Small model shapes used by the tests (beside the workloads in synth.presets)."""
from synth.presets import ModelShape

MICRO = ModelShape("micro", 2, 64, 4, 2, 16, 96, 128, 1e-5, 10000.0, False)
MICRO_TIED = ModelShape("micro_tied", 2, 64, 4, 2, 16, 96, 128, 1e-5, 10000.0, True)
MICRO_MHA = ModelShape("micro_mha", 1, 64, 4, 4, 16, 96, 128, 1e-5, 10000.0, False)

# Shapes the GPU library accepts (head_dim 64/128), with ragged tails:
# ffn and vocab are not multiples of the 512-column chunk / 4-row task.
MINI = ModelShape("mini", 2, 128, 4, 2, 64, 264, 322, 1e-5, 10000.0, False)
MINI_TIED = ModelShape("mini_tied", 2, 128, 4, 2, 64, 264, 322, 1e-5, 10000.0, True)
MINI_G8 = ModelShape("mini_g8", 1, 256, 8, 1, 128, 520, 258, 1e-5, 500000.0, False)
# head_dim 128 with 1 and 2 query heads per KV head (a bf16 cache at head_dim
# 128 scores on the matrix cores, whatever the group size).
MINI_HD128_G1 = ModelShape("mini_hd128_g1", 2, 256, 2, 2, 128, 520, 258, 1e-5, 500000.0, False)
MINI_HD128_G2 = ModelShape("mini_hd128_g2", 2, 256, 4, 2, 128, 520, 258, 1e-5, 500000.0, False)

# Shapes whose projections fit the tiled weight layout (rows multiples of 16,
# columns multiples of 32), untied, tied and with 8 query heads per KV head.
MINI_TILE = ModelShape("mini_tile", 2, 128, 4, 2, 64, 256, 336, 1e-5, 10000.0, False)
MINI_TILE_TIED = ModelShape("mini_tile_tied", 2, 128, 4, 2, 64, 256, 336, 1e-5, 10000.0, True)
MINI_TILE_G8 = ModelShape("mini_tile_g8", 1, 256, 8, 1, 128, 512, 272, 1e-5, 500000.0, False)
