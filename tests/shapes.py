"""Small model shapes used by the tests (beside the workloads in synth.presets)."""
from synth.presets import ModelShape

MICRO = ModelShape("micro", 2, 64, 4, 2, 16, 96, 128, 1e-5, 10000.0, False)
MICRO_TIED = ModelShape("micro_tied", 2, 64, 4, 2, 16, 96, 128, 1e-5, 10000.0, True)
MICRO_MHA = ModelShape("micro_mha", 1, 64, 4, 4, 16, 96, 128, 1e-5, 10000.0, False)
