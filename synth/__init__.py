"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

Holds the model shapes/workloads (`presets`) and a counter-based generator
(`gen`) for weights and prompt ids.  It contains none of the decoder's
arithmetic; the oracle and the GPU path each take their inputs from here.
"""
from . import presets, gen  # noqa: F401
