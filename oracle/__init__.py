"""The oracle: plain, slow CPU implementations of one decode step.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or run anything here.  It shares no code with the
GPU path (decode_persistent_megakernel_02_amd) and neither imports the other;
both take their inputs from the seeded generators in synth/.
"""
