"""MI355X persistent decode megakernel: Python side of libmk.so.

`abi` mirrors the C entry points one to one; `runtime` adds the small amount
of glue a caller needs (uploading bf16 weights to device tensors, building an
mk_config from a model shape).  Every step of the decode path runs in the HIP
kernels of libmk.so; nothing here computes any part of it.
"""
