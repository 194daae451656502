"""MI355X-native fused normalization: norm fused into bf16 GEMM and attention.

The compute lives in libfng.so (hand-written HIP for gfx950, C ABI declared in
include/fng.h).  `binding` is the thin ctypes layer over it; `inputs` draws the
seeded synthetic workloads.  Importing this package loads nothing; the library
is opened on first use and must have been built (`python -m
attention_fng_prenorm_amd.build`).
"""

__all__ = ["binding", "inputs"]
