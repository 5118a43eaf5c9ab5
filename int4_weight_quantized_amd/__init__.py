"""int4-weight quantized linear layers for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library libw4.so (C ABI declared in
include/w4.h); `int4_weight_quantized_amd.ops` is the thin ctypes binding
over it. Nothing here falls back to a CPU or PyTorch implementation: if the
library is missing, calls raise.
"""
__all__ = ["ops", "workloads"]
