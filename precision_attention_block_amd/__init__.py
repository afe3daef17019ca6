"""Block-scaled FP8 / MXFP4 FlashAttention forward with optional 3D
sliding-tile sparsity for AMD Instinct MI355X (gfx950).

The compute path is libpab.so (HIP kernels behind the C ABI in include/pab.h);
`binding` marshals torch tensors into it.  See `api.attention` for the
one-call entry point."""
from . import binding
from .api import attention, quantize_qkv

__all__ = ["binding", "attention", "quantize_qkv"]
