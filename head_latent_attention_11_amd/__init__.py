"""MLA decode over the compressed latent KV cache on AMD MI355X (gfx950).

The compute lives in libmla.so (HIP kernels behind the C ABI of
include/mla.h); this package is its thin Python binding.  Build the library
with ``python -m head_latent_attention_11_amd.build``.
"""
from .binding import (BF16, F32, FP8_E4M3, LIB_PATH, MLADims, MLAError, absorb_q,  # noqa: F401
                      cache_append, decode_attn, decode_workspace_size, load_library,
                      status_string, up_proj_v, version)
