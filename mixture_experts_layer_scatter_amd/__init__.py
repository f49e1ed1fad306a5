"""MI355X-native forward pass of one Mixture-of-Experts layer (HIP, gfx950).

The compute lives in libmoe.so (C ABI in include/moe.h); this package holds its
thin torch binding.  Submodules load the library on first use and raise when it
has not been built.
"""
from ._lib import LIB_PATH, MoeError, EXPORTS  # noqa: F401
from .api import (Dims, ExpertCache, capacity, combine, expert_ffn, expert_ffn_fp8,  # noqa: F401
                  expert_ffn_mxfp4, gate, layer_forward, layer_forward_cached, layer_forward_fp8,
                  layer_forward_mxfp4, load_stats, load_stats_buffer, permute, quantize_fp8,
                  quantize_mxfp4, read_load_stats, route, workspace, workspace_bytes,
                  layer_forward_static, static_scratch_bytes, quantize_mxfp8, expert_ffn_w4a8,
                  layer_forward_w4a8, layer_forward_cached_w4a8)
