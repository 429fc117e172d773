"""HGA (Hierarchical Global Attention) routed attention for AMD Instinct MI355X.

The compute lives in libhga.so (hand-written HIP kernels for gfx950 behind the
C ABI declared in include/hga.h); this package only binds it (ctypes) and
manages device buffers with PyTorch.
"""
from ._lib import (HGA_BF16, HGA_BWD_KERNELS, HGA_F32, HGA_MAX_CHUNKS, HgaError, HgaShape,  # noqa: F401
                   LIB_PATH, hga_attend_bwd, hga_attend_bwd_timed, hga_attend_bwd_workspace_size, hga_attend_fwd,
                   hga_build_summaries, hga_decode_attend, hga_decode_route, hga_decode_step,
                   hga_decode_workspace_size,
                   hga_route, hga_route_causal, hga_status_string, lib, make_shape)

__all__ = [
    "HGA_BF16", "HGA_F32", "HGA_MAX_CHUNKS", "HgaError", "HgaShape", "LIB_PATH", "lib", "make_shape",
    "hga_build_summaries", "hga_route", "hga_route_causal", "hga_attend_fwd", "hga_attend_bwd_workspace_size",
    "hga_attend_bwd", "hga_attend_bwd_timed", "HGA_BWD_KERNELS", "hga_status_string",
    "hga_decode_step", "hga_decode_route", "hga_decode_attend", "hga_decode_workspace_size",
]
