"""Gated DeltaNet token mixer for AMD MI355X (gfx950).

The compute lives in libgdn.so (hand-written HIP kernels behind a C ABI,
include/gdn.h); this package is its Python binding plus thin helpers that
allocate outputs with torch and chain the four calls.
"""
from ._lib import (GDN_BF16, GDN_F32, GdnError, gdn_chunk_prefill, gdn_conv_chunk_prefill,  # noqa: F401
                   gdn_chunk_prefill_noalloc, gdn_chunk_prefill_workspace_size, gdn_prefill_layer, gdn_conv1d_fwd, gdn_gated_rmsnorm,
                   gdn_recurrent_step, gdn_recurrent_step_norm, gdn_recurrent_step_slots, lib,
                   library_path, version)
from .mixer import DecodeGraph, decode_step, prefill_layer  # noqa: F401
