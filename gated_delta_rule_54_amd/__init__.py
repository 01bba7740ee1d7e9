"""MI355X-native Kimi Delta Attention (KDA) operator.

The operator runs in hand-written HIP kernels for gfx950 behind the C ABI
of include/kda.h (libkda.so, built in-tree by
``python -m gated_delta_rule_54_amd.build``).  This package is the thin
Python binding over that ABI; torch provides device memory and streams.
"""
from .kda import (KdaDesc, KdaError, chunk_bwd_workspace_bytes,  # noqa: F401
                  chunk_fwd_workspace_bytes, kda_chunk_bwd, kda_chunk_fwd, kda_chunk_fwd_conv,
                  kda_decode_step, kda_output_gate_norm, kda_short_conv_swish, load_library,
                  make_desc)

__all__ = ["kda_chunk_fwd", "kda_chunk_fwd_conv", "kda_chunk_bwd", "kda_decode_step",
           "kda_output_gate_norm", "kda_short_conv_swish", "chunk_fwd_workspace_bytes",
           "chunk_bwd_workspace_bytes", "load_library", "make_desc", "KdaDesc", "KdaError"]
