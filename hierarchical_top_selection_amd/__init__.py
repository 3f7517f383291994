"""MI355X (gfx950) PISA hot path: key pyramid, hierarchical LSE block selection,
block-sparse attention and the decode step, behind the C ABI of include/pisa.h.

The functions below are the thin torch binding of that ABI (see ``binding``);
``workloads`` holds the seeded synthetic inputs.
"""
from .binding import (build_pyramid, decode_step, pyramid_nodes, select_blocks, select_flat, sparse_attn_bwd,
                      sparse_attn_fwd)

__all__ = ["build_pyramid", "select_blocks", "select_flat", "sparse_attn_fwd", "sparse_attn_bwd", "decode_step", "pyramid_nodes"]
