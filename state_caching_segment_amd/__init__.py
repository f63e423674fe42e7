"""libhypic: segment state caching for linear-attention layers on MI355X.

The compute lives in the HIP library ``libhypic.so`` (C ABI in
``include/hypic.h``); ``hypic`` is its ctypes binding.
"""
from .hypic import (DTYPE, EXPORTS, FAMILY, NOALLOC_WORKSPACE_BYTES, OP_BUILD, OP_COMPOSE_SEQ, OP_COMPOSE_TREE,
                    OP_SEAM, SEQ, TREE, HypicError, Store, hypic_content_key, hypic_compose, hypic_compose_tree_noalloc, hypic_last_error,
                    hypic_compose_compact, hypic_conv_warmup, hypic_layout, hypic_pair_compact, hypic_rerotate, hypic_seam_advance, hypic_segment_build, hypic_segment_prefill,
                    hypic_status_string, hypic_t_elems, hypic_tokens, hypic_workspace_bytes, layout, load, tokens)

__all__ = ["DTYPE", "EXPORTS", "FAMILY", "NOALLOC_WORKSPACE_BYTES", "OP_BUILD", "OP_COMPOSE_SEQ", "OP_COMPOSE_TREE",
           "OP_SEAM", "SEQ", "TREE", "HypicError", "Store", "hypic_content_key", "hypic_compose", "hypic_compose_tree_noalloc", "hypic_last_error",
           "hypic_compose_compact", "hypic_conv_warmup", "hypic_layout", "hypic_pair_compact", "hypic_rerotate", "hypic_seam_advance", "hypic_segment_build", "hypic_segment_prefill",
           "hypic_status_string", "hypic_t_elems", "hypic_tokens", "hypic_workspace_bytes", "layout", "load",
           "tokens"]
