"""MI355X-native RBS block-sparse prefill attention.

The compute lives in librbs.so (hand-written HIP for gfx950, C ABI in
include/rbs.h); this package holds the ctypes binding, a host-to-device
upload helper and the seeded synthetic workloads. The shared library is
loaded on first use; a missing library raises, there is no fallback.
"""
from ._lib import (RbsError, block_mask_attn_fwd, block_mask_workspace_bytes,
                   blocksparse_attn_fwd, blocksparse_attn_fwd_fp8, blocksparse_attn_fwd_per_head,
                   blocksparse_attn_fwd_shared_query,
                   lib, rbs_block_stats, rbs_block_stats_per_head, rbs_select,
                   rbs_select_capacity, rbs_select_per_head, rbs_select_static)

__all__ = ["RbsError", "block_mask_attn_fwd", "block_mask_workspace_bytes",
           "blocksparse_attn_fwd", "blocksparse_attn_fwd_fp8", "blocksparse_attn_fwd_per_head",
           "blocksparse_attn_fwd_shared_query",
           "lib", "rbs_block_stats",
           "rbs_block_stats_per_head", "rbs_select", "rbs_select_capacity",
           "rbs_select_per_head", "rbs_select_static"]
