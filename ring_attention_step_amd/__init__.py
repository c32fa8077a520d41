"""Ring attention's per-step blockwise forward (and its backward) for AMD Instinct MI355X (gfx950).

The compute lives in libra.so (hand-written HIP kernels + host runtime, C ABI in
include/ra.h); this package is its thin Python binding.
"""
from ._binding import (LAYOUTS, RA_BF16, RA_BLOCK_ACCUMULATE, RA_BLOCK_FORCE_SIMT, RA_CONTIGUOUS, RA_F32, RA_STRIPED, RAError,
                       load_library, ra_abi_version, ra_block_attn_fwd, ra_lse_merge, ra_mask_offset,
                       ra_release, ra_ring_forward, ra_ring_pair_offset, ra_ring_workspace_size,
                       ra_stripe_permute, ra_unmasked_pairs, ring_desc, block_desc, ra_attn_bwd_delta,
                       ra_block_attn_bwd, ra_ring_bwd_workspace_size, ra_ring_backward, ra_ring_forward_noalloc,
                       ra_ring_noalloc_max_bytes)

__all__ = ["LAYOUTS", "RA_BF16", "RA_BLOCK_ACCUMULATE", "RA_BLOCK_FORCE_SIMT", "RA_CONTIGUOUS", "RA_F32", "RA_STRIPED", "RAError",
           "load_library", "ra_abi_version", "ra_block_attn_fwd", "ra_lse_merge", "ra_mask_offset",
           "ra_release", "ra_ring_forward", "ra_ring_pair_offset", "ra_ring_workspace_size",
           "ra_stripe_permute", "ra_unmasked_pairs", "ring_desc", "block_desc", "ra_attn_bwd_delta",
           "ra_block_attn_bwd", "ra_ring_bwd_workspace_size", "ra_ring_backward", "ra_ring_forward_noalloc",
           "ra_ring_noalloc_max_bytes"]
