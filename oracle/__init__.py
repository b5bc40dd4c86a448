"""CPU oracle (fp64 NumPy) for block-sparse video attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the bench's CPU-baseline
leg, never by the product path.  Shares no code with the HIP kernels or their binding.
"""
from .bsa_oracle import (widen_bf16, num_blocks, padded_len, tile_perm, tile_perm_by_sort,
                         reorder, inverse_reorder, block_ranges, pool, block_scores,
                         block_mass, route_row, route, RowRoute, Routing, sparse_attn,
                         masked_dense_attn, dense_attn_raster, block_mask_dense, layer)
from .check import check_mask, check_row, compare_out, MaskReport, OutReport
from .stripe import block_coords, stripe_keep, stripe_mask
from .hilbert import cube_bits, hilbert_index, hilbert_order, hilbert_perm
