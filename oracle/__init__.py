"""CPU oracle of the hybrid tile-sparse (dense / 2:4) linear layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check of the
package entry file and by the benchmark's CPU-baseline leg -- never by the
library or its Python binding.  Plain numpy, float64 products, no code shared
with the GPU path.
"""
from .hybrid import (TILE_DENSE, TILE_SPARSE24, VALID_NIBBLES, widen_f32, widen_f64, check_grid,
                     as_tiles, from_tiles, selection_scores, keep_two_of_four, kept_positions,
                     sparse_tile_keep, masked_weights, plan, pack, unpack, gemm_ref, hybrid_ref,
                     within_tolerance, column_norms, wanda_tile_cost, wanda_tile_map, density,
                     mask_scores, malformed_groups, pack_masked, masked_weights_from_mask, wanda_global_maps,
                     silu_mul_ref, gated_ref, storage_type, e4m3_value)

__all__ = ["TILE_DENSE", "TILE_SPARSE24", "VALID_NIBBLES", "widen_f32", "widen_f64", "check_grid",
           "as_tiles", "from_tiles", "selection_scores", "keep_two_of_four", "kept_positions",
           "sparse_tile_keep", "masked_weights", "plan", "pack", "unpack", "gemm_ref", "hybrid_ref",
           "within_tolerance", "column_norms", "wanda_tile_cost", "wanda_tile_map", "density",
           "mask_scores", "malformed_groups", "pack_masked", "masked_weights_from_mask", "wanda_global_maps",
           "silu_mul_ref", "gated_ref", "storage_type", "e4m3_value"]
