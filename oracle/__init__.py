"""CPU fp64 oracle (test infrastructure only; see mla_oracle's module docstring)."""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import (DK, DV, DROPE, bf16_bits_to_f64, e4m3fn_bits_to_f64, ancestor_masks,
                         causal_masks, visible_positions, verify_attention, sparse_rows,
                         sparse_decode_attention, split_bounds, combine_partials,
                         split_emulated_verify, brute_force_verify, brute_force_sparse)
