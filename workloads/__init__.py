"""Seeded synthetic inputs for tree-verify attention.

This package only draws random numbers and lays them out in memory.  It holds
none of the attention arithmetic: the fp64 oracle and the HIP library both
consume what it produces, and neither imports the other.
"""
from .commit import free_list, make_tokens, place_tree_in_cache  # noqa: F401
from .configs import (  # noqa: F401
    CONFIG_NAMES,
    TREE_12,
    TREE_CHAIN4,
    TREE_SINGLE,
    TreeVerifyInputs,
    bf16_bits_from_f32,
    make_config,
    make_inputs,
)
