"""Seeded synthetic inputs for paged MLA decode.

This package only draws random numbers and lays them out: sequence lengths,
a physical page permutation, the block table, and bf16 bit patterns for the
queries, the two up-projection weights, the latent cache pool, and the
hidden states and down-projection weight of newly appended tokens. It holds
none of the attention arithmetic, so both the CPU oracle (through the tests)
and the HIP path (through the tests and the benchmark) can take their inputs
from it without sharing any computation.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    D_C,
    D_HC,
    D_MODEL,
    D_R,
    NUM_HEADS,
    PAGE,
    MlaInputs,
    f32_to_bf16_bits,
    make_inputs,
    make_custom,
    make_append_inputs,
    pages_per_seq,
    poison_unused,
)
