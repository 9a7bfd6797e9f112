"""CPU oracle for absorbed MLA decode over a paged latent cache.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, fp64 statement of
what the GPU path computes.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library path never does, and
this package imports nothing from the library.  It shares no code, tables or
helpers with the HIP kernels.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
printed values of the pages (``tests/golden/``), textbook special cases,
invariants and brute force.  No function here is "parity unpinned".
"""

from .cache_append import (  # noqa: F401
    append_kv,
    append_positions,
    append_rows,
    append_to_pool,
    down_project,
    rope_angles,
    rope_q,
    rope_rotate,
    rope_table,
    slot_of,
)
from .capacity import (  # noqa: F401
    element_reduction,
    kv_cache_bytes,
    page_bytes,
    physical_cache_bytes,
    stage_ring_bytes,
)
from .prefill import decompress_kv  # noqa: F401
from .mla_oracle import (  # noqa: F401
    absorb_q,
    attention_probs,
    bf16_bits_to_f64,
    combine_fragments,
    decode_absorbed,
    decode_decompressed,
    f64_to_bf16_bits,
    gather_rows,
    split_decode_absorbed,
    up_proj,
)
from .fp8_cache import (  # noqa: F401
    append_to_pool_mxfp8,
    dequantize_pool,
    e4m3_round,
    e4m3_value,
    mx_dequantize,
    mx_quantize,
    mx_scale_exponent,
    pack_rows,
    quantize_pool,
    unpack_rows,
)
from . import fp8_cache  # noqa: F401,E402
