"""Closed-form latent-cache arithmetic (oracle, test infrastructure only).

Follows the capacity paragraph of bjbfmj.com/news/60700: cache bytes equal
layers x (d_c + d_R) x bytes per element x tokens x concurrent sequences, with
no page tables, alignment or quantisation scales counted.  The page's own
calculator lost its operators in extraction; the reading used here rejects any
non-positive layers, d_c, element size, token or sequence count and any
negative d_R (d_R = 0 is a cache without the RoPE branch).

The page and pipeline-stage sizes follow "撕开 DeepSeek MLA 源码" (sheratonhq.com),
section 3 (page_size 64 vs 16) and section 5 (three stages of a 64-token tile
of latent plus RoPE rows).  All results are exact Python integers / Fractions.
"""

from __future__ import annotations

from fractions import Fraction


def kv_cache_bytes(layers: int, d_c: int, d_r: int, elem_bytes: int, tokens: int, sequences: int = 1) -> int:
    """Unsharded logical cache bytes: L x (d_c + d_R) x b x tokens x sequences."""
    for v in (layers, d_c, elem_bytes, tokens, sequences):
        if not isinstance(v, int) or v <= 0:
            raise ValueError("invalid dimension")
    if not isinstance(d_r, int) or d_r < 0:
        raise ValueError("invalid dimension")
    return layers * (d_c + d_r) * elem_bytes * tokens * sequences


def page_bytes(page_tokens: int, d_c: int, d_r: int, elem_bytes: int) -> int:
    """Bytes of one cache page: page_tokens rows of (d_c + d_R) elements."""
    return kv_cache_bytes(1, d_c, d_r, elem_bytes, page_tokens, 1)


def physical_cache_bytes(seqlens, page_tokens: int, d_c: int, d_r: int, elem_bytes: int, layers: int = 1) -> int:
    """Page-rounded allocation: every sequence holds ceil(L / page) whole pages."""
    pages = sum(-(-int(L) // page_tokens) for L in seqlens)
    return layers * pages * page_bytes(page_tokens, d_c, d_r, elem_bytes)


def stage_ring_bytes(tile_tokens: int, d_c: int, d_r: int, elem_bytes: int, stages: int) -> int:
    """On-chip bytes of a ring of ``stages`` tiles, each holding latent and RoPE rows."""
    return (tile_tokens * d_c + tile_tokens * d_r) * elem_bytes * stages


def element_reduction(stored: int, baseline: int) -> Fraction:
    """Fraction of elements saved: 1 - stored / baseline."""
    return 1 - Fraction(stored, baseline)
