"""Pins the oracle's cache arithmetic to the numbers the pages print."""

import os
from fractions import Fraction

import pytest

from oracle import capacity

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "capacity_closed_forms.txt")
KIB, MIB, GIB, TIB = 1024, 1024 ** 2, 1024 ** 3, 1024 ** 4


def _golden():
    vals = {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, value, unit, source = [x.strip() for x in line.split("|")]
            assert source, name
            vals[name] = (Fraction(value), unit)
    return vals


G = _golden()


def _computed():
    kv = capacity.kv_cache_bytes
    mha_row = 2 * 128 * 128 * 2          # K and V, 128 heads x 128 dims, 2-byte elements
    return {
        "row_elements": Fraction(512 + 64),
        "row_bytes_bf16": Fraction(kv(1, 512, 64, 2, 1)),
        "mha_row_bytes_bf16": Fraction(mha_row),
        "row_reduction": 1 - Fraction(kv(1, 512, 64, 2, 1), mha_row),
        "mla_64k_b16_60l_bytes": Fraction(kv(60, 512, 64, 2, 65536, 16)),
        "mha_64k_b16_60l_bytes": Fraction(60 * mha_row * 65536 * 16),
        "page64_bytes": Fraction(capacity.page_bytes(64, 512, 64, 2)),
        "page16_bytes": Fraction(capacity.page_bytes(16, 512, 64, 2)),
        "stage_ring_bytes": Fraction(capacity.stage_ring_bytes(64, 512, 64, 2, 3)),
        "per_token_60l_bytes": Fraction(kv(60, 512, 64, 2, 1)),
        "per_token_60l_kib": Fraction(kv(60, 512, 64, 2, 1), KIB),
        "per_token_6l_kib": Fraction(kv(6, 512, 64, 2, 1), KIB),
        "seq_128ki_60l_gib": Fraction(kv(60, 512, 64, 2, 128 * 1024), GIB),
        "element_reduction_576_8192": capacity.element_reduction(576, 8192),
    }


@pytest.mark.parametrize("name", sorted(G))
def test_closed_form_matches_page(name):
    assert _computed()[name] == G[name][0], name


def test_every_golden_value_is_checked():
    assert set(_computed()) == set(G)


def test_printed_roundings_agree():
    # The pages print these rounded; the exact values must round to the printed digits.
    assert round(float(G["row_reduction"][0]) * 100, 2) == 98.24
    assert round(float(G["element_reduction_576_8192"][0]) * 100, 2) == 92.97
    assert G["mla_64k_b16_60l_bytes"][0] == Fraction(135, 2) * GIB == 69120 * MIB
    assert G["mha_64k_b16_60l_bytes"][0] == Fraction(15, 4) * TIB
    assert G["page64_bytes"][0] == 72 * KIB and G["stage_ring_bytes"][0] == 216 * KIB


def test_physical_rounds_up_to_pages():
    # 1 token still holds a whole page; 64 tokens exactly one; 65 two.
    assert capacity.physical_cache_bytes([1], 64, 512, 64, 2) == 73728
    assert capacity.physical_cache_bytes([64], 64, 512, 64, 2) == 73728
    assert capacity.physical_cache_bytes([65, 1], 64, 512, 64, 2) == 3 * 73728
    assert capacity.physical_cache_bytes([65], 64, 512, 64, 2, layers=60) == 60 * 2 * 73728


@pytest.mark.parametrize("args", [
    (0, 512, 64, 2, 1, 1), (60, 0, 64, 2, 1, 1), (60, 512, -1, 2, 1, 1),
    (60, 512, 64, 0, 1, 1), (60, 512, 64, 2, 0, 1), (60, 512, 64, 2, 1, 0), (-60, 512, 64, 2, 1, 1),
])
def test_invalid_dimensions_raise(args):
    with pytest.raises(ValueError):
        capacity.kv_cache_bytes(*args)


def test_no_rope_branch_allowed():
    assert capacity.kv_cache_bytes(1, 512, 0, 2, 1) == 1024
