"""MXFP8 latent cache: element code, block scale and cache-row format.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU baseline, never by the library path.

The pages keep the latent cache at four bits per value and gather it with
16-byte vector loads at byte offsets of half the element index ("撕开 DeepSeek
MLA 源码", sheratonhq.com, section 5, the misaligned-address case of the NVFP4
gather); they give neither the element code nor the scale layout, and the
capacity paragraph of bjbfmj.com/news/60700 leaves quantisation scale factors
out of its formula explicitly.  The reading taken here is the MI355X-native
analogue, one of the formats CDNA4 converts in hardware:

* Element code: OCP 8-bit floating point E4M3 ("FN": no infinities) -- sign,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
  subnormals m/8 * 2^-6; codes 0x7F and 0xFF are NaN; the largest finite
  magnitude is 1.75 * 2^8 = 448.  (OCP 8-bit Floating Point Specification
  (OFP8), rev. 1.0, the E4M3 table.)
* Block scale: the OCP Microscaling (MX) v1.0 MXFP8 layout -- blocks of 32
  consecutive latent values share one E8M0 scale byte s, value 2^(s - 127).
  A value is code_value * 2^(s - 127).  The scale of a block is the smallest
  power of two 2^X for which every |v| / 2^X <= 448 (so no element saturates;
  the MX specification's own suggestion, X = floor(log2 amax) - 8, clips
  values in (448, 512) * 2^X by up to 1/8); an all-zero block takes s = 0.
  X is clamped to [-127, 127].  Elements are v / 2^X rounded to the nearest
  E4M3 value, ties to the even code.
* Cache row (656 bytes, every part 16-byte aligned for 16-byte loads): the 512
  latent codes, then the 16 scale bytes of its 16 blocks, then k_R as 64 bf16
  (128 bytes; the RoPE branch is kept at 16 bits, as the pages keep RoPE in
  higher precision -- sheratonhq.com section 4, fp32 RoPE).  A page is 64 such
  rows, 41 984 bytes; paging is unchanged (row t mod 64 of page
  block_table[b][t div 64]).

Dequantisation is exact in bf16 whenever the product is a normal bf16 number
(an E4M3 value has at most 4 significant bits and the scale is a power of
two), so attention over the MXFP8 cache is attention over the dequantised
cache: ``dequantize_pool`` then the fp64 decode of ``mla_oracle``.
"""

from __future__ import annotations

import numpy as np

LATENT = 512
ROPE = 64
MX_BLOCK = 32
SCALE_BIAS = 127
E4M3_MAX = 448.0
SCALES_PER_ROW = LATENT // MX_BLOCK            # 16
CODES_OFF = 0
SCALES_OFF = LATENT                            # 512
ROPE_OFF = SCALES_OFF + SCALES_PER_ROW         # 528
ROW_BYTES = ROPE_OFF + 2 * ROPE                # 656


# --------------------------------------------------------------------------- E4M3


def e4m3_value(codes) -> np.ndarray:
    """Exact value of E4M3 codes (uint8) as float64; 0x7F / 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite values, ascending with the code (0x00 .. 0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_value(_POS_CODES)


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 code of each value (|x| <= 448 expected; larger magnitudes
    saturate to 448), ties to the even code; the sign bit is x's sign bit."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------- MX blocks


def mx_scale_exponent(block_amax) -> np.ndarray:
    """X of each block: the smallest integer with amax <= 448 * 2^X, in [-127, 127]
    (amax = 0 gives -127)."""
    amax = np.asarray(block_amax, dtype=np.float64)
    _, e = np.frexp(amax)                       # amax = f * 2^e, 0.5 <= f < 1
    x0 = e - 9                                  # floor(log2 amax) - 8: amax / 2^x0 in [256, 512)
    x = np.where(amax > E4M3_MAX * np.ldexp(1.0, x0), x0 + 1, x0)
    x = np.where(amax == 0, -SCALE_BIAS, x)
    return np.clip(x, -SCALE_BIAS, SCALE_BIAS).astype(np.int64)


def mx_quantize(values):
    """Quantise [..., 512] latent values: codes uint8 [..., 512] and scale bytes uint8 [..., 16]."""
    v = np.asarray(values, dtype=np.float64)
    blocks = v.reshape(*v.shape[:-1], SCALES_PER_ROW, MX_BLOCK)
    x = mx_scale_exponent(np.abs(blocks).max(axis=-1))
    codes = e4m3_round(np.ldexp(blocks, -x[..., None]))
    return codes.reshape(v.shape), (x + SCALE_BIAS).astype(np.uint8)


def mx_dequantize(codes, scale_bytes) -> np.ndarray:
    """Values of codes [..., 512] with their scale bytes [..., 16] (float64, exact)."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scale_bytes, dtype=np.int64)
    vals = e4m3_value(c).reshape(*c.shape[:-1], SCALES_PER_ROW, MX_BLOCK)
    return np.ldexp(vals, (s - SCALE_BIAS)[..., None]).reshape(c.shape)


# --------------------------------------------------------------------------- cache rows and pools


def pack_rows(latent_values, rope_bits) -> np.ndarray:
    """Cache rows [..., 656] uint8 from latent values [..., 512] and k_R bf16 bits [..., 64]."""
    codes, scales = mx_quantize(latent_values)
    rope = np.ascontiguousarray(np.asarray(rope_bits, dtype=np.uint16))
    out = np.zeros((*codes.shape[:-1], ROW_BYTES), dtype=np.uint8)
    out[..., CODES_OFF:CODES_OFF + LATENT] = codes
    out[..., SCALES_OFF:SCALES_OFF + SCALES_PER_ROW] = scales
    out[..., ROPE_OFF:] = rope.astype("<u2").view(np.uint8).reshape(*rope.shape[:-1], 2 * ROPE)
    return out


def unpack_rows(rows8) -> np.ndarray:
    """Values [..., 576] (float64) of cache rows [..., 656]: dequantised latent, then k_R."""
    r = np.asarray(rows8, dtype=np.uint8)
    lat = mx_dequantize(r[..., CODES_OFF:CODES_OFF + LATENT], r[..., SCALES_OFF:SCALES_OFF + SCALES_PER_ROW])
    rope_bits = np.ascontiguousarray(r[..., ROPE_OFF:]).view("<u2")
    with np.errstate(invalid="ignore"):
        rope = (rope_bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.concatenate([lat, rope], axis=-1)


def quantize_pool(pool_bits) -> np.ndarray:
    """MXFP8 pool [pages, 64, 656] from a bf16 pool [pages, 64, 576] (bit patterns)."""
    p = np.asarray(pool_bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        lat = (p[..., :LATENT].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return pack_rows(lat, p[..., LATENT:])


def dequantize_pool(pool8) -> np.ndarray:
    """float64 pool [pages, 64, 576] holding the values an MXFP8 pool stands for."""
    return unpack_rows(pool8)


def append_to_pool_mxfp8(pool8, rows, block_table, seqlens, s_q: int, max_pos: int) -> np.ndarray:
    """Copy of an MXFP8 pool with new token i of sequence b written to its slot.

    ``rows [B, s_q, 576]`` are the exact new rows (latent, then k_R): the latent
    is quantised to MXFP8 and k_R rounded to bf16 (nearest, ties to even).  A
    token is skipped when its position is outside [0, max_pos) or its slot does
    not exist -- the rules of the bf16 append.
    """
    from .cache_append import append_positions, slot_of
    from .mla_oracle import f64_to_bf16_bits

    out = np.array(pool8, dtype=np.uint8, copy=True)
    rows = np.asarray(rows, dtype=np.float64)
    pos = append_positions(seqlens, s_q)
    for b in range(rows.shape[0]):
        for i in range(s_q):
            p = int(pos[b, i])
            if p < 0 or p >= max_pos:
                continue
            slot = slot_of(block_table, b, p, out.shape[0], out.shape[1])
            if slot is None:
                continue
            out[slot] = pack_rows(rows[b, i, :LATENT], f64_to_bf16_bits(rows[b, i, LATENT:]))
    return out
