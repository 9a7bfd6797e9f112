"""Pins of the MXFP8 cache oracle (oracle/fp8_cache.py) against things other than
itself: torch's float8_e4m3fn codec (a library routine), the fixed points of the
OCP E4M3 table, brute force over every code, closed forms of the scale choice and
of the row size, and the exactness and error bounds the format guarantees."""

import math

import numpy as np
import pytest

import oracle
from oracle import fp8_cache as F
from synth import make_custom

torch = pytest.importorskip("torch")


def torch_e4m3_values(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.double().numpy()


def torch_e4m3_round(x):
    """torch's codec on fp32 inputs (it takes a float64 tensor through fp32 first, a second
    rounding, so the comparison is made on values that fp32 holds exactly)."""
    x32 = np.asarray(x, dtype=np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64))
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ------------------------------------------------------------------------------------- element code


def test_e4m3_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(F.e4m3_value(codes), torch_e4m3_values(codes), equal_nan=True)


def test_e4m3_fixed_points():
    # OCP OFP8 rev. 1.0, E4M3: largest normal S.1111.110 = 448, smallest normal 2^-6,
    # largest subnormal 0.875 * 2^-6, smallest subnormal 2^-9, S.1111.111 = NaN.
    v = F.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6 and v(0x07) == 0.875 * 2.0 ** -6 and v(0x01) == 2.0 ** -9
    assert v(0x38) == 1.0 and v(0x40) == 2.0 and v(0xB8) == -1.0 and v(0x39) == 1.125
    assert v(0x00) == 0.0 and np.signbit(v(0x80)) and v(0x80) == 0.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    finite = F.e4m3_value(np.arange(256))
    assert np.count_nonzero(np.isfinite(finite)) == 254
    pos = F.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)                     # codes 0x00..0x7E ascend


def test_e4m3_round_matches_torch_including_ties():
    rng = np.random.default_rng(3)
    pos = F.e4m3_value(np.arange(0x7F))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)  # exact ties between neighbours
    x = np.concatenate([rng.uniform(-448, 448, 20000).astype(np.float32),
                        rng.normal(0, 1e-2, 5000).astype(np.float32), mids, -mids, pos.astype(np.float32),
                        -pos.astype(np.float32), np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1000))]).astype(np.float64)
    assert np.array_equal(F.e4m3_round(x), torch_e4m3_round(x))


def test_e4m3_round_saturates_and_keeps_sign():
    assert list(F.e4m3_round([449.0, 1e6, -500.0, -1e30])) == [0x7E, 0x7E, 0xFE, 0xFE]
    assert F.e4m3_round([-1e-30])[0] == 0x80 and F.e4m3_round([1e-30])[0] == 0x00


# ------------------------------------------------------------------------------------- block scale


def brute_scale_exponent(amax):
    if amax == 0:
        return -127
    for x in range(-127, 128):
        if amax <= 448.0 * 2.0 ** x:
            return x
    return 127


def test_scale_exponent_closed_forms():
    cases = [448.0 * 2.0 ** k for k in range(-20, 21)] + \
            [448.0 * 2.0 ** k * (1 + 2.0 ** -40) for k in range(-20, 21)] + \
            [2.0 ** m for m in range(-30, 31)] + [0.0, 2.0 ** -140, 2.0 ** 200, 3.0, 500.0, 447.9]
    got = F.mx_scale_exponent(np.array(cases))
    for a, g in zip(cases, got):
        assert g == brute_scale_exponent(a), a
    # closed forms: 448 * 2^k -> k; just above -> k + 1; 2^m -> m - 8 (2^m / 448 = 2^(m-8) / 1.75)
    assert list(F.mx_scale_exponent(np.array([448.0 * 2.0 ** 5, 448.0 * 2.0 ** 5 * (1 + 2.0 ** -40), 2.0 ** 3]))) \
        == [5, 6, -5]


def brute_quantize_block(v):
    """Every finite code tried at the block's scale; nearest value, ties to the even code."""
    x = brute_scale_exponent(float(np.max(np.abs(v))))
    codes = np.arange(256)
    vals = np.array([F.e4m3_value(c) * 2.0 ** x for c in codes])
    out = []
    for e in v:
        best = None
        for c, cv in zip(codes, vals):
            if not np.isfinite(cv) or (cv == 0 and c == 0x80):
                continue
            d = abs(cv - e)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        c = best[1]
        if c == 0 and np.signbit(e):
            c = 0x80
        out.append(c)
    return np.array(out, dtype=np.uint8), x + 127


def test_quantize_brute_force():
    rng = np.random.default_rng(5)
    blocks = [rng.normal(0, 1, 32), rng.normal(0, 1e-3, 32) * np.exp(rng.uniform(-8, 8, 32)),
              np.r_[rng.normal(0, 1, 31), 448.0], np.r_[rng.normal(0, 1, 31), -3e4],
              np.zeros(32), np.r_[np.zeros(31), 1e-3], rng.uniform(-1, 1, 32) * 2.0 ** -100]
    row = np.concatenate(blocks + [rng.normal(0, 5, 32)] * (16 - len(blocks)))
    codes, scales = F.mx_quantize(row)
    for j in range(16):
        bc, bs = brute_quantize_block(row[32 * j:32 * j + 32])
        assert scales[j] == bs, j
        assert np.array_equal(codes[32 * j:32 * j + 32], bc), j


def test_roundtrip_error_bound_and_no_saturation():
    rng = np.random.default_rng(6)
    v = rng.normal(0, 1, (200, 512)) * np.exp(rng.uniform(-5, 5, (200, 1)))
    codes, scales = F.mx_quantize(v)
    d = F.mx_dequantize(codes, scales)
    step = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32, axis=-1)
    scaled = np.abs(v) / step
    assert scaled.max() <= 448.0
    normal = scaled >= 2.0 ** -6
    # nearest rounding: half a unit in the last of 3 mantissa bits, relative 2^-4; subnormals 2^-10 * 2^X
    assert np.all(np.abs(d - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal])
    assert np.all(np.abs(d - v)[~normal] <= 2.0 ** -10 * step[~normal])


def test_grid_values_are_reproduced():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 0x7F, (20, 512)).astype(np.uint8) | (rng.integers(0, 2, (20, 512)) << 7).astype(np.uint8)
    codes[:, ::32] = 0x7E                                 # every block reaches 448 * 2^X
    scales = rng.integers(120, 135, (20, 16)).astype(np.uint8)
    vals = F.mx_dequantize(codes, scales)
    c2, s2 = F.mx_quantize(vals)
    assert np.array_equal(s2, scales)
    assert np.array_equal(F.mx_dequantize(c2, s2), vals)  # -0 may come back as +0 codes, same value


# ------------------------------------------------------------------------------------- rows and pools


def test_row_layout_and_size():
    assert (F.CODES_OFF, F.SCALES_OFF, F.ROPE_OFF, F.ROW_BYTES) == (0, 512, 528, 656)
    assert all(o % 16 == 0 for o in (F.SCALES_OFF, F.ROPE_OFF, F.ROW_BYTES))
    # bytes per token per layer: 512 one-byte codes + 512/32 scale bytes + 64 two-byte k_R
    assert F.ROW_BYTES == 512 * 1 + 512 // 32 + 64 * 2
    assert 64 * F.ROW_BYTES == 41984
    # the pages' bf16 row is 1152 B (60 layers: 69120 B); the MXFP8 row is 41/72 of it
    assert oracle.kv_cache_bytes(1, 512, 64, 2, 1) == 1152
    assert F.ROW_BYTES * 72 == 1152 * 41
    rng = np.random.default_rng(8)
    lat = rng.normal(0, 1, 512)
    rope = rng.integers(0, 0x7F00, 64).astype(np.uint16)
    r = F.pack_rows(lat, rope)
    codes, scales = F.mx_quantize(lat)
    assert np.array_equal(r[:512], codes) and np.array_equal(r[512:528], scales)
    assert np.array_equal(r[528:656:2], (rope & 0xFF).astype(np.uint8))       # little-endian bf16
    assert np.array_equal(r[529:656:2], (rope >> 8).astype(np.uint8))
    back = F.unpack_rows(r)
    assert np.array_equal(back[512:], oracle.bf16_bits_to_f64(rope))


def test_dequantized_values_are_exact_bf16():
    inp = make_custom(11, 2, 1, [300, 70])
    deq = F.dequantize_pool(F.quantize_pool(inp.pool))
    assert np.array_equal(oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(deq)), deq)


def test_decode_over_a_lossless_pool_equals_bf16_decode():
    # a bf16 pool whose latent already lies on the MXFP8 grid quantises without loss
    inp = make_custom(12, 3, 2, [200, 64, 129])
    deq = F.dequantize_pool(F.quantize_pool(inp.pool))
    grid_bits = oracle.f64_to_bf16_bits(deq)
    pool8 = F.quantize_pool(grid_bits)
    assert np.array_equal(F.dequantize_pool(pool8), deq)
    qa = oracle.absorb_q(inp.q_c, inp.w_uk)
    o1, l1 = oracle.decode_absorbed(qa, inp.q_r, grid_bits, inp.block_table, inp.seqlens, 2, inp.scale)
    o2, l2 = oracle.decode_absorbed(qa, inp.q_r, F.dequantize_pool(pool8), inp.block_table, inp.seqlens, 2,
                                    inp.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_quantized_decode_stays_near_bf16_decode():
    # the cache error moves each score by at most scale * sum|q_abs| * |c - deq(c)|
    inp = make_custom(13, 2, 1, [500, 90])
    qa = oracle.absorb_q(inp.q_c, inp.w_uk)
    pool8 = F.quantize_pool(inp.pool)
    deq = F.dequantize_pool(pool8)
    o1, l1 = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, 1, inp.scale)
    o2, l2 = oracle.decode_absorbed(qa, inp.q_r, deq, inp.block_table, inp.seqlens, 1, inp.scale)
    full = oracle.bf16_bits_to_f64(inp.pool)
    dc = np.abs(full[..., :512] - deq[..., :512]).max()
    shift = inp.scale * np.abs(qa).sum(axis=-1).max() * dc
    assert np.abs(l1 - l2).max() <= shift
    assert 0 < np.abs(o1 - o2).max() <= (math.exp(2 * shift) - 1) * np.abs(full[..., :512]).max() + dc


def test_append_writes_the_bf16_append_slots():
    inp = make_custom(14, 4, 3, [130, 64, 2, 1])
    pool8 = F.quantize_pool(inp.pool)
    rng = np.random.default_rng(15)
    rows = rng.normal(0, 1, (4, 3, 576))
    rows_bits = oracle.f64_to_bf16_bits(rows)
    new16 = oracle.append_to_pool(inp.pool, rows_bits, inp.block_table, inp.seqlens, 3, 4096)
    new8 = F.append_to_pool_mxfp8(pool8, rows, inp.block_table, inp.seqlens, 3, 4096)
    ch16 = {tuple(x) for x in np.argwhere(np.any(new16 != inp.pool, axis=-1))}
    ch8 = {tuple(x) for x in np.argwhere(np.any(new8 != pool8, axis=-1))}
    assert ch8 == ch16 and len(ch8) == 3 + 3 + 2 + 1
    # positions at or past max_pos are skipped (sequence 0 writes 127..129, sequence 1 61..63)
    short8 = F.append_to_pool_mxfp8(pool8, rows, inp.block_table, inp.seqlens, 3, 100)
    short16 = oracle.append_to_pool(inp.pool, rows_bits, inp.block_table, inp.seqlens, 3, 100)
    assert {tuple(x) for x in np.argwhere(np.any(short8 != pool8, axis=-1))} == \
        {tuple(x) for x in np.argwhere(np.any(short16 != inp.pool, axis=-1))}
    assert int(np.count_nonzero(np.any(short8 != pool8, axis=-1))) == 3 + 2 + 1
    for b in range(4):
        for i in range(3):
            p = int(inp.seqlens[b]) - 3 + i
            if p < 0:
                continue
            pg = int(inp.block_table[b, p // 64])
            got = F.unpack_rows(new8[pg, p % 64])
            assert np.array_equal(got[512:], oracle.bf16_bits_to_f64(rows_bits[b, i, 512:]))
            codes, scales = F.mx_quantize(rows[b, i, :512])
            assert np.array_equal(got[:512], F.mx_dequantize(codes, scales))
