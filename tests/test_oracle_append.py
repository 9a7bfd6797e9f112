"""Pins the fp64 cache-append oracle (down-projection, rotary tables, RoPE
rotation, slot write, query rotation) to things other than itself: printed
closed-form angles and textbook cosine values, complex multiplication, exact
quarter turns, the relative-position property of RoPE, scalar brute force,
one-hot hidden states, and consistency with the (separately pinned) page
gather."""

import math

import numpy as np
import pytest

import oracle
from synth import make_append_inputs, make_custom

COS1 = 0.5403023058681398      # cos(1 rad)
SIN1 = 0.8414709848078965      # sin(1 rad)
TEN_POW_M3875 = 1.333521432163324e-4   # 10 ** -3.875 = 10000 ** (-62 / 64)


# --------------------------------------------------------------------------- tables


def test_table_row_zero_is_the_identity():
    t = oracle.rope_table(4)
    assert t.dtype == np.float32 and t.shape == (4, 64)
    assert np.array_equal(t[0], np.r_[np.ones(32), np.zeros(32)].astype(np.float32))


def test_table_closed_form_angles():
    a = oracle.rope_angles(200)
    assert a.shape == (200, 32)
    assert a[1, 0] == 1.0                                   # theta_0 = 1
    assert abs(a[10, 8] - 1.0) < 1e-14                      # theta_8 = 10000^(-1/4) = 0.1
    assert abs(a[100, 16] - 1.0) < 1e-14                    # theta_16 = 10000^(-1/2) = 0.01
    assert abs(a[1, 31] / TEN_POW_M3875 - 1.0) < 1e-14      # theta_31 = 10000^(-62/64)
    t = oracle.rope_table(200)
    assert t[1, 0] == np.float32(COS1) and t[1, 32] == np.float32(SIN1)
    assert abs(t[100, 16] - COS1) < 1e-7 and abs(t[100, 48] - SIN1) < 1e-7
    assert abs(t[10, 8] - COS1) < 1e-7 and abs(t[10, 40] - SIN1) < 1e-7


def test_table_other_base_and_width():
    a = oracle.rope_angles(3, d_r=8, base=16.0)            # theta_i = 16^(-i/4) = 2^-i
    assert np.array_equal(a[2], 2.0 * np.array([1.0, 0.5, 0.25, 0.125]))


def test_table_is_linear_in_position():
    """cos((p+q) theta) = cos p cos q - sin p sin q: the angle grows linearly with p."""
    t = oracle.rope_table(70000).astype(np.float64)
    for p, q in [(1, 1), (7, 300), (4096, 61000), (123, 65000)]:
        c = t[p, :32] * t[q, :32] - t[p, 32:] * t[q, 32:]
        s = t[p, 32:] * t[q, :32] + t[p, :32] * t[q, 32:]
        assert np.max(np.abs(c - t[p + q, :32])) < 4e-7
        assert np.max(np.abs(s - t[p + q, 32:])) < 4e-7
    assert np.max(np.abs(t[:, :32] ** 2 + t[:, 32:] ** 2 - 1.0)) < 3e-7


def test_long_positions_keep_phase_in_fp32_table():
    """Entries at p = 131071 are within fp32 rounding of the fp64 values: the angle is not an fp32 product."""
    t = oracle.rope_table(131072)
    p = 131071
    exact = np.array([math.cos(p * 10000.0 ** (-2 * i / 64)) for i in range(32)])
    assert np.max(np.abs(t[p, :32] - exact)) <= 2.0 ** -24


# --------------------------------------------------------------------------- rotation


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 64))
    phi = rng.uniform(-7.0, 7.0, (5, 32))
    tab = np.concatenate([np.cos(phi), np.sin(phi)], axis=1)
    z = (v[:, 0::2] + 1j * v[:, 1::2]) * np.exp(1j * phi)
    got = oracle.rope_rotate(v, tab)
    assert np.max(np.abs(got[:, 0::2] - z.real)) < 1e-13
    assert np.max(np.abs(got[:, 1::2] - z.imag)) < 1e-13


def test_quarter_turn_and_half_turn_exact():
    v = np.arange(1.0, 65.0)
    quarter = np.r_[np.zeros(32), np.ones(32)]
    got = oracle.rope_rotate(v, quarter)
    assert np.array_equal(got[0::2], -v[1::2]) and np.array_equal(got[1::2], v[0::2])
    half = np.r_[-np.ones(32), np.zeros(32)]
    assert np.array_equal(oracle.rope_rotate(v, half), -v)


def test_rotation_keeps_pair_norms_and_position_zero():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((9, 64))
    t = oracle.rope_table(9, dtype=np.float64)
    got = oracle.rope_rotate(v, t)
    n0 = v[:, 0::2] ** 2 + v[:, 1::2] ** 2
    n1 = got[:, 0::2] ** 2 + got[:, 1::2] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-12
    assert np.array_equal(got[0], v[0])


def test_relative_position_property():
    """<R(m) q, R(n) k> depends on m - n only."""
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    t = oracle.rope_table(5000, dtype=np.float64)

    def dot(m, n):
        return float(oracle.rope_rotate(q, t[m]) @ oracle.rope_rotate(k, t[n]))

    for m, n in [(5, 3), (100, 0), (17, 17), (3, 40)]:
        base = dot(m, n)
        for s in (1, 64, 999, 4000):
            assert abs(dot(m + s, n + s) - base) < 1e-9
    assert abs(dot(5, 3) - dot(3, 5)) > 1e-3      # not symmetric: the sign of the offset matters


# --------------------------------------------------------------------------- down-projection and rows


def test_down_project_brute_force():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 3, 6))
    w = rng.standard_normal((6, 10))
    got = oracle.down_project(x, w)
    for b in range(2):
        for i in range(3):
            for j in range(10):
                s = 0.0
                for k in range(6):
                    s += x[b, i, k] * w[k, j]
                assert abs(got[b, i, j] - s) < 1e-12


def test_one_hot_hidden_state_selects_a_weight_row():
    _, w_a = make_append_inputs(5, 1, 1, d_model=256)
    t = oracle.rope_table(100)
    for k, p in [(0, 0), (17, 0), (255, 0), (17, 37)]:
        x = np.zeros((1, 1, 256), dtype=np.uint16)
        x[0, 0, k] = 0x3F80                                   # bf16 1.0
        row = oracle.append_rows(x, w_a, t, np.array([[p]]))[0, 0]
        w_row = oracle.bf16_bits_to_f64(w_a[k])
        assert np.array_equal(row[:512], w_row[:512])         # c is W_DKV's row k, unrotated
        if p == 0:
            assert np.array_equal(row[512:], w_row[512:])
        else:
            assert np.max(np.abs(row[512:] - oracle.rope_rotate(w_row[512:], t[p]))) == 0.0
            assert not np.array_equal(row[512:], w_row[512:])


def test_positions_follow_the_decode_visibility_convention():
    pos = oracle.append_positions(np.array([1, 64, 3000]), 2)
    assert np.array_equal(pos, [[-1, 0], [62, 63], [2998, 2999]])


def test_append_writes_the_slot_the_gather_reads():
    inp = make_custom(60, 3, 2, [2, 65, 700], extra_blocks=1)
    x, w_a = make_append_inputs(61, 3, 2, d_model=256)
    t = oracle.rope_table(4096)
    rows, pool = oracle.append_kv(x, w_a, t, inp.block_table, inp.seqlens, inp.pool, 2)
    bits = oracle.f64_to_bf16_bits(rows)
    changed = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(3):
        L = int(inp.seqlens[b])
        g = oracle.gather_rows(pool, inp.block_table, b, L)
        assert np.array_equal(g[L - 2:], bits[b])
        assert np.array_equal(g[:L - 2], oracle.gather_rows(inp.pool, inp.block_table, b, L - 2))
        for p in (L - 2, L - 1):
            changed[inp.block_table[b, p // 64], p % 64] = True
    assert np.array_equal(pool[~changed], inp.pool[~changed])


def test_append_skips_slots_that_do_not_exist():
    inp = make_custom(62, 3, 1, [10, 64, 129])
    x, w_a = make_append_inputs(63, 3, 1, d_model=256)
    bt = inp.block_table.copy()
    bt[1, 0] = -1                                  # sequence 1: no page for its new token
    t = oracle.rope_table(100)                     # sequence 2's position 128 is past the table
    _, pool = oracle.append_kv(x, w_a, t, bt, inp.seqlens, inp.pool, 1)
    diff = np.argwhere(np.any(pool != inp.pool, axis=-1))
    assert diff.tolist() == [[int(bt[0, 0]), 9]]
    seqlens = inp.seqlens.copy()
    seqlens[0] = 200                               # past the block-table row
    _, pool2 = oracle.append_kv(x, w_a, oracle.rope_table(300), bt, seqlens, inp.pool, 1)
    assert np.argwhere(np.any(pool2 != inp.pool, axis=-1)).tolist() == [[int(bt[2, 2]), 0]]


def test_query_and_key_turn_the_same_way():
    """The RoPE score of the query at position m and the appended key at n depends on m - n only."""
    rng = np.random.default_rng(7)
    x, w_a = make_append_inputs(8, 1, 1, d_model=256)
    u = rng.standard_normal((1, 1, 4, 64))
    t = oracle.rope_table(3000, dtype=np.float64)

    def score(m, n):
        q = oracle.rope_q(u, t, np.array([[m]]))[0, 0]
        k = oracle.append_rows(x, w_a, t, np.array([[n]]))[0, 0, 512:]
        return q @ k

    for m, n in [(10, 4), (0, 0), (2, 900)]:
        ref = score(m, n)
        for s in (1, 63, 2000):
            assert np.max(np.abs(score(m + s, n + s) - ref)) < 1e-9
    a = score(10, 4)
    assert np.max(np.abs(score(4, 10) - a)) > 1e-3


def test_rope_q_leaves_positions_without_a_table_row():
    rng = np.random.default_rng(9)
    u = rng.standard_normal((2, 1, 3, 64))
    t = oracle.rope_table(50)
    got = oracle.rope_q(u, t, np.array([[49], [50]]))
    assert np.array_equal(got[1], u[1])
    assert np.max(np.abs(got[0] - oracle.rope_rotate(u[0], t[49]))) == 0.0


@pytest.mark.parametrize("p", [0, 1, 4095])
def test_rope_q_each_head_uses_the_token_angles(p):
    rng = np.random.default_rng(10)
    u = rng.standard_normal((1, 1, 5, 64))
    t = oracle.rope_table(4096)
    got = oracle.rope_q(u, t, np.array([[p]]))[0, 0]
    phi = oracle.rope_angles(4096)[p]
    z = (u[0, 0, :, 0::2] + 1j * u[0, 0, :, 1::2]) * np.exp(1j * phi)[None, :]
    assert np.max(np.abs(got[:, 0::2] - z.real)) < 1e-6 and np.max(np.abs(got[:, 1::2] - z.imag)) < 1e-6
