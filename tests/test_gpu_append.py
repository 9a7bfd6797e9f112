"""GPU parity of the cache-append step (down-projection, fp32 RoPE key, slot
write), the query rotation and the rotary table, against the fp64 oracle.

Tolerance, from the arithmetic: the kernels multiply bf16 by bf16 exactly in
fp32 and round at most once per MFMA k-step of 32 products, per split partial
and per rotation operation, so a projected value carries an fp32 error of at
most E = (d/32 + 64) 2^-24 S, S = sum_k |x_k W_kn| (for the rotated key, the
cosine/sine-weighted S of its pair plus 4 2^-24 (|a cos| + |b sin|)), and is
then rounded once to bf16 (half an ulp, at most 2^-8 of the value).  Every
element must satisfy |gpu - exact| <= E + 2^-8 (|exact| + E).  Since E is far
below a bf16 ulp except where a sum cancels to a small value, the kernel's bits
equal the oracle's round-to-nearest-even of the exact value for all but at most
1% of the elements.  Rows the call must not write are compared bit for bit."""

import numpy as np
import pytest

import oracle
from synth import make_append_inputs, make_custom, make_inputs

from ._gpu import (assert_bf16_match, assert_close, dev_bf16, dev_i32, host_bits, projection_err,
                   require_gpu, rotation_err)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


import mla_latent_kv_04_amd as mla  # noqa: E402
import torch  # noqa: E402

MAX_POS = 131072


@pytest.fixture(scope="module")
def tables():
    """(device table written by the library, host table of the oracle) -- built independently."""
    dev = mla.rope_table(MAX_POS)
    torch.cuda.synchronize()
    return dev, oracle.rope_table(MAX_POS)


def _ordered(bits):
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def test_rope_table_matches_oracle(tables):
    dev, ref = tables
    got = dev.cpu().numpy()
    assert got.shape == ref.shape == (MAX_POS, 64)
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    # signs agree wherever the value is not tiny; entries are fp32 roundings of the same fp64 values
    assert np.max(np.abs(got.astype(np.float64) - ref)) <= 2.0 ** -24
    assert np.count_nonzero(ulps) <= 1e-4 * ulps.size
    assert np.array_equal(got[0], ref[0])


def _run_append(inp, x, w_a, dev_table):
    pool = dev_bf16(inp.pool)
    mla.append_kv(dev_bf16(x), dev_bf16(w_a), dev_table, pool, dev_i32(inp.block_table), dev_i32(inp.seqlens))
    torch.cuda.synchronize()
    return host_bits(pool)


CASES = [
    # (name, seed, batch, s_q, seqlens, d_model)
    ("ragged-b5-d7168", 70, 5, 1, [1, 64, 65, 3000, 130], 7168),
    ("verify-b3-d7168", 71, 3, 2, [2, 64, 4097], 7168),
    ("130-tokens-d2048", 72, 65, 2, None, 2048),
    ("1024-tokens-d1024", 73, 1, 1024, [5000], 1024),
    ("4096-tokens-d512", 74, 2, 2048, [2048, 2500], 512),
    ("one-slab-d256", 75, 7, 1, [9, 1, 64, 127, 128, 129, 700], 256),
    ("two-slabs-per-split-d16384", 84, 3, 1, [5, 64, 1000], 16384),
    ("seven-splits-d3584", 85, 64, 1, None, 3584),
    ("d768-64-columns", 86, 4, 2, [2, 3, 64, 65], 768),
]


@pytest.mark.parametrize("name,seed,batch,s_q,seqlens,d", CASES, ids=[c[0] for c in CASES])
def test_append_parity(tables, name, seed, batch, s_q, seqlens, d):
    if seqlens is None:
        seqlens = np.random.default_rng(seed).integers(2, 300, batch)
    inp = make_custom(seed, batch, s_q, seqlens, extra_blocks=1)
    x, w_a = make_append_inputs(seed + 1000, batch, s_q, d_model=d)
    print(f"append parity {name}: T={batch * s_q} d={d}", flush=True)
    got_pool = _run_append(inp, x, w_a, tables[0])
    rows, ref_pool = oracle.append_kv(x, w_a, tables[1], inp.block_table, inp.seqlens, inp.pool, s_q)
    written = np.any(ref_pool != inp.pool, axis=-1) | np.any(got_pool != inp.pool, axis=-1)
    # rows outside the new tokens' slots: bit for bit untouched
    pos = oracle.append_positions(inp.seqlens, s_q)
    slots = np.zeros(inp.pool.shape[:2], dtype=bool)
    for b in range(batch):
        for i in range(s_q):
            pg, r = oracle.slot_of(inp.block_table, b, int(pos[b, i]), inp.num_pages)
            slots[pg, r] = True
    assert not np.any(written & ~slots)
    assert np.array_equal(got_pool[~slots], inp.pool[~slots])
    got_rows = np.stack([np.stack([got_pool[oracle.slot_of(inp.block_table, b, int(pos[b, i]), inp.num_pages)]
                                   for i in range(s_q)]) for b in range(batch)])
    E = projection_err(x, w_a, tables[1], pos)
    assert_bf16_match(got_rows[..., :512], rows[..., :512], E[..., :512], f"{name} latent")
    assert_bf16_match(got_rows[..., 512:], rows[..., 512:], E[..., 512:], f"{name} rope key")


def test_append_is_bitwise_reproducible(tables):
    inp = make_custom(76, 4, 1, [100, 200, 300, 4000])
    x, w_a = make_append_inputs(77, 4, 1)
    a = _run_append(inp, x, w_a, tables[0])
    b = _run_append(inp, x, w_a, tables[0])
    assert np.array_equal(a, b)


def test_append_skips_slots_that_do_not_exist(tables):
    inp = make_custom(78, 4, 1, [10, 64, 129, 50])
    x, w_a = make_append_inputs(79, 4, 1, d_model=512)
    bt = inp.block_table.copy()
    bt[1, 0] = -1                            # no page for sequence 1's new token
    bt[3, 0] = inp.num_pages + 5             # page id past the pool
    seqlens = inp.seqlens.copy()
    seqlens[2] = 64 * bt.shape[1] + 1        # position past the block-table row
    pool = dev_bf16(inp.pool)
    small = tables[0][:10]                   # sequence 0's position 9 is the table's last row
    mla.append_kv(dev_bf16(x), dev_bf16(w_a), small.contiguous(), pool, dev_i32(bt), dev_i32(seqlens))
    torch.cuda.synchronize()
    got = host_bits(pool)
    changed = np.argwhere(np.any(got != inp.pool, axis=-1)).tolist()
    assert changed == [[int(bt[0, 0]), 9]]
    rows, ref_pool = oracle.append_kv(x, w_a, tables[1][:10], bt, seqlens, inp.pool, 1)
    E = projection_err(x[0, 0], w_a, tables[1][:10], 9)
    assert_bf16_match(got[int(bt[0, 0]), 9], rows[0, 0], E, "the one valid row")
    assert np.array_equal(np.argwhere(np.any(ref_pool != inp.pool, axis=-1)).tolist(), changed)


def test_append_full_size_decode_step(tables):
    """The launch the benchmark times: 64 sequences of the batch-64 32K workload, one new
    token each, hidden size 7168, into the full shared pool (about 1.2 GB)."""
    inp = make_inputs("c3", with_pool=False)
    x, w_a = make_append_inputs(80, inp.batch, 1)
    print(f"append full size: pool pages={inp.num_pages}", flush=True)
    pattern = np.int16(0x1234)
    pool = torch.full((inp.num_pages, 64, 576), int(pattern), dtype=torch.int16, device="cuda")
    mla.append_kv(dev_bf16(x), dev_bf16(w_a), tables[0], pool.view(torch.bfloat16), dev_i32(inp.block_table),
                  dev_i32(inp.seqlens))
    torch.cuda.synchronize()
    changed = torch.nonzero((pool != pattern).any(dim=-1)).cpu().numpy()
    pos = oracle.append_positions(inp.seqlens, 1)[:, 0]
    slots = sorted(oracle.slot_of(inp.block_table, b, int(pos[b]), inp.num_pages) for b in range(inp.batch))
    assert sorted(map(tuple, changed.tolist())) == slots
    got = np.stack([host_bits(pool[pg, r].view(torch.bfloat16)) for pg, r in
                    (oracle.slot_of(inp.block_table, b, int(pos[b]), inp.num_pages) for b in range(inp.batch))])
    rows = oracle.append_rows(x, w_a, tables[1], pos[:, None])[:, 0]
    E = projection_err(x[:, 0], w_a, tables[1], pos)
    assert_bf16_match(got[:, :512], rows[:, :512], E[:, :512], "latent")
    assert_bf16_match(got[:, 512:], rows[:, 512:], E[:, 512:], "rope key")


@pytest.mark.parametrize("batch,s_q,heads,seqlens", [(3, 1, 128, [1, 64, 131072]), (2, 2, 128, [2, 70000]),
                                                       (1, 3, 5, [40])])
def test_rope_q_parity(tables, batch, s_q, heads, seqlens):
    rng = np.random.default_rng(81 + batch)
    from synth import f32_to_bf16_bits
    q = f32_to_bf16_bits(rng.standard_normal((batch, s_q, heads, 64), dtype=np.float32))
    sl = np.asarray(seqlens, dtype=np.int32)
    t = dev_bf16(q)
    mla.rope_q(t, tables[0], dev_i32(sl))
    torch.cuda.synchronize()
    got = host_bits(t)
    pos = oracle.append_positions(sl, s_q)
    ref = oracle.rope_q(q, tables[1], pos)
    qf = oracle.bf16_bits_to_f64(q)
    t = tables[1].astype(np.float64)[np.clip(pos, 0, MAX_POS - 1)][:, :, None, :]
    assert_bf16_match(got, ref, rotation_err(qf[..., 0::2], qf[..., 1::2], t[..., :32], t[..., 32:]), "rotated q_R")


def test_rope_q_leaves_positions_without_a_table_row(tables):
    rng = np.random.default_rng(90)
    from synth import f32_to_bf16_bits
    q = f32_to_bf16_bits(rng.standard_normal((3, 2, 128, 64), dtype=np.float32))
    sl = np.array([1, 100, 101], dtype=np.int32)     # positions (-1, 0), (98, 99), (99, 100)
    t = dev_bf16(q)
    mla.rope_q(t, tables[0][:100].contiguous(), dev_i32(sl))
    torch.cuda.synchronize()
    got = host_bits(t)
    assert np.array_equal(got[0, 0], q[0, 0]) and np.array_equal(got[2, 1], q[2, 1])
    assert np.array_equal(got[0, 1], q[0, 1])        # position 0 is the identity rotation
    pos = oracle.append_positions(sl, 2)
    ref = oracle.rope_q(q, tables[1][:100], pos)
    qf = oracle.bf16_bits_to_f64(q)
    t = tables[1].astype(np.float64)[np.clip(pos, 0, 99)][:, :, None, :]
    assert_bf16_match(got, ref, rotation_err(qf[..., 0::2], qf[..., 1::2], t[..., :32], t[..., 32:]), "rotated q_R")


def test_append_then_decode_sees_the_new_rows(tables):
    """Append the new tokens' rows, rotate their queries, decode: against the oracle doing the same."""
    inp = make_custom(82, 3, 2, [2, 700, 4099], extra_blocks=1)
    x, w_a = make_append_inputs(83, 3, 2)
    q_abs = oracle.f64_to_bf16_bits(oracle.absorb_q(inp.q_c, inp.w_uk))
    pos = oracle.append_positions(inp.seqlens, 2)
    pool = dev_bf16(inp.pool)
    q_r = dev_bf16(inp.q_r)
    mla.append_kv(dev_bf16(x), dev_bf16(w_a), tables[0], pool, dev_i32(inp.block_table), dev_i32(inp.seqlens))
    mla.rope_q(q_r, tables[0], dev_i32(inp.seqlens))
    ol, lse = mla.decode_paged(dev_bf16(q_abs), q_r, pool, dev_i32(inp.block_table), dev_i32(inp.seqlens),
                               scale=inp.scale)
    torch.cuda.synchronize()
    _, ref_pool = oracle.append_kv(x, w_a, tables[1], inp.block_table, inp.seqlens, inp.pool, 2)
    ref_qr = oracle.f64_to_bf16_bits(oracle.rope_q(inp.q_r, tables[1], pos))
    ref_ol, ref_lse = oracle.decode_absorbed(q_abs, ref_qr, ref_pool, inp.block_table, inp.seqlens, 2, inp.scale)
    assert_close(oracle.bf16_bits_to_f64(host_bits(ol)), ref_ol, "out_latent after append")
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 2e-3 + 2 ** -8 * np.max(np.abs(ref_lse))


@pytest.mark.parametrize("batch,s_q,seqlens,d", [(64, 1, None, 7168), (2, 2048, [2048, 2100], 512),
                                                 (3, 2, [2, 64, 4097], 2048)])
def test_append_rotates_the_query_in_the_same_launch(tables, batch, s_q, seqlens, d):
    if seqlens is None:
        seqlens = np.random.default_rng(87).integers(1, 5000, batch)
    inp = make_custom(88, batch, s_q, seqlens)
    x, w_a = make_append_inputs(89, batch, s_q, d_model=d)
    pool = dev_bf16(inp.pool)
    q_r = dev_bf16(inp.q_r)
    mla.append_kv(dev_bf16(x), dev_bf16(w_a), tables[0], pool, dev_i32(inp.block_table), dev_i32(inp.seqlens),
                  q_r=q_r)
    torch.cuda.synchronize()
    pos = oracle.append_positions(inp.seqlens, s_q)
    ref = oracle.rope_q(inp.q_r, tables[1], pos)
    qf = oracle.bf16_bits_to_f64(inp.q_r)
    t = tables[1].astype(np.float64)[pos][:, :, None, :]
    assert_bf16_match(host_bits(q_r), ref, rotation_err(qf[..., 0::2], qf[..., 1::2], t[..., :32], t[..., 32:]),
                      "q_R rotated by the append launch")
    rows, ref_pool = oracle.append_kv(x, w_a, tables[1], inp.block_table, inp.seqlens, inp.pool, s_q)
    got_pool = host_bits(pool)
    same = np.all(ref_pool == inp.pool, axis=-1)
    assert np.array_equal(got_pool[same], inp.pool[same])
    E = projection_err(x, w_a, tables[1], pos)
    got_rows = np.stack([np.stack([got_pool[oracle.slot_of(inp.block_table, b, int(pos[b, i]), inp.num_pages)]
                                   for i in range(s_q)]) for b in range(batch)])
    assert_bf16_match(got_rows, rows, E, "rows")


def test_one_workspace_across_plans(tables):
    """Calls with different split plans share one workspace that starts as NaN garbage;
    each result is right."""
    cases = [(64, 1, 7168), (3, 1, 16384), (5, 2, 768), (1, 1024, 1024), (2, 2048, 512), (64, 1, 7168)]
    need = max(mla.append_workspace_size(mla.make_append_params(b, s, d, 80, 4096, MAX_POS)) for b, s, d in cases)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for n, (b, s_q, d) in enumerate(cases):
        seqlens = np.random.default_rng(100 + n).integers(s_q, 64 * 40, b)
        inp = make_custom(100 + n, b, s_q, seqlens)
        x, w_a = make_append_inputs(200 + n, b, s_q, d_model=d)
        pool = dev_bf16(inp.pool)
        mla.append_kv(dev_bf16(x), dev_bf16(w_a), tables[0], pool, dev_i32(inp.block_table), dev_i32(inp.seqlens),
                      workspace=ws)
        torch.cuda.synchronize()
        rows, _ = oracle.append_kv(x, w_a, tables[1], inp.block_table, inp.seqlens, inp.pool, s_q)
        pos = oracle.append_positions(inp.seqlens, s_q)
        got_pool = host_bits(pool)
        got_rows = np.stack([np.stack([got_pool[oracle.slot_of(inp.block_table, bb, int(pos[bb, i]), inp.num_pages)]
                                       for i in range(s_q)]) for bb in range(b)])
        assert_bf16_match(got_rows, rows, projection_err(x, w_a, tables[1], pos), f"case {n}")
