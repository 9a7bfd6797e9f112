"""GPU properties that hold at any size: bitwise reproducibility, independence
from physical page placement, split-count invariance, NaN poison in unread
rows, a dominant needle token, and the degenerate cases."""

import numpy as np
import pytest

import oracle
from synth import make_custom, poison_unused

from ._gpu import LSE_ATOL, absorbed_inputs, assert_close, dev_bf16, dev_i32, host_bits, require_gpu, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


import mla_latent_kv_04_amd as mla  # noqa: E402
import torch  # noqa: E402


def _run(inp, pool, bt, qa_bits, num_splits=0, q_r=None):
    ol, lse = mla.decode_paged(dev_bf16(qa_bits), dev_bf16(inp.q_r if q_r is None else q_r), pool, bt,
                               dev_i32(inp.seqlens), scale=inp.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return host_bits(ol), lse.cpu().numpy()


def test_run_to_run_and_page_placement_bitwise():
    inp = make_custom(51, 4, 1, [3000, 64, 1, 777], permute=False, extra_blocks=1)
    qa = absorbed_inputs(inp)
    d = upload(inp)
    a1, l1 = _run(inp, d["pool"], d["bt"], qa, num_splits=16)
    a2, l2 = _run(inp, d["pool"], d["bt"], qa, num_splits=16)
    assert np.array_equal(a1, a2) and np.array_equal(l1, l2)
    perm = np.random.default_rng(3).permutation(inp.num_pages)
    pool2 = np.empty_like(inp.pool)
    pool2[perm] = inp.pool
    bt2 = np.where(inp.block_table >= 0, perm[np.maximum(inp.block_table, 0)], -1)
    a3, l3 = _run(inp, dev_bf16(pool2), dev_i32(bt2), qa, num_splits=16)
    assert np.array_equal(a1, a3) and np.array_equal(l1, l3)


def test_split_count_invariance():
    inp = make_custom(52, 3, 2, [5000, 300, 2], extra_blocks=1)
    qa = absorbed_inputs(inp)
    d = upload(inp)
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, 2, inp.scale)
    base = None
    for ns in (1, 2, 7, 64, 300, 0):
        ol, lse = _run(inp, d["pool"], d["bt"], qa, num_splits=ns)
        got = oracle.bf16_bits_to_f64(ol)
        assert_close(got, ref_ol, f"splits={ns}")
        assert np.max(np.abs(lse - ref_lse)) <= LSE_ATOL
        if base is None:
            base = got
        assert_close(got, base, f"splits={ns} vs 1")


def test_nan_poison_in_unread_rows_and_pages():
    inp = make_custom(53, 3, 2, [130, 1, 64], extra_blocks=3)
    qa = absorbed_inputs(inp)
    clean_ol, clean_lse = _run(inp, dev_bf16(inp.pool), dev_i32(inp.block_table), qa, num_splits=5)
    poisoned = poison_unused(make_custom(53, 3, 2, [130, 1, 64], extra_blocks=3))
    # an unused table entry pointing outside the pool must not be read either
    bt = poisoned.block_table.copy()
    bt[bt < 0] = 10 ** 6
    p_ol, p_lse = _run(inp, dev_bf16(poisoned.pool), dev_i32(bt), qa, num_splits=5)
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(p_ol)))
    assert np.array_equal(p_ol, clean_ol) and np.array_equal(p_lse, clean_lse)


@pytest.mark.parametrize("s_q,pos", [(1, 0), (1, 63), (1, 64), (1, 2999), (2, 2999)])
def test_needle_takes_all_the_weight(s_q, pos):
    L = 3000
    inp = make_custom(54, 1, s_q, [L], extra_blocks=1)
    qa = np.zeros((1, s_q, 128, 512), dtype=np.uint16)                 # content term zero
    q_r = np.full((1, s_q, 128, 64), 0x3F80, dtype=np.uint16)          # q_R = 1
    pool = inp.pool.copy()
    pool[..., 512:] = 0                                                # k_R = 0 ...
    alpha = 45.0 / (64 * inp.scale)                                    # ... except the needle: score 45 above the rest
    page = inp.block_table[0, pos // 64]
    pool[page, pos % 64, 512:] = oracle.f64_to_bf16_bits(np.full(64, alpha))
    ol, _ = _run(inp, dev_bf16(pool), dev_i32(inp.block_table), qa, num_splits=7, q_r=q_r)
    got = oracle.bf16_bits_to_f64(ol)
    c = oracle.bf16_bits_to_f64(pool[page, pos % 64, :512])
    for i in range(s_q):
        if pos <= L - s_q + i:
            # weight of the needle is 1 - O(L e^-45): out_latent is c_needle to bf16 rounding
            assert np.max(np.abs(got[0, i] - c[None, :])) <= 2 ** -8 * np.max(np.abs(c))
        else:
            assert np.max(np.abs(got[0, i] - c[None, :])) > 0.1      # the needle is not visible to this query


@pytest.mark.parametrize("margin,pos", [(100.0, 1000), (300.0, 2999), (100.0, 70)])
def test_score_far_above_the_first_tile_redoes_the_segment(margin, pos):
    """A score more than 64 log2 units above its segment's first-tile maximum makes the
    kernel redo the segment with the true maximum; at 100 or 300 (natural units) above
    the rest, exp against the first tile's maximum would overflow fp32."""
    L = 3000
    inp = make_custom(58, 1, 1, [L], extra_blocks=1)
    qa = np.zeros((1, 1, 128, 512), dtype=np.uint16)
    q_r = np.full((1, 1, 128, 64), 0x3F80, dtype=np.uint16)
    pool = inp.pool.copy()
    pool[..., 512:] = 0
    alpha = margin / (64 * inp.scale)
    page = inp.block_table[0, pos // 64]
    pool[page, pos % 64, 512:] = oracle.f64_to_bf16_bits(np.full(64, alpha))
    a_bf16 = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(np.array([alpha])))[0]
    needle_score = 64 * a_bf16 * inp.scale                          # the score after bf16 rounding of k_R
    ol, lse = _run(inp, dev_bf16(pool), dev_i32(inp.block_table), qa, num_splits=7, q_r=q_r)
    got = oracle.bf16_bits_to_f64(ol)
    c = oracle.bf16_bits_to_f64(pool[page, pos % 64, :512])
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got[0, 0] - c[None, :])) <= 2 ** -8 * np.max(np.abs(c))
    # lse = needle + ln(1 + (L - 1) e^-needle) = needle to fp32 precision
    assert np.max(np.abs(lse[0, 0] - needle_score)) <= 1e-5 * needle_score + 1e-3


def test_single_token_bit_exact():
    inp = make_custom(55, 3, 1, [1, 1, 1])
    qa = absorbed_inputs(inp)
    ol, lse = _run(inp, dev_bf16(inp.pool), dev_i32(inp.block_table), qa)
    for b in range(3):
        row = inp.pool[inp.block_table[b, 0], 0, :512]
        assert np.array_equal(ol[b, 0], np.broadcast_to(row, (128, 512)))


def test_no_visible_tokens_and_empty_batch():
    inp = make_custom(56, 2, 2, [1, 5])
    qa = absorbed_inputs(inp)
    ol, lse = _run(inp, dev_bf16(inp.pool), dev_i32(inp.block_table), qa)
    got = oracle.bf16_bits_to_f64(ol)
    assert np.all(got[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))       # query 0 of a length-1 step sees nothing
    row = inp.pool[inp.block_table[0, 0], 0, :512]
    assert np.array_equal(ol[0, 1], np.broadcast_to(row, (128, 512)))
    ref_ol, _ = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, 2, inp.scale, batches=[1])
    assert_close(got[1:], ref_ol, "out_latent")
    e = torch.empty(0, 1, 128, 512, dtype=torch.bfloat16, device="cuda")
    ol0, lse0 = mla.decode_paged(e, torch.empty(0, 1, 128, 64, dtype=torch.bfloat16, device="cuda"),
                                 dev_bf16(inp.pool), dev_i32(np.zeros((0, 1))), dev_i32(np.zeros(0)))
    assert ol0.shape == (0, 1, 128, 512)


def test_max_table_row_fully_used():
    # every entry of the table row is used: L = max_blocks * 64 exactly
    inp = make_custom(57, 2, 1, [64 * 40, 64 * 40])
    qa = absorbed_inputs(inp)
    ol, lse = _run(inp, dev_bf16(inp.pool), dev_i32(inp.block_table), qa, num_splits=9)
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, 1, inp.scale)
    assert_close(oracle.bf16_bits_to_f64(ol), ref_ol, "out_latent")


@pytest.mark.parametrize("s_q,num_splits", [(1, 0), (2, 0), (1, 9)])
def test_sequences_sharing_pages(s_q, num_splits):
    """Several sequences whose block-table rows name the same few physical pages (a shared
    prefix cache; the benchmark's L2-resident leg maps every page onto the first 32 the same
    way): each sequence still sees exactly its own table, page by page."""
    inp = make_custom(57, 5, s_q, [700, 64, 1500, 33, 2048])
    shared = 7
    bt = np.where(inp.block_table >= 0, inp.block_table % shared, -1).astype(np.int32)
    print(f"[case] shared pages={shared} s_q={s_q} splits={num_splits} seqlens={inp.seqlens.tolist()}", flush=True)
    qa = absorbed_inputs(inp)
    ol, lse = _run(inp, dev_bf16(inp.pool), dev_i32(bt), qa, num_splits=num_splits)
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, bt, inp.seqlens, s_q, inp.scale)
    assert_close(oracle.bf16_bits_to_f64(ol), ref_ol, "out_latent over shared pages")
    assert np.max(np.abs(lse - ref_lse)) <= LSE_ATOL
