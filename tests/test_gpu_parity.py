"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar: block-table gathers bit-exact; floating outputs within
max|gpu - ref| <= 1e-2 * max|ref| + 2e-3 per output tensor; lse within 2e-3 when
both sides score with the same bf16 q_abs, and within the derived bf16-rounding
bound of scale * 2^-8 * sum|q_abs c| (+2e-3) against the unrounded definition.
Paged-decode parity feeds both sides the same bf16 q_abs (RNE of the exact
q_c . W_UK); the fused path is checked against the decompress oracle."""

import numpy as np
import pytest

import oracle
from synth import make_custom, make_inputs

from ._gpu import (LSE_ATOL, absorbed_inputs, assert_close, dev_bf16, host_bits, host_f64,
                   lse_bound_for_rounded_q, require_gpu, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


import mla_latent_kv_04_amd as mla  # noqa: E402


def _print_case(name, inp):
    print(f"[case] {name} seed={inp.seed} B={inp.batch} s_q={inp.s_q} L={list(inp.seqlens[:8])}"
          f"{'...' if inp.batch > 8 else ''} pages={inp.num_pages}", flush=True)


def _paged(inp, d, qa_bits, num_splits=0):
    qa = dev_bf16(qa_bits)
    ol, lse = mla.decode_paged(qa, d["q_r"], d["pool"], d["bt"], d["sl"], scale=inp.scale, num_splits=num_splits)
    import torch
    torch.cuda.synchronize()
    return ol, lse


# ------------------------------------------------------------------ gather

@pytest.mark.parametrize("seqlens", [[1, 64, 65, 300], [4096] * 3])
def test_gather_bit_exact(seqlens):
    inp = make_custom(21, len(seqlens), 1, seqlens, extra_blocks=1)
    _print_case("gather", inp)
    d = upload(inp)
    dense = host_bits(mla.gather_kv(d["pool"], d["bt"], d["sl"]))
    mb = inp.max_blocks
    want = np.zeros((inp.batch, mb * 64, 576), dtype=np.uint16)
    for b in range(inp.batch):
        L = int(inp.seqlens[b])
        want[b, :L] = oracle.gather_rows(inp.pool, inp.block_table, b, L)
    assert np.array_equal(dense, want)


# ------------------------------------------------------------------ projections

@pytest.mark.parametrize("tokens", [1, 17, 64, 65, 130, 192])
def test_absorb_q(tokens):
    inp = make_custom(22, tokens, 1, [1] * tokens)
    d = upload(inp)
    got = host_f64(mla.absorb_q(d["q_c"], d["w_uk"]))
    ref = oracle.absorb_q(inp.q_c, inp.w_uk)
    assert_close(got, ref, "q_abs")
    # tighter: each value is the bf16 rounding of an fp32 sum of 128 products
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 1e-3)) < 2 ** -7


@pytest.mark.parametrize("tokens", [1, 17, 64, 65, 130, 192])
def test_up_proj(tokens):
    inp = make_custom(23, tokens, 1, [1] * tokens)
    rng = np.random.default_rng(5)
    ol_bits = oracle.f64_to_bf16_bits(rng.standard_normal((tokens, 1, 128, 512)))
    d = upload(inp)
    got = host_f64(mla.up_proj(dev_bf16(ol_bits), d["w_uv"]))
    ref = oracle.up_proj(ol_bits, inp.w_uv)
    assert_close(got, ref, "out")
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 1e-3)) < 2 ** -7


# ------------------------------------------------------------------ paged decode, small ragged cases

SMALL = [
    (31, 1, [1, 65, 200]),
    (32, 2, [2, 64, 130]),
    (33, 1, [64, 128, 63, 1000, 7]),
    (34, 2, [3, 65, 640]),
    (35, 1, [2500]),
]


@pytest.mark.parametrize("num_splits", [0, 1, 3, 40])
@pytest.mark.parametrize("seed,s_q,seqlens", SMALL)
def test_decode_paged_small(seed, s_q, seqlens, num_splits):
    inp = make_custom(seed, len(seqlens), s_q, seqlens, extra_blocks=2)
    _print_case(f"paged splits={num_splits}", inp)
    d = upload(inp)
    qa = absorbed_inputs(inp)
    ol, lse = _paged(inp, d, qa, num_splits)
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, s_q, inp.scale)
    assert_close(host_f64(ol), ref_ol, "out_latent")
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) <= LSE_ATOL



@pytest.mark.parametrize("batch,s_q", [(64, 1), (65, 1), (33, 2)])
@pytest.mark.parametrize("num_splits", [0, 40])
def test_decode_paged_around_the_in_kernel_plan_limit(batch, s_q, num_splits):
    """Up to 64 work units (batch x queries) the decode workgroups compute the page prefix
    sums themselves; above that a separate kernel does.  64, 65 and 66 units of short
    ragged sequences (1 to 300 tokens), against the oracle, on both sides of that limit."""
    rng = np.random.default_rng(36 + batch + s_q)
    seqlens = [int(x) for x in rng.integers(s_q, 301, size=batch)]
    inp = make_custom(37 + batch, batch, s_q, seqlens, extra_blocks=1)
    _print_case(f"paged units={batch * s_q} splits={num_splits}", inp)
    d = upload(inp)
    qa = absorbed_inputs(inp)
    ol, lse = _paged(inp, d, qa, num_splits)
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, s_q, inp.scale)
    assert_close(host_f64(ol), ref_ol, "out_latent")
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) <= LSE_ATOL

@pytest.mark.parametrize("batch,s_q", [(40, 1), (70, 1), (36, 2)])
def test_decode_paged_segment_aware_split(batch, s_q):
    """The library's own split over ragged lengths long enough for ranges of 48 tiles or
    more, where it lays the units on a cost line (each unit start counts 6 tiles, so a range
    that takes in a unit start gets fewer tiles): the in-kernel plan (40 units) and the plan
    kernel (70 and 72 units), with sequences that have no visible token, against the oracle
    for every sequence."""
    import bench
    rng = np.random.default_rng(90 + batch + s_q)
    seqlens = [int(x) for x in rng.integers(s_q, 24000, size=batch)]
    seqlens[3] = s_q - 1                      # a sequence whose queries see no token
    seqlens[batch - 1] = 1                    # one token (query 0 of two sees none)
    ranges, seg, _ = bench.split_plan(bench.unit_tiles(seqlens, s_q), 256, True)
    assert seg == bench.SEG_COST and len(ranges) > 200, "the case must exercise the cost-line split"
    inp = make_custom(91 + batch, batch, s_q, seqlens, extra_blocks=1)
    _print_case(f"segment-aware split units={batch * s_q}", inp)
    d = upload(inp)
    qa = absorbed_inputs(inp)
    ol, lse = _paged(inp, d, qa, 0)
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, s_q, inp.scale)
    got = host_f64(ol)
    for b in range(batch):
        assert_close(got[b:b + 1], ref_ol[b:b + 1], f"out_latent seq {b} (L={seqlens[b]})")
    got_lse = lse.double().cpu().numpy()
    empty = np.isneginf(ref_lse)
    assert empty.any() and np.all(np.isneginf(got_lse[empty]))
    assert np.max(np.abs(got_lse[~empty] - ref_lse[~empty])) <= LSE_ATOL


@pytest.mark.parametrize("tiles_per_split", [1, 2, 3])
@pytest.mark.parametrize("s_q", [1, 2])
def test_decode_short_fragments_with_partial_tiles(tiles_per_split, s_q):
    """Split plans whose ranges hold only 1, 2 or 3 tiles of 32 tokens, over lengths around tile
    and page borders (a sequence's last tile often holds a single token): every fragment is
    then a first step, a last step or both, so an error in either cannot be diluted by the
    steady steps of a long range."""
    seqlens = [2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 129, 200]
    inp = make_custom(70 + tiles_per_split + 3 * s_q, len(seqlens), s_q, seqlens, extra_blocks=1)
    tiles = sum(-(-(L - s_q + i + 1) // 32) for L in seqlens for i in range(s_q))
    num_splits = -(-tiles // tiles_per_split)
    _print_case(f"short fragments splits={num_splits}", inp)
    d = upload(inp)
    qa = absorbed_inputs(inp)
    ol, lse = _paged(inp, d, qa, num_splits)
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, s_q, inp.scale)
    got = host_f64(ol)
    for b in range(inp.batch):
        assert_close(got[b:b + 1], ref_ol[b:b + 1], f"out_latent seq {b} (L={seqlens[b]})")
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) <= LSE_ATOL


# ------------------------------------------------------------------ the five workloads
# Every sequence of every workload, paged and fused: tests/test_gpu_00_workloads.py.


# ------------------------------------------------------------------ fused path vs the decompress definition

def test_fused_c1_all_heads():
    inp = make_inputs("c1")
    _print_case("fused c1", inp)
    d = upload(inp)
    out, lse = mla.decode(d["q_c"], d["q_r"], d["w_uk"], d["w_uv"], d["pool"], d["bt"], d["sl"], scale=inp.scale)
    ref, ref_lse = oracle.decode_decompressed(inp.q_c, inp.q_r, inp.w_uk, inp.w_uv, inp.pool, inp.block_table,
                                              inp.seqlens, 1, inp.scale)
    assert_close(host_f64(out), ref, "out")
    # the fused path scores with bf16 q_abs: lse against the unrounded definition within the derived bound
    assert np.all(np.abs(lse.double().cpu().numpy() - ref_lse) <= lse_bound_for_rounded_q(inp))


@pytest.mark.parametrize("seed,s_q,seqlens", [(41, 2, [2, 77, 300]), (42, 1, [1, 4096, 129])])
def test_fused_small_vs_decompressed(seed, s_q, seqlens):
    inp = make_custom(seed, len(seqlens), s_q, seqlens)
    d = upload(inp)
    out, lse = mla.decode(d["q_c"], d["q_r"], d["w_uk"], d["w_uv"], d["pool"], d["bt"], d["sl"], scale=inp.scale,
                          num_splits=5)
    heads = [0, 1, 31, 32, 77, 127]
    ref, ref_lse = oracle.decode_decompressed(inp.q_c, inp.q_r, inp.w_uk, inp.w_uv, inp.pool, inp.block_table,
                                              inp.seqlens, s_q, inp.scale, heads=heads)
    got = host_f64(out)[:, :, heads]
    assert_close(got, ref, "out")
    bound = lse_bound_for_rounded_q(inp, heads=heads)
    assert np.all(np.abs(lse.double().cpu().numpy()[:, :, heads] - ref_lse) <= bound)


# ------------------------------------------------------------------ the page stream alone (ceiling measurement)

def _stream_expected(inp):
    """Sum (mod 2^32) over every 32-token tile of every (sequence, query) unit of the 256
    little-endian dwords of the tile's first row's latent: what mla_stream_pages must read."""
    total = 0
    for b in range(inp.batch):
        L = int(inp.seqlens[b])
        for i in range(inp.s_q):
            n = L - inp.s_q + i + 1
            if n <= 0:
                continue
            rows = oracle.gather_rows(inp.pool, inp.block_table, b, n)[::32, :512]      # first row of each tile
            words = rows.astype(np.uint64).reshape(-1, 256, 2)
            total += int((words[..., 0] | (words[..., 1] << np.uint64(16))).sum())
    return total % (1 << 32)


@pytest.mark.parametrize("num_splits", [0, 1, 3, 40])
@pytest.mark.parametrize("seed,s_q,seqlens", [(61, 1, [1, 33, 64, 65, 300, 2500]), (62, 2, [2, 31, 32, 97, 1000])])
def test_stream_pages_reads_every_tile_once(seed, s_q, seqlens, num_splits):
    inp = make_custom(seed, len(seqlens), s_q, seqlens, extra_blocks=1)
    _print_case(f"stream splits={num_splits}", inp)
    d = upload(inp)
    sums = mla.stream_pages(d["pool"], d["bt"], d["sl"], s_q=s_q, num_splits=num_splits)
    import torch
    torch.cuda.synchronize()
    got = int(sums.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    assert got == _stream_expected(inp)


def test_stream_pages_many_units_and_c3():
    """Above 64 units the prefix sums come from the plan kernel; and the full batch-64 workload
    in the benchmark's configuration."""
    rng = np.random.default_rng(63)
    for inp in (make_custom(64, 70, 1, [int(x) for x in rng.integers(1, 400, size=70)], extra_blocks=1),
                # the plan kernel with the segment-aware split (ranges of 48+ tiles)
                make_custom(65, 70, 1, [int(x) for x in rng.integers(1, 24000, size=70)], extra_blocks=1),
                make_inputs("c3")):
        _print_case("stream", inp)
        d = upload(inp)
        sums = mla.stream_pages(d["pool"], d["bt"], d["sl"])
        import torch
        torch.cuda.synchronize()
        got = int(sums.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
        assert got == _stream_expected(inp)
