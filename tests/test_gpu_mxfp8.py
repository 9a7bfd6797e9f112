"""GPU parity of the MXFP8 latent cache: the bf16 -> MXFP8 conversion (bit-exact
against the oracle's quantiser), the paged and fused decode over an MXFP8 cache
(against the fp64 oracle on the dequantised cache, the bf16 path's bar) and the
cache append into an MXFP8 cache (against the oracle's quantisation of the exact
rows, within a bound derived from the fp32 sums)."""

import numpy as np
import pytest

import oracle
from oracle import fp8_cache as F
from synth import make_append_inputs, make_custom, make_inputs, poison_unused

from ._gpu import (LSE_ATOL, absorbed_inputs, assert_bf16_match, assert_close, dev_bf16, dev_i32, host_bits,
                   host_f64, projection_err, require_gpu, upload)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


import mla_latent_kv_04_amd as mla  # noqa: E402


def _case(name, inp):
    print(f"[case] mxfp8 {name} seed={inp.seed} B={inp.batch} s_q={inp.s_q} L={list(inp.seqlens[:8])}"
          f"{'...' if inp.batch > 8 else ''} pages={inp.num_pages}", flush=True)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host_u8(t):
    return t.contiguous().cpu().numpy()


# ------------------------------------------------------------------ bf16 -> MXFP8


def _edge_pool(seed):
    """Rows that reach the edges of the code: zero blocks, blocks whose maximum is exactly
    448 * 2^k or just above, ties between neighbouring codes, subnormal codes, -0, and a
    wide spread of block magnitudes."""
    rng = np.random.default_rng(seed)
    vals = rng.normal(0, 1, (3, 64, 576)) * np.exp(rng.uniform(-12, 12, (3, 64, 1)))
    pos = F.e4m3_value(np.arange(0x7F))
    mids = (pos[1:] + pos[:-1]) / 2
    r = vals[0]
    r[0, :512] = 0.0                                            # all-zero row
    r[1, :32] = 0.0
    r[1, 5] = -0.0
    r[2, :32] = rng.choice(pos, 32) * 2.0 ** 3
    r[2, 7] = 448.0 * 8                                         # block max exactly 448 * 2^3
    r[3, :32] = mids[rng.integers(0, len(mids), 32)] * 2.0 ** -2
    r[3, 0] = 448.0 / 4                                         # scale 2^-2: ties are exact in bf16
    r[4, :32] = rng.normal(0, 1, 32) * 1e-3
    r[4, 0] = 452.0                                             # just above 448 * 2^0 (exact in bf16)
    r[5, :32] = rng.normal(0, 1e-4, 32)
    r[5, 1] = 3.0                                               # many subnormal codes
    return oracle.f64_to_bf16_bits(vals)


@pytest.mark.parametrize("source", ["edges", "synthetic"])
def test_quantize_bit_exact(source):
    if source == "edges":
        pool = _edge_pool(61)
    else:
        inp = make_custom(62, 3, 1, [300, 64, 1000])
        pool = inp.pool
    print(f"[case] mxfp8 quantize {source} pages={pool.shape[0]}", flush=True)
    got = host_u8(mla.quantize_kv_mxfp8(dev_bf16(pool)))
    torch.cuda.synchronize()
    want = F.quantize_pool(pool)
    assert got.shape == want.shape
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first {bad[:5].tolist()}"


# ------------------------------------------------------------------ decode over an MXFP8 cache


def _upload8(inp):
    d = upload(inp)
    pool8 = F.quantize_pool(inp.pool)
    d["pool8"] = dev_u8(pool8)
    return d, pool8


SMALL = [
    (71, 1, [1, 65, 200]),
    (72, 2, [2, 64, 130]),
    (73, 1, [64, 128, 63, 1000, 7]),
    (74, 2, [3, 65, 640]),
    (75, 1, [2500]),
    (76, 5, [5, 37, 96, 97]),
]


@pytest.mark.parametrize("num_splits", [0, 3, 40])
@pytest.mark.parametrize("seed,s_q,seqlens", SMALL)
def test_decode_paged_small(seed, s_q, seqlens, num_splits):
    inp = make_custom(seed, len(seqlens), s_q, seqlens, extra_blocks=2)
    _case(f"paged splits={num_splits}", inp)
    d, pool8 = _upload8(inp)
    qa = absorbed_inputs(inp)
    ol, lse = mla.decode_paged_mxfp8(dev_bf16(qa), d["q_r"], d["pool8"], d["bt"], d["sl"], scale=inp.scale,
                                     num_splits=num_splits)
    torch.cuda.synchronize()
    deq = F.dequantize_pool(pool8)
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, deq, inp.block_table, inp.seqlens, s_q, inp.scale)
    assert_close(host_f64(ol), ref_ol, "out_latent")
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) <= LSE_ATOL



@pytest.mark.parametrize("num_splits", [0, 40])
def test_decode_paged_above_the_in_kernel_plan_limit(num_splits):
    """65 work units (65 sequences of 1 to 300 tokens): the page prefix sums come from the
    separate plan kernel instead of each workgroup's own scan.  Against the oracle on the
    dequantised cache, and bit for bit against the bf16 kernel on that cache."""
    rng = np.random.default_rng(79)
    seqlens = [int(x) for x in rng.integers(1, 301, size=65)]
    inp = make_custom(79, 65, 1, seqlens, extra_blocks=1)
    _case(f"paged units=65 splits={num_splits}", inp)
    d, pool8 = _upload8(inp)
    qa = absorbed_inputs(inp)
    ol, lse = mla.decode_paged_mxfp8(dev_bf16(qa), d["q_r"], d["pool8"], d["bt"], d["sl"], scale=inp.scale,
                                     num_splits=num_splits)
    deq = F.dequantize_pool(pool8)
    o16, l16 = mla.decode_paged(dev_bf16(qa), d["q_r"], dev_bf16(oracle.f64_to_bf16_bits(deq)), d["bt"], d["sl"],
                                scale=inp.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, deq, inp.block_table, inp.seqlens, 1, inp.scale)
    assert_close(host_f64(ol), ref_ol, "out_latent")
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) <= LSE_ATOL
    assert np.array_equal(host_bits(ol), host_bits(o16)) and torch.equal(lse, l16)

def test_decode_matches_the_bf16_kernel_on_the_dequantised_cache():
    """Both kernels feed the same bf16 tiles to the same MFMA sequence, so over a bf16
    cache holding the dequantised values the MXFP8 decode reproduces the bf16 decode
    bit for bit (an extra check between the two kernels; parity is against the oracle)."""
    inp = make_custom(77, 4, 2, [70, 1, 640, 3000], extra_blocks=1)
    _case("vs bf16 kernel", inp)
    d, pool8 = _upload8(inp)
    qa = dev_bf16(absorbed_inputs(inp))
    deq_bits = oracle.f64_to_bf16_bits(F.dequantize_pool(pool8))
    o8, l8 = mla.decode_paged_mxfp8(qa, d["q_r"], d["pool8"], d["bt"], d["sl"], scale=inp.scale, num_splits=7)
    o16, l16 = mla.decode_paged(qa, d["q_r"], dev_bf16(deq_bits), d["bt"], d["sl"], scale=inp.scale, num_splits=7)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o8), host_bits(o16))
    assert torch.equal(l8, l16)


def test_unused_rows_hold_nan_bytes():
    inp = poison_unused(make_custom(78, 3, 1, [100, 64, 33], extra_blocks=2))
    _case("poisoned", inp)
    pool8 = F.quantize_pool(np.where(np.isnan(oracle.bf16_bits_to_f64(inp.pool)), np.uint16(0), inp.pool))
    used = np.zeros(pool8.shape[:2], dtype=bool)
    for b in range(inp.batch):
        t = np.arange(int(inp.seqlens[b]))
        used[inp.block_table[b, t // 64], t % 64] = True
    pool8[~used] = 0xFF                                   # NaN codes, NaN scale bytes, NaN k_R
    d = upload(inp)
    qa = absorbed_inputs(inp)
    ol, lse = mla.decode_paged_mxfp8(dev_bf16(qa), d["q_r"], dev_u8(pool8), d["bt"], d["sl"], scale=inp.scale,
                                     num_splits=5)
    torch.cuda.synchronize()
    got = host_f64(ol)
    assert np.all(np.isfinite(got))
    ref_ol, ref_lse = oracle.decode_absorbed(qa, inp.q_r, F.dequantize_pool(pool8), inp.block_table, inp.seqlens, 1,
                                             inp.scale)
    assert_close(got, ref_ol, "out_latent")


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_workload_sampled(name):
    """Full-size workloads: the MXFP8 cache made on the device from the workload's bf16
    cache; the oracle quantises the sampled sequences' rows itself."""
    inp = make_inputs(name)
    _case(name, inp)
    d = upload(inp)
    pool8_dev = mla.quantize_kv_mxfp8(d["pool"])
    del d["pool"]
    qa = absorbed_inputs(inp)
    ol, lse = mla.decode_paged_mxfp8(dev_bf16(qa), d["q_r"], pool8_dev, d["bt"], d["sl"], scale=inp.scale)
    torch.cuda.synchronize()
    L = inp.seqlens
    batches = sorted({int(np.argmin(L)), int(np.argmax(L)), inp.batch // 2})
    got = host_f64(ol)[batches]
    glse = lse.double().cpu().numpy()[batches]
    for bi, b in enumerate(batches):
        n = int(L[b])
        rows8 = F.quantize_pool(oracle.gather_rows(inp.pool, inp.block_table, b, n)[None])
        rows = F.unpack_rows(rows8)                        # one "page" holding the sequence's rows in order
        ref_ol, ref_lse = oracle.decode_absorbed(qa[b:b + 1], inp.q_r[b:b + 1], rows,
                                                 np.zeros((1, 1), dtype=np.int32), np.array([n]), inp.s_q, inp.scale)
        assert_close(got[bi:bi + 1], ref_ol, f"out_latent b={b}")
        assert np.max(np.abs(glse[bi:bi + 1] - ref_lse)) <= LSE_ATOL


def test_fused_small_vs_decompressed():
    inp = make_custom(79, 3, 2, [2, 77, 300])
    _case("fused", inp)
    d, pool8 = _upload8(inp)
    out, lse = mla.decode_mxfp8(d["q_c"], d["q_r"], d["w_uk"], d["w_uv"], d["pool8"], d["bt"], d["sl"],
                                scale=inp.scale, num_splits=4)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_decompressed(inp.q_c, inp.q_r, inp.w_uk, inp.w_uv, F.dequantize_pool(pool8),
                                              inp.block_table, inp.seqlens, 2, inp.scale)
    assert_close(host_f64(out), ref, "out")
    # the scores use bf16 q_abs: allow scale * 2^-8 * sum|q_abs c| on top of LSE_ATOL
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) <= 1e-2


# ------------------------------------------------------------------ append into an MXFP8 cache


@pytest.mark.parametrize("batch,s_q,d_model", [(64, 1, 7168), (5, 3, 512), (130, 1, 1024)])
def test_append_mxfp8(batch, s_q, d_model):
    seqlens = [64 * (i % 3) + (i * 37) % 64 + s_q for i in range(batch)]
    inp = make_custom(80 + batch, batch, s_q, seqlens, extra_blocks=1)
    print(f"[case] mxfp8 append B={batch} s_q={s_q} d={d_model}", flush=True)
    x, w_a = make_append_inputs(81, batch, s_q, d_model=d_model)
    pool8 = F.quantize_pool(inp.pool)
    kv8 = dev_u8(pool8)
    table = oracle.rope_table(4096)
    mla.append_kv_mxfp8(dev_bf16(x), dev_bf16(w_a), torch.from_numpy(table).cuda(), kv8, dev_i32(inp.block_table),
                        dev_i32(inp.seqlens))
    torch.cuda.synchronize()
    got = host_u8(kv8)
    pos = oracle.append_positions(inp.seqlens, s_q)
    rows = oracle.append_rows(x, w_a, table, pos)
    want = F.append_to_pool_mxfp8(pool8, rows, inp.block_table, inp.seqlens, s_q, 4096)
    changed = np.any(want != pool8, axis=-1)
    assert np.array_equal(got[~changed], pool8[~changed]), "rows other than the new tokens' changed"
    err = projection_err(x, w_a, table, pos)                  # [B, s_q, 576], before any rounding
    rope_got, rope_exact, rope_err = [], [], []
    for b in range(batch):
        for i in range(s_q):
            p = int(pos[b, i])
            g, w = got[int(inp.block_table[b, p // 64]), p % 64], want[int(inp.block_table[b, p // 64]), p % 64]
            exact, e = rows[b, i, :512], err[b, i, :512]
            gs, ws = g[512:528].astype(int), w[512:528].astype(int)
            # a scale byte may differ only where the block maximum lies within the error of a
            # boundary 448 * 2^X of the oracle's scale 2^X (below it or at it)
            amax = np.abs(exact).reshape(16, 32).max(axis=1)
            e_blk = e.reshape(16, 32).max(axis=1)
            x_or = ws - 127
            near = (np.abs(amax - 448.0 * np.ldexp(1.0, x_or - 1)) <= e_blk) | \
                   (np.abs(amax - 448.0 * np.ldexp(1.0, x_or)) <= e_blk)
            assert np.all((gs == ws) | near), (b, i, gs, ws)
            # the kernel rounds its fp32 value v (|v - exact| <= e) to the code grid of its own
            # scale: half a step, 2^-4 |v| for normal codes, 2^-10 2^X for subnormal ones
            gv = F.mx_dequantize(g[:512], g[512:528])
            step = np.repeat(np.ldexp(1.0, gs - 127), 32)
            bound = e + np.maximum(2.0 ** -4 * (np.abs(exact) + e), 2.0 ** -10 * step)
            assert np.all(np.abs(gv - exact) <= bound), (b, i, float(np.max(np.abs(gv - exact) - bound)))
            frac = np.count_nonzero(g[:512] != w[:512]) / 512
            assert frac <= 0.02, (b, i, frac)
            rope_got.append(np.ascontiguousarray(g[528:]).view("<u2"))
            rope_exact.append(rows[b, i, 512:])
            rope_err.append(err[b, i, 512:])
    # k_R: the fp32 rotation rounded once to bf16, the bf16 append's bar
    assert_bf16_match(np.stack(rope_got), np.stack(rope_exact), np.stack(rope_err), "k_R")
