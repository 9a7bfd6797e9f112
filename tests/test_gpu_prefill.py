"""GPU parity of a prefill chunk against the fp64 oracle: the decompress branch
(per-head K and V expanded from the latent, then causal attention over the
192-wide score), the absorbed branch (the decode with many queries per
sequence), and the threshold dispatch between them.

Tolerances: the expanded K and V are bf16 results of fp32 sums of exact bf16
products, so they are held to the derived bound |gpu - exact| <= E + 2^-8 (|exact| + E)
with E = (512/16 + 64) 2^-24 sum_c |c W| (one fp32 rounding per MFMA k-step of 16
and per chunk).  Attention outputs use the stated tolerance
max|err| <= 1e-2 max|ref| + 2e-3.  lse moves with the bf16 rounding of K (each
score moves by at most scale 2^-8 sum_d |q_d K_d|) and of the queries' inputs,
so it is held to that shift over the visible keys plus 2e-3."""

import numpy as np
import pytest

import oracle
from synth import make_custom, poison_unused

from ._gpu import U, assert_bf16_match, assert_close, dev_bf16, dev_i32, host_bits, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


import mla_latent_kv_04_amd as mla  # noqa: E402
import torch  # noqa: E402

HEADS = [0, 1, 64, 127]


def _run(inp, mode=0, threshold=0, with_ws=False):
    params = mla.make_prefill_params(inp.batch, inp.s_q, inp.max_blocks, inp.num_pages, inp.scale, mode, threshold)
    ws = torch.empty(mla.prefill_workspace_size(params), dtype=torch.uint8, device="cuda")
    out, lse = mla.prefill(dev_bf16(inp.q_c), dev_bf16(inp.q_r), dev_bf16(inp.w_uk), dev_bf16(inp.w_uv),
                           dev_bf16(inp.pool), dev_i32(inp.block_table), dev_i32(inp.seqlens), scale=inp.scale,
                           mode=mode, threshold=threshold, workspace=ws)
    torch.cuda.synchronize()
    if with_ws:
        return out, lse, ws
    return out, lse


def _lse_bound(inp, heads):
    """Per (b, i, h): scale 2^-8 max over visible t of sum_d |q_c,d K_t,d| (bf16 rounding of K), + 2e-3."""
    K, _ = oracle.decompress_kv(inp.pool, inp.block_table, inp.seqlens, inp.w_uk[heads], inp.w_uv[heads])
    qc = np.abs(oracle.bf16_bits_to_f64(inp.q_c[:, :, heads]))
    out = np.zeros((inp.batch, inp.s_q, len(heads)))
    for b in range(inp.batch):
        L = int(inp.seqlens[b])
        for hi in range(len(heads)):
            m = qc[b, :, hi] @ np.abs(K[b, hi, :L]).T          # [s_q, L]
            for i in range(inp.s_q):
                n = L - inp.s_q + i + 1
                out[b, i, hi] = m[i, :n].max() if n > 0 else 0.0
    return inp.scale * 2.0 ** -8 * out + 2e-3


def _check(inp, out, lse, what, heads=HEADS):
    ref, ref_lse = oracle.decode_decompressed(inp.q_c, inp.q_r, inp.w_uk, inp.w_uv, inp.pool, inp.block_table,
                                              inp.seqlens, inp.s_q, inp.scale, heads=heads)
    got = oracle.bf16_bits_to_f64(host_bits(out))[:, :, heads]
    assert_close(got, ref, what)
    gl = lse.cpu().numpy()[:, :, heads]
    none = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(gl), none), f"{what}: queries without visible tokens differ"
    assert np.all(got[none] == 0)
    bound = _lse_bound(inp, heads)
    assert np.all(np.abs(gl[~none] - ref_lse[~none]) <= bound[~none]), f"{what}: lse"


def test_expanded_keys_and_values_match_the_oracle():
    inp = make_custom(90, 2, 256, [300, 256], extra_blocks=1)
    print("decompress: B=2 L=[300,256]", flush=True)
    _, _, ws = _run(inp, mode=2, with_ws=True)
    max_len = inp.max_blocks * 64
    n = inp.batch * max_len * 128 * 128
    kb = host_bits(ws[:2 * n].view(torch.int16)).reshape(inp.batch, 128, max_len, 128).transpose(0, 2, 1, 3)
    off = (2 * n + 255) // 256 * 256
    vb = host_bits(ws[off:off + 2 * n].view(torch.int16)).reshape(inp.batch, 128, max_len, 128).transpose(0, 2, 1, 3)
    K, V = oracle.decompress_kv(inp.pool, inp.block_table, inp.seqlens, inp.w_uk, inp.w_uv, max_len=max_len)
    wk = np.abs(oracle.bf16_bits_to_f64(inp.w_uk))
    wv = np.abs(oracle.bf16_bits_to_f64(inp.w_uv))
    for b in range(inp.batch):
        L = int(inp.seqlens[b])
        c = np.abs(oracle.bf16_bits_to_f64(oracle.gather_rows(inp.pool, inp.block_table, b, L))[:, :512])
        ek = (512 / 16 + 64) * U * np.einsum("tc,hdc->thd", c, wk)
        ev = (512 / 16 + 64) * U * np.einsum("tc,hce->the", c, wv)
        assert_bf16_match(kb[b, :L], K[b, :, :L].transpose(1, 0, 2), ek, f"K of sequence {b}")
        assert_bf16_match(vb[b, :L], V[b, :, :L].transpose(1, 0, 2), ev, f"V of sequence {b}")



def test_expansion_over_many_ragged_sequences_leaves_other_rows_alone():
    """Seven sequences from 1 to 200 tokens (partial, exact and single-row pages; the
    pages of all sequences are dealt out to the expansion's waves in turn), NaN in every
    pool row no sequence may read, unused table entries out of the pool's range, and a
    workspace pre-filled with a marker: every row t < L_b of K and V matches the oracle,
    every other row keeps the marker."""
    lens = [1, 63, 64, 65, 129, 200, 7]
    inp = poison_unused(make_custom(97, len(lens), 1, lens, extra_blocks=1))
    print(f"decompress: B={inp.batch} L={lens}", flush=True)
    params = mla.make_prefill_params(inp.batch, inp.s_q, inp.max_blocks, inp.num_pages, inp.scale, 2, 0)
    ws = torch.full((mla.prefill_workspace_size(params),), 0x5A, dtype=torch.uint8, device="cuda")
    bt = inp.block_table.copy()
    bt[bt < 0] = 10 ** 6              # unused table entries point outside the pool: never read
    mla.prefill(dev_bf16(inp.q_c), dev_bf16(inp.q_r), dev_bf16(inp.w_uk), dev_bf16(inp.w_uv), dev_bf16(inp.pool),
                dev_i32(bt), dev_i32(inp.seqlens), scale=inp.scale, mode=2, workspace=ws)
    torch.cuda.synchronize()
    max_len = inp.max_blocks * 64
    n = inp.batch * 128 * max_len * 128
    off = (2 * n + 255) // 256 * 256
    kb = host_bits(ws[:2 * n].view(torch.int16)).reshape(inp.batch, 128, max_len, 128)
    vb = host_bits(ws[off:off + 2 * n].view(torch.int16)).reshape(inp.batch, 128, max_len, 128)
    wk = np.abs(oracle.bf16_bits_to_f64(inp.w_uk))
    wv = np.abs(oracle.bf16_bits_to_f64(inp.w_uv))
    K, V = oracle.decompress_kv(inp.pool, inp.block_table, inp.seqlens, inp.w_uk, inp.w_uv, max_len=max_len)
    for b, L in enumerate(lens):
        c = np.abs(oracle.bf16_bits_to_f64(oracle.gather_rows(inp.pool, inp.block_table, b, L))[:, :512])
        ek = (512 / 16 + 64) * U * np.einsum("tc,hdc->htd", c, wk)
        ev = (512 / 16 + 64) * U * np.einsum("tc,hce->hte", c, wv)
        assert_bf16_match(kb[b, :, :L], K[b, :, :L], ek, f"K of sequence {b} (L={L})")
        assert_bf16_match(vb[b, :, :L], V[b, :, :L], ev, f"V of sequence {b} (L={L})")
        marker = np.uint16(0x5A5A)
        assert np.all(kb[b, :, L:] == marker), f"K rows past L={L} of sequence {b} were written"
        assert np.all(vb[b, :, L:] == marker), f"V rows past L={L} of sequence {b} were written"

CASES = [
    # (name, seed, batch, s_q, seqlens, mode)
    ("chunk-256-auto", 91, 2, 256, [256, 700], 0),
    ("chunk-300-ragged", 92, 3, 300, [300, 301, 1000], 0),
    ("whole-prompt-64-forced", 93, 1, 64, [64], 2),
    ("longer-than-cache-forced", 94, 2, 40, [20, 200], 2),
    ("one-query-tile-edge", 95, 2, 129, [129, 4000], 2),
    # a single query per sequence through the decompress branch, one sequence holding
    # just that token (it sees only itself: the output is its own V row)
    ("single-query-forced", 104, 2, 1, [1, 77], 2),
]


@pytest.mark.parametrize("name,seed,batch,s_q,seqlens,mode", CASES, ids=[c[0] for c in CASES])
def test_decompress_branch(name, seed, batch, s_q, seqlens, mode):
    inp = make_custom(seed, batch, s_q, seqlens, extra_blocks=1)
    print(f"prefill decompress {name}", flush=True)
    out, lse = _run(inp, mode=mode)
    _check(inp, out, lse, name)


@pytest.mark.parametrize("name,seed,batch,s_q,seqlens,mode", [
    ("chunk-100-auto", 96, 2, 100, [100, 500], 0),
    ("chunk-7-forced", 97, 3, 7, [7, 64, 1000], 1),
    ("chunk-255-auto", 98, 1, 255, [3000], 0),
    ("chunk-256-forced", 105, 2, 256, [256, 1500], 1),   # the largest s_q the absorbed decode takes
], ids=["chunk-100-auto", "chunk-7-forced", "chunk-255-auto", "chunk-256-forced"])
def test_absorbed_branch(name, seed, batch, s_q, seqlens, mode):
    inp = make_custom(seed, batch, s_q, seqlens, extra_blocks=1)
    print(f"prefill absorbed {name}", flush=True)
    out, lse = _run(inp, mode=mode)
    ref, ref_lse = oracle.decode_decompressed(inp.q_c, inp.q_r, inp.w_uk, inp.w_uv, inp.pool, inp.block_table,
                                              inp.seqlens, s_q, inp.scale, heads=HEADS)
    assert_close(oracle.bf16_bits_to_f64(host_bits(out))[:, :, HEADS], ref, name)


def test_decompress_branch_with_rising_scores():
    """Scores that rise along the keys (content queries 0, q_R = e_0, k_R[t][0] = t / 4).
    In the 4000-token sequence every query sees past 3700 keys, so a later score exceeds
    the largest score of the first 64 keys by more than 64 in log2 units and the
    attention must redo those query tiles against their true maxima; in the
    300-token sequence the scores stay within that headroom.  Both against the oracle."""
    lens = [4000, 300]
    inp = make_custom(103, 2, 300, lens, extra_blocks=1)
    inp.q_c[:] = 0
    inp.q_r[:] = 0
    inp.q_r[..., 0] = np.uint16(0x3F80)                       # 1.0
    inp.pool[:, :, 512:] = 0
    for b, L in enumerate(lens):
        t = np.arange(L)
        inp.pool[inp.block_table[b, t // 64], t % 64, 512] = oracle.f64_to_bf16_bits(t / 4.0)
    print("prefill decompress rising scores", flush=True)
    out, lse = _run(inp, mode=2)
    _check(inp, out, lse, "rising scores")


def test_both_branches_agree():
    inp = make_custom(99, 2, 200, [200, 900], extra_blocks=1)
    a, la = _run(inp, mode=1)
    d, ld = _run(inp, mode=2)
    ga = oracle.bf16_bits_to_f64(host_bits(a))
    gd = oracle.bf16_bits_to_f64(host_bits(d))
    assert np.max(np.abs(ga - gd)) <= 2 * (1e-2 * np.max(np.abs(gd)) + 2e-3)
    _check(inp, d, ld, "decompress at 200")


def test_decompress_is_bitwise_reproducible():
    inp = make_custom(100, 2, 256, [256, 333], extra_blocks=1)
    a, la = _run(inp, mode=2)
    b, lb = _run(inp, mode=2)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


@pytest.mark.parametrize("s_q,seqlens", [(5, [5, 100, 2000]), (64, [64, 1000])])
def test_decode_paged_with_many_queries(s_q, seqlens):
    """The absorbed decode with s_q > 2 (the absorbed branch of a short chunk) against the latent-space oracle."""
    inp = make_custom(101 + s_q, len(seqlens), s_q, seqlens, extra_blocks=1)
    qa = oracle.f64_to_bf16_bits(oracle.absorb_q(inp.q_c, inp.w_uk))
    ol, lse = mla.decode_paged(dev_bf16(qa), dev_bf16(inp.q_r), dev_bf16(inp.pool), dev_i32(inp.block_table),
                               dev_i32(inp.seqlens), scale=inp.scale)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, s_q, inp.scale)
    assert_close(oracle.bf16_bits_to_f64(host_bits(ol)), ref, f"out_latent s_q={s_q}")
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 2e-3


def test_full_size_prompt_sampled():
    """The benchmark's prefill launch: 8 sequences, a 4096-token prompt each (M = L = 4096),
    queries and keys generated on the device; a few (sequence, head, query) outputs
    checked against the oracle."""
    B, L = 8, 4096
    base = make_custom(102, B, 1, [L] * B)
    g = torch.Generator(device="cuda")
    g.manual_seed(103)
    q_c = torch.randn((B, L, 128, 128), device="cuda", generator=g).to(torch.bfloat16)
    q_r = torch.randn((B, L, 128, 64), device="cuda", generator=g).to(torch.bfloat16)
    print("prefill full size B=8 L=M=4096", flush=True)
    out, lse = mla.prefill(q_c, q_r, dev_bf16(base.w_uk), dev_bf16(base.w_uv), dev_bf16(base.pool),
                           dev_i32(base.block_table), dev_i32(base.seqlens), scale=base.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    b, heads, queries = 5, [3, 100], [0, 1, 63, 64, 2047, 4095]
    qc = host_bits(q_c[b:b + 1, :, heads].contiguous())
    qr = host_bits(q_r[b:b + 1, :, heads].contiguous())
    ref, ref_lse = oracle.decode_decompressed(qc, qr, base.w_uk[heads], base.w_uv[heads], base.pool,
                                              base.block_table[b:b + 1], base.seqlens[b:b + 1], L, base.scale,
                                              queries=queries)
    got = oracle.bf16_bits_to_f64(host_bits(out[b:b + 1][:, queries][:, :, heads].contiguous()))
    assert_close(got, ref, "sampled outputs")
    gl = lse[b:b + 1][:, queries][:, :, heads].cpu().numpy()
    # the derived bound of _lse_bound: bf16 rounding of the expanded keys moves each score by at most
    # scale * 2^-8 * sum_d |q_c,d K_t,d|, so lse by at most its maximum over the visible keys; + 2e-3
    K, _ = oracle.decompress_kv(base.pool, base.block_table[b:b + 1], base.seqlens[b:b + 1], base.w_uk[heads],
                                base.w_uv[heads])
    qabs = np.abs(oracle.bf16_bits_to_f64(qc[0][queries]))            # [queries, heads, 128]
    bound = np.zeros((len(queries), len(heads)))
    for hi in range(len(heads)):
        m = qabs[:, hi] @ np.abs(K[0, hi, :L]).T                       # [queries, L]
        for qi, i in enumerate(queries):
            bound[qi, hi] = m[qi, :i + 1].max()                        # query i sees the first i + 1 keys
    bound = base.scale * 2.0 ** -8 * bound + 2e-3
    assert np.all(np.abs(gl[0] - ref_lse[0]) <= bound), "sampled lse beyond the derived bound"
