"""Pins the fp64 attention oracle to things other than itself: scalar brute
force, a textbook attention special case (torch SDPA in fp64), closed forms,
sequential-decode equivalence of the two-token verify step, invariants of the
page gather, and the log-sum-exp merge identity."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import make_custom, poison_unused


def _rand_case(seed, B, s_q, seqlens, H, d_hc, d_c, d_r, page, permute=True):
    """Small float64 case with its own page permutation."""
    rng = np.random.default_rng(seed)
    seqlens = np.asarray(seqlens)
    n_b = (seqlens + page - 1) // page
    P = int(n_b.sum())
    perm = rng.permutation(P) if permute else np.arange(P)
    bt = np.full((B, int(n_b.max()) + 1), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        bt[b, :n_b[b]] = perm[off:off + n_b[b]]
        off += n_b[b]
    return dict(
        q_c=rng.standard_normal((B, s_q, H, d_hc)), q_r=rng.standard_normal((B, s_q, H, d_r)),
        w_uk=rng.standard_normal((H, d_hc, d_c)) / math.sqrt(d_c), w_uv=rng.standard_normal((H, d_c, d_hc)) / math.sqrt(d_c),
        pool=rng.standard_normal((P, page, d_c + d_r)), block_table=bt, seqlens=seqlens, s_q=s_q,
        scale=1.0 / math.sqrt(d_hc + d_r))


def _brute(case):
    """Scalar loops over the definition: expand K, V per head, softmax, weighted sum."""
    q_c, q_r, w_uk, w_uv, pool, bt = (case[k] for k in ("q_c", "q_r", "w_uk", "w_uv", "pool", "block_table"))
    B, s_q, H, d_hc = q_c.shape
    d_c = w_uk.shape[2]
    d_r = q_r.shape[3]
    page = pool.shape[1]
    out = np.zeros((B, s_q, H, d_hc))
    lse = np.zeros((B, s_q, H))
    for b in range(B):
        L = int(case["seqlens"][b])
        for i in range(s_q):
            n = L - s_q + i + 1
            for h in range(H):
                scores, vals = [], []
                for t in range(n):
                    row = pool[bt[b][t // page]][t % page]
                    k = [sum(row[c] * w_uk[h][d][c] for c in range(d_c)) for d in range(d_hc)]
                    v = [sum(row[c] * w_uv[h][c][e] for c in range(d_c)) for e in range(d_hc)]
                    sc = sum(q_c[b][i][h][d] * k[d] for d in range(d_hc)) + sum(q_r[b][i][h][j] * row[d_c + j] for j in range(d_r))
                    scores.append(sc * case["scale"])
                    vals.append(v)
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                z = sum(ws)
                for e in range(d_hc):
                    out[b, i, h, e] = sum(ws[t] * vals[t][e] for t in range(n)) / z
                lse[b, i, h] = mx + math.log(z)
    return out, lse


def _decomp(case, **kw):
    return oracle.decode_decompressed(case["q_c"], case["q_r"], case["w_uk"], case["w_uv"], case["pool"],
                                      case["block_table"], case["seqlens"], case["s_q"], case["scale"], **kw)


def _absorbed(case):
    qa = oracle.absorb_q(case["q_c"], case["w_uk"])
    ol, lse = oracle.decode_absorbed(qa, case["q_r"], case["pool"], case["block_table"], case["seqlens"],
                                     case["s_q"], case["scale"])
    return ol, lse


TINY = dict(H=2, d_hc=4, d_c=8, d_r=2, page=4)


@pytest.mark.parametrize("s_q,seqlens", [(1, [1, 5, 7]), (2, [2, 4, 7]), (1, [4, 8, 3]), (5, [5, 9, 12])])
def test_decompressed_matches_brute_force(s_q, seqlens):
    case = _rand_case(3, 3, s_q, seqlens, **TINY)
    out, lse = _decomp(case)
    bout, blse = _brute(case)
    assert np.max(np.abs(out - bout)) <= 1e-12 * np.max(np.abs(bout))
    assert np.max(np.abs(lse - blse)) <= 1e-12 * np.max(np.abs(blse))


@pytest.mark.parametrize("s_q,seqlens", [(1, [1, 5, 7]), (2, [2, 6, 7]), (6, [6, 9, 20])])
def test_absorbed_equals_decompressed_tiny(s_q, seqlens):
    case = _rand_case(4, 3, s_q, seqlens, **TINY)
    out, lse = _decomp(case)
    ol, lse2 = _absorbed(case)
    out2 = oracle.up_proj(ol, case["w_uv"])
    assert np.max(np.abs(out - out2)) <= 1e-12 * np.max(np.abs(out))
    assert np.max(np.abs(lse - lse2)) <= 1e-12 * np.max(np.abs(lse))


def test_absorbed_equals_decompressed_real_dims():
    # Batch 1, 2048 tokens, real head dims, first 8 of 128 heads -- the bf16 generator's values.
    inp = make_custom(42, 1, 1, [2048], permute=False)
    case = dict(q_c=inp.q_c, q_r=inp.q_r, w_uk=inp.w_uk, w_uv=inp.w_uv, pool=inp.pool, block_table=inp.block_table,
                seqlens=inp.seqlens, s_q=1, scale=inp.scale)
    heads = list(range(8))
    out, lse = _decomp(case, heads=heads)
    qa = oracle.absorb_q(inp.q_c, inp.w_uk)
    ol, lse2 = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, 1, inp.scale)
    out2 = oracle.up_proj(ol, inp.w_uv)[:, :, heads]
    assert np.max(np.abs(out - out2)) <= 1e-12 * np.max(np.abs(out))
    assert np.max(np.abs(lse - lse2[:, :, heads])) <= 1e-12 * np.max(np.abs(lse))


def test_absorb_and_up_proj_match_loops():
    rng = np.random.default_rng(5)
    H, d_hc, d_c = 3, 4, 6
    q = rng.standard_normal((2, H, d_hc))
    w = rng.standard_normal((H, d_hc, d_c))
    qa = oracle.absorb_q(q, w)
    for t in range(2):
        for h in range(H):
            for c in range(d_c):
                assert abs(qa[t, h, c] - sum(q[t, h, d] * w[h, d, c] for d in range(d_hc))) < 1e-12
    ol = rng.standard_normal((2, H, d_c))
    wv = rng.standard_normal((H, d_c, d_hc))
    out = oracle.up_proj(ol, wv)
    for t in range(2):
        for h in range(H):
            for e in range(d_hc):
                assert abs(out[t, h, e] - sum(ol[t, h, c] * wv[h, c, e] for c in range(d_c))) < 1e-12


def test_selection_weights_reduce_to_sdpa():
    """With W_UK[h] and W_UV[h] picking latent columns (a different choice per
    head), MLA is plain scaled-dot-product attention with q = [q_c || q_R],
    k = [c[:, sigma_h] || k_R], v = c[:, tau_h] and head dim 192."""
    H, d_hc, d_c, d_r, page = 6, 128, 512, 64, 64
    case = _rand_case(6, 2, 1, [300, 129], H, d_hc, d_c, d_r, page)
    rng = np.random.default_rng(7)
    sig = [rng.permutation(d_c)[:d_hc] for _ in range(H)]
    tau = [rng.permutation(d_c)[:d_hc] for _ in range(H)]
    w_uk = np.zeros((H, d_hc, d_c))
    w_uv = np.zeros((H, d_c, d_hc))
    for h in range(H):
        w_uk[h, np.arange(d_hc), sig[h]] = 1.0
        w_uv[h, tau[h], np.arange(d_hc)] = 1.0
    case.update(w_uk=w_uk, w_uv=w_uv)
    out, _ = _decomp(case)
    ol, _ = _absorbed(case)
    out_abs = oracle.up_proj(ol, w_uv)
    for b in range(2):
        L = int(case["seqlens"][b])
        rows = oracle.gather_rows(case["pool"], case["block_table"], b, L)
        c, r = torch.from_numpy(rows[:, :d_c]), torch.from_numpy(rows[:, d_c:])
        for h in range(H):
            q = torch.cat([torch.from_numpy(case["q_c"][b, 0, h]), torch.from_numpy(case["q_r"][b, 0, h])])
            k = torch.cat([c[:, sig[h]], r], dim=1)
            v = c[:, tau[h]]
            ref = F.scaled_dot_product_attention(q[None, None, None], k[None, None], v[None, None])[0, 0, 0].numpy()
            assert np.max(np.abs(out[b, 0, h] - ref)) < 1e-12
            assert np.max(np.abs(out_abs[b, 0, h] - ref)) < 1e-12


def test_two_token_verify_equals_two_decode_steps():
    """Query i of an s_q=2 step (length L, both new tokens included) equals an
    ordinary one-token decode over the first L-1+i tokens."""
    H, d_hc, d_c, d_r, page = 4, 16, 32, 8, 8
    case = _rand_case(8, 2, 2, [17, 9], H, d_hc, d_c, d_r, page)
    out2, lse2 = _decomp(case)
    ol2, llse2 = _absorbed(case)
    for i in range(2):
        c1 = dict(case)
        c1.update(s_q=1, q_c=case["q_c"][:, i:i + 1], q_r=case["q_r"][:, i:i + 1],
                  seqlens=case["seqlens"] - 1 + i)
        o1, l1 = _decomp(c1)
        assert np.array_equal(o1[:, 0], out2[:, i]) and np.array_equal(l1[:, 0], lse2[:, i])
        a1, al1 = _absorbed(c1)
        assert np.array_equal(a1[:, 0], ol2[:, i]) and np.array_equal(al1[:, 0], llse2[:, i])


@pytest.mark.parametrize("s_q", [3, 8])
def test_prefill_chunk_equals_sequential_decode_steps(s_q):
    """A chunk of s_q new tokens (prefill) equals s_q one-token decode steps: query i sees
    the first L - s_q + i + 1 tokens."""
    H, d_hc, d_c, d_r, page = 4, 16, 32, 8, 8
    case = _rand_case(18, 2, s_q, [s_q + 9, s_q], H, d_hc, d_c, d_r, page)
    out, lse = _decomp(case)
    for i in range(s_q):
        c1 = dict(case)
        c1.update(s_q=1, q_c=case["q_c"][:, i:i + 1], q_r=case["q_r"][:, i:i + 1],
                  seqlens=case["seqlens"] - s_q + 1 + i)
        o1, l1 = _decomp(c1)
        # equal up to fp64 rounding (the expanded K and V are products over different row counts)
        assert np.max(np.abs(o1[:, 0] - out[:, i])) <= 1e-12 * np.max(np.abs(out))
        assert np.max(np.abs(l1[:, 0] - lse[:, i])) <= 1e-12 * np.max(np.abs(lse))


def test_whole_prompt_is_causal_sdpa():
    """With every cached token new (s_q = L), the decompress path is textbook causal
    attention: torch SDPA (fp64, CPU, is_causal) on q = [q_c | q_R], k = [c W_UK^T | k_R],
    v = c W_UV, per head."""
    H, d_hc, d_c, d_r, page, L = 3, 8, 16, 4, 4, 11
    case = _rand_case(19, 1, L, [L], H, d_hc, d_c, d_r, page, permute=True)
    out, lse = _decomp(case)
    rows = oracle.gather_rows(case["pool"], case["block_table"], 0, L)
    c, r = torch.from_numpy(rows[:, :d_c]), torch.from_numpy(rows[:, d_c:])
    for h in range(H):
        k = torch.cat([c @ torch.from_numpy(case["w_uk"][h]).T, r], dim=1)
        v = c @ torch.from_numpy(case["w_uv"][h])
        q = torch.cat([torch.from_numpy(case["q_c"][0, :, h]), torch.from_numpy(case["q_r"][0, :, h])], dim=1)
        ref = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True, scale=case["scale"])[0]
        assert np.max(np.abs(out[0, :, h] - ref.numpy())) <= 1e-12 * float(ref.abs().max())


def test_softmax_rows_sum_to_one():
    case = _rand_case(9, 1, 1, [200], 8, 16, 64, 8, 16)
    qa = oracle.absorb_q(case["q_c"], case["w_uk"])
    rows = oracle.gather_rows(case["pool"], case["block_table"], 0, 200)
    p, lse = oracle.attention_probs(qa[0, 0], case["q_r"][0, 0], rows, case["scale"])
    assert p.shape == (8, 200) and np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12


def test_single_token_is_that_row():
    case = _rand_case(10, 2, 1, [1, 1], 4, 8, 16, 4, 8)
    ol, lse = _absorbed(case)
    qa = oracle.absorb_q(case["q_c"], case["w_uk"])
    for b in range(2):
        row = oracle.gather_rows(case["pool"], case["block_table"], b, 1)[0]
        assert np.array_equal(ol[b, 0], np.broadcast_to(row[:16], (4, 16)))
        s = (qa[b, 0] @ row[:16] + case["q_r"][b, 0] @ row[16:]) * case["scale"]
        assert np.max(np.abs(lse[b, 0] - s)) <= 1e-14 * np.max(np.abs(s))


def test_zero_query_gives_mean_and_identical_rows_give_the_row():
    case = _rand_case(11, 1, 1, [37], 3, 8, 16, 4, 8)
    case["q_c"][:] = 0
    case["q_r"][:] = 0
    ol, lse = _absorbed(case)
    rows = oracle.gather_rows(case["pool"], case["block_table"], 0, 37)
    assert np.max(np.abs(ol[0, 0] - rows[:, :16].mean(axis=0))) < 1e-14
    assert np.max(np.abs(lse - math.log(37))) < 1e-14
    case = _rand_case(12, 1, 1, [37], 3, 8, 16, 4, 8)
    case["pool"][:] = case["pool"][0, 0]
    ol, _ = _absorbed(case)
    assert np.max(np.abs(ol[0, 0] - case["pool"][0, 0, :16])) < 1e-14


@pytest.mark.parametrize("pos", [0, 63, 64, 199])
def test_needle_dominates(pos):
    """A token whose RoPE key aligns with every head's q_R (score 40+ above the
    rest, content term zero) takes all the weight: out_latent is its latent."""
    H, d_c, d_r = 4, 32, 8
    case = _rand_case(13, 1, 1, [200], H, 8, d_c, d_r, 64)
    case["q_c"][:] = 0
    v = np.ones(d_r)
    case["q_r"][0, 0, :] = v
    rows_phys = case["pool"]
    rows_phys[..., d_c:] = 0
    page = case["block_table"][0, pos // 64]
    rows_phys[page, pos % 64, d_c:] = v * (45.0 / (d_r * case["scale"]))
    ol, _ = _absorbed(case)
    out, _ = _decomp(case)
    c = rows_phys[page, pos % 64, :d_c]
    assert np.max(np.abs(ol[0, 0] - c)) < 1e-15 * 200 * 10
    assert np.max(np.abs(out[0, 0] - oracle.up_proj(np.broadcast_to(c, (H, d_c))[None], case["w_uv"])[0])) < 1e-12


def test_page_placement_does_not_matter():
    case = _rand_case(14, 3, 2, [70, 130, 5], 4, 8, 16, 4, 16, permute=False)
    ol, lse = _absorbed(case)
    out, lse_d = _decomp(case)
    rng = np.random.default_rng(15)
    P = case["pool"].shape[0]
    perm = rng.permutation(P)                      # physical page p moves to slot perm[p]
    pool2 = np.empty_like(case["pool"])
    pool2[perm] = case["pool"]
    bt2 = np.where(case["block_table"] >= 0, perm[np.maximum(case["block_table"], 0)], -1)
    c2 = dict(case, pool=pool2, block_table=bt2)
    ol2, lse2 = _absorbed(c2)
    out2, lse_d2 = _decomp(c2)
    assert np.array_equal(ol, ol2) and np.array_equal(lse, lse2)
    assert np.array_equal(out, out2) and np.array_equal(lse_d, lse_d2)


def test_gather_matches_loops_and_skips_unused_slots():
    inp = make_custom(16, 3, 1, [65, 1, 130], permute=True, extra_blocks=2)
    poison_unused(inp)
    for b in range(3):
        L = int(inp.seqlens[b])
        rows = oracle.gather_rows(inp.pool, inp.block_table, b, L)
        for t in range(L):
            assert np.array_equal(rows[t], inp.pool[inp.block_table[b][t // 64], t % 64])
    qa = oracle.absorb_q(inp.q_c, inp.w_uk)
    ol, lse = oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, 1, inp.scale)
    assert np.all(np.isfinite(ol)) and np.all(np.isfinite(lse))


def test_generator_poison_marks_only_unreadable_rows():
    inp = make_custom(17, 2, 1, [65, 3], permute=True)
    poison_unused(inp)
    nan_rows = np.isnan(oracle.bf16_bits_to_f64(inp.pool[..., 0]))
    # 65 tokens -> 2 pages (63 unused rows), 3 tokens -> 1 page (61 unused rows)
    assert nan_rows.sum() == 63 + 61


@pytest.mark.parametrize("bounds", [[0, 200], [0, 64, 200], [0, 1, 2, 128, 199, 200], [0, 100, 101, 200]])
def test_split_and_merge_equals_whole(bounds):
    case = _rand_case(18, 1, 1, [200], 5, 8, 16, 4, 64)
    qa = oracle.absorb_q(case["q_c"], case["w_uk"])[0, 0]
    rows = oracle.gather_rows(case["pool"], case["block_table"], 0, 200)
    frags = oracle.split_decode_absorbed(qa, case["q_r"][0, 0], rows, bounds, case["scale"])
    out, lse = oracle.combine_fragments([f[0] for f in frags], [f[1] for f in frags])
    p, lse_w = oracle.attention_probs(qa, case["q_r"][0, 0], rows, case["scale"])
    whole = p @ rows[:, :16]
    assert np.max(np.abs(out - whole)) <= 1e-13 * np.max(np.abs(whole))
    assert np.max(np.abs(lse - lse_w)) <= 1e-13 * np.max(np.abs(lse_w))
    if len(frags) == 1:
        assert np.array_equal(out, frags[0][0]) and np.array_equal(lse, frags[0][1])


def test_queries_that_see_nothing_get_zero_and_minus_infinity():
    """L < s_q: the first s_q - L queries of the chunk see no token (the library's contract)."""
    H, d_hc, d_c, d_r, page = 2, 4, 8, 2, 4
    case = _rand_case(20, 2, 5, [3, 6], H, d_hc, d_c, d_r, page)
    out, lse = _decomp(case)
    ol, lse2 = _absorbed(case)
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    assert np.all(ol[0, :2] == 0) and np.all(np.isneginf(lse2[0, :2]))
    assert np.all(np.isfinite(lse[0, 2:])) and np.all(np.isfinite(lse[1]))
    # the rest is unaffected: query 2 of sequence 0 sees exactly token 0
    one = dict(case)
    one.update(s_q=1, q_c=case["q_c"][:, 2:3], q_r=case["q_r"][:, 2:3], seqlens=np.array([1, 4]))
    o1, _ = _decomp(one)
    assert np.max(np.abs(o1[0, 0] - out[0, 2])) <= 1e-12 * np.max(np.abs(out[0, 2]))
    sel, _ = oracle.decode_decompressed(case["q_c"], case["q_r"], case["w_uk"], case["w_uv"], case["pool"],
                                        case["block_table"], case["seqlens"], 5, case["scale"], queries=[4, 1])
    assert np.array_equal(sel[:, 0], out[:, 4]) and np.array_equal(sel[:, 1], out[:, 1])
