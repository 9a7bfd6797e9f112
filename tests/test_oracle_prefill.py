"""Pins the fp64 decompress oracle (per-head keys and values expanded from the
cached latent) to scalar brute force, one-hot latents, zero padding past each
length, and page-placement invariance."""

import numpy as np

import oracle
from synth import make_custom


def _case(seed, B, seqlens, H=3, d_hc=4, d_c=6, d_r=2, page=4):
    rng = np.random.default_rng(seed)
    seqlens = np.asarray(seqlens)
    n_b = (seqlens + page - 1) // page
    P = int(n_b.sum())
    perm = rng.permutation(P)
    bt = np.full((B, int(n_b.max()) + 1), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        bt[b, :n_b[b]] = perm[off:off + n_b[b]]
        off += n_b[b]
    return dict(pool=rng.standard_normal((P, page, d_c + d_r)), bt=bt, seqlens=seqlens,
                w_uk=rng.standard_normal((H, d_hc, d_c)), w_uv=rng.standard_normal((H, d_c, d_hc)), d_c=d_c)


def test_decompress_brute_force():
    c = _case(1, 2, [5, 3])
    K, V = oracle.decompress_kv(c["pool"], c["bt"], c["seqlens"], c["w_uk"], c["w_uv"], d_c=c["d_c"])
    H, d_hc, d_c = c["w_uk"].shape
    page = c["pool"].shape[1]
    for b in range(2):
        for t in range(int(c["seqlens"][b])):
            row = c["pool"][c["bt"][b, t // page], t % page]
            for h in range(H):
                for d in range(d_hc):
                    k = sum(row[x] * c["w_uk"][h, d, x] for x in range(d_c))
                    v = sum(row[x] * c["w_uv"][h, x, d] for x in range(d_c))
                    assert abs(K[b, h, t, d] - k) < 1e-12 and abs(V[b, h, t, d] - v) < 1e-12
    assert np.all(K[1, :, 3:] == 0) and np.all(V[1, :, 3:] == 0)
    assert K.shape == (2, H, 5, d_hc)


def test_one_hot_latent_selects_weight_columns():
    c = _case(2, 1, [4])
    pool = np.zeros_like(c["pool"])
    page = pool.shape[1]
    for t, x in enumerate([0, 3, 5, 2]):
        pool[c["bt"][0, t // page], t % page, x] = 1.0
        pool[c["bt"][0, t // page], t % page, c["d_c"]:] = 7.0       # the RoPE key takes no part
    K, V = oracle.decompress_kv(pool, c["bt"], c["seqlens"], c["w_uk"], c["w_uv"], d_c=c["d_c"])
    for t, x in enumerate([0, 3, 5, 2]):
        assert np.array_equal(K[0, :, t], c["w_uk"][:, :, x])
        assert np.array_equal(V[0, :, t], c["w_uv"][:, x, :])


def test_page_placement_and_max_len():
    inp = make_custom(3, 2, 1, [70, 129], permute=True)
    K1, V1 = oracle.decompress_kv(inp.pool, inp.block_table, inp.seqlens, inp.w_uk[:2], inp.w_uv[:2], max_len=192)
    perm = np.random.default_rng(4).permutation(inp.num_pages)
    pool2 = np.empty_like(inp.pool)
    pool2[perm] = inp.pool
    bt2 = np.where(inp.block_table >= 0, perm[np.maximum(inp.block_table, 0)], -1)
    K2, V2 = oracle.decompress_kv(pool2, bt2, inp.seqlens, inp.w_uk[:2], inp.w_uv[:2], max_len=192)
    assert K1.shape == (2, 2, 192, 128) and np.array_equal(K1, K2) and np.array_equal(V1, V2)
    assert np.all(K1[0, :, 70:] == 0)
