"""fp64 oracle for Multi-Head Latent Attention decode over a paged cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU baseline, never by the library path.

What is computed (sources are the pages' own sections):

* Cache row.  Each token stores a latent ``c`` of d_c = 512 values and a
  decoupled RoPE key ``k_R`` of d_R = 64 values, 576 bf16 in total
  ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 1).
* Paging.  Tokens are stored in fixed pages of 64 rows; token ``t`` of
  sequence ``b`` is row ``t mod 64`` of physical page ``block_table[b][t div 64]``
  (same page, section 3, ``page_size`` 64 in the plugin JSON; section 5 on the
  page-table base).
* Decompress path (the definition).  Per head h, keys and values are expanded
  from the latent: K = c . W_UK[h] and V = c . W_UV[h] ("DeepSeek的推理为什么比别
  人便宜一个数量级", leslieaibin.github.io, section "MLA", the up-projection
  equations; sheratonhq.com section 4, path A, which expands keys with
  ``w_uk[h, d_hc, d_c]`` contracted over d_c).  Scores add the content term
  q_c . K and the RoPE term q_R . k_R and multiply their sum by 1/sqrt(d_hc + d_R)
  (sheratonhq.com section 4).  Softmax over the visible tokens, then P . V.
* Absorbed path.  q_abs = q_c . W_UK[h] (contracted over d_hc, sheratonhq.com
  section 4, path B); scores q_abs . c + q_R . k_R; the same softmax; the output
  stays in latent space, out_latent = P . c, and is up-projected afterwards,
  out = out_latent . W_UV[h] (leslieaibin.github.io "MLA", V = c . W_UV, by
  associativity of the sum over tokens).

Readings where the pages are silent (each listed with its reason in the
design notes): W_UV is laid out [H, d_c, d_hc]; q_R and k_R arrive already
rotated; softmax is the standard max-subtracted one; with s_q > 1 query i of
a sequence of length L (which already includes the s_q new tokens) sees
tokens t <= L - s_q + i, and a query that sees no token (L < s_q) gets a zero
output and lse = -inf; ``lse`` is the natural log of the softmax
denominator of the scaled scores.  Nothing here rounds: all arithmetic is
fp64 on the exact values of the bf16 inputs.
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------- bf16


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits), nearest, ties to even.

    Done in value space rather than on bits: write |x| = m * 2**e with
    0.5 <= m < 1, scale so the 8 kept bits form an integer part, round that
    with ties to even, scale back.  The bf16 subnormal step 2**-133 bounds
    the quantum from below; results beyond the largest finite bf16 become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    finite = np.isfinite(flat)
    xf = flat[finite]
    _, e = np.frexp(xf)
    q_exp = np.maximum(e - 8, -133)          # exponent of one unit in the last kept place
    r = np.rint(np.ldexp(xf, -q_exp))        # rint: round half to even
    y = np.ldexp(r, q_exp)
    big = np.abs(y) > 3.3895313892515355e38  # largest finite bf16
    y = np.where(big, np.copysign(np.inf, y), y)
    bits32 = y.astype(np.float32).view(np.uint32)
    res[finite] = (bits32 >> np.uint32(16)).astype(np.uint16)
    nonfinite = flat[~finite]
    res[~finite] = (nonfinite.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    res[~finite & np.isnan(flat)] = np.uint16(0x7FC0)
    return out


# --------------------------------------------------------------------------- gather


def gather_rows(pool, block_table, b: int, n: int) -> np.ndarray:
    """Rows of tokens 0..n-1 of sequence b from the paged pool.

    Token t is row ``t mod P`` of page ``block_table[b, t div P]`` where P is the
    page size (``pool.shape[1]``).  Returns ``[n, row]`` with the pool's dtype.
    """
    pool = np.asarray(pool)
    page = pool.shape[1]
    t = np.arange(int(n))
    pages = np.asarray(block_table)[b, t // page]
    return pool[pages, t % page]


def _as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64, copy=False)


def _softmax_lse(s: np.ndarray):
    """Standard softmax along the last axis with max subtraction; also ln of the denominator."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def _visible(L: int, s_q: int, i: int) -> int:
    """Number of keys query i of a step with s_q new tokens may attend to."""
    return int(L) - s_q + i + 1


# --------------------------------------------------------------------------- decompress path (definition)


def decode_decompressed(q_c, q_r, w_uk, w_uv, pool, block_table, seqlens, s_q: int, scale: float,
                        batches=None, heads=None, queries=None):
    """Plain multi-head attention after expanding K and V from the cached latent.

    Shapes (H heads, d_hc content dim, d_c latent, d_R rope, P page):
    q_c [B, s_q, H, d_hc], q_r [B, s_q, H, d_R], w_uk [H, d_hc, d_c],
    w_uv [H, d_c, d_hc], pool [pages, P, d_c + d_R], block_table [B, max_blocks],
    seqlens [B].  Arrays may be bf16 bits (uint16) or floats.

    Returns ``out [nb, nq, nh, d_hc]`` and ``lse [nb, nq, nh]`` for the selected
    sequences, query indices (of the s_q new tokens) and heads (all by default).
    """
    q_c = _as_f64(q_c)
    q_r = _as_f64(q_r)
    w_uk = _as_f64(w_uk)
    w_uv = _as_f64(w_uv)
    d_c = w_uk.shape[2]
    batches = list(range(q_c.shape[0])) if batches is None else list(batches)
    heads = list(range(q_c.shape[2])) if heads is None else list(heads)
    queries = list(range(s_q)) if queries is None else list(queries)
    out = np.zeros((len(batches), len(queries), len(heads), w_uv.shape[2]))
    lse = np.zeros((len(batches), len(queries), len(heads)))
    for bi, b in enumerate(batches):
        L = int(seqlens[b])
        rows = _as_f64(gather_rows(pool, block_table, b, L))
        c, r = rows[:, :d_c], rows[:, d_c:]
        for hi, h in enumerate(heads):
            K = c @ w_uk[h].T          # K[t, d] = sum_c' c[t, c'] W_UK[h, d, c']
            V = c @ w_uv[h]            # V[t, e] = sum_c' c[t, c'] W_UV[h, c', e]
            for qi, i in enumerate(queries):
                n = _visible(L, s_q, i)
                if n <= 0:                 # no visible token: zero output, lse = -inf
                    out[bi, qi, hi] = 0.0
                    lse[bi, qi, hi] = -np.inf
                    continue
                s = (K[:n] @ q_c[b, i, h] + r[:n] @ q_r[b, i, h]) * scale
                p, lz = _softmax_lse(s)
                out[bi, qi, hi] = p @ V[:n]
                lse[bi, qi, hi] = lz
    return out, lse


# --------------------------------------------------------------------------- absorbed path


def absorb_q(q_c, w_uk) -> np.ndarray:
    """q_abs[..., h, c] = sum_d q_c[..., h, d] * W_UK[h, d, c]  (fp64, unrounded)."""
    q_c = _as_f64(q_c)
    w_uk = _as_f64(w_uk)
    lead = q_c.shape[:-2]
    H, d_hc = q_c.shape[-2:]
    q = q_c.reshape(-1, H, d_hc).transpose(1, 0, 2)        # [H, T, d_hc]
    qa = np.matmul(q, w_uk)                                  # [H, T, d_c]
    return qa.transpose(1, 0, 2).reshape(*lead, H, w_uk.shape[2])


def attention_probs(q_abs_row, q_r_row, rows, scale: float):
    """Softmax weights of one query over given cache rows: [H, n] and lse [H]."""
    q_abs_row = _as_f64(q_abs_row)
    q_r_row = _as_f64(q_r_row)
    rows = _as_f64(rows)
    d_c = q_abs_row.shape[-1]
    s = (q_abs_row @ rows[:, :d_c].T + q_r_row @ rows[:, d_c:].T) * scale   # [H, n]
    return _softmax_lse(s)


def decode_absorbed(q_abs, q_r, pool, block_table, seqlens, s_q: int, scale: float, batches=None):
    """Latent-space decode: out_latent[b, i, h, :] = sum_t p[t] * c[t].

    ``q_abs [B, s_q, H, d_c]`` (fp64 or bf16 bits), ``q_r [B, s_q, H, d_R]``.
    Returns ``out_latent [nb, s_q, H, d_c]`` and ``lse [nb, s_q, H]``.
    """
    q_abs = _as_f64(q_abs)
    q_r = _as_f64(q_r)
    d_c = q_abs.shape[-1]
    batches = list(range(q_abs.shape[0])) if batches is None else list(batches)
    H = q_abs.shape[2]
    out = np.zeros((len(batches), s_q, H, d_c))
    lse = np.zeros((len(batches), s_q, H))
    for bi, b in enumerate(batches):
        L = int(seqlens[b])
        rows = _as_f64(gather_rows(pool, block_table, b, L))
        for i in range(s_q):
            n = _visible(L, s_q, i)
            if n <= 0:                     # no visible token: zero output, lse = -inf
                lse[bi, i] = -np.inf
                continue
            p, lz = attention_probs(q_abs[b, i], q_r[b, i], rows[:n], scale)
            out[bi, i] = p @ rows[:n, :d_c]
            lse[bi, i] = lz
    return out, lse


def up_proj(out_latent, w_uv) -> np.ndarray:
    """out[..., h, e] = sum_c out_latent[..., h, c] * W_UV[h, c, e]."""
    ol = _as_f64(out_latent)
    w_uv = _as_f64(w_uv)
    lead = ol.shape[:-2]
    H, d_c = ol.shape[-2:]
    x = ol.reshape(-1, H, d_c).transpose(1, 0, 2)           # [H, T, d_c]
    y = np.matmul(x, w_uv)                                   # [H, T, d_hc]
    return y.transpose(1, 0, 2).reshape(*lead, H, w_uv.shape[2])


# --------------------------------------------------------------------------- split-KV and merge


def split_decode_absorbed(q_abs_row, q_r_row, rows, bounds, scale: float):
    """Per-fragment partial results of one query over consecutive token ranges.

    ``bounds`` = [t0, t1, ..., tk]; fragment j covers tokens [t_j, t_{j+1}).  Each
    fragment returns its own normalised output (softmax within the fragment)
    and the ln of its own denominator.
    """
    rows = _as_f64(rows)
    d_c = _as_f64(q_abs_row).shape[-1]
    frags = []
    for a, z in zip(bounds[:-1], bounds[1:]):
        p, lz = attention_probs(q_abs_row, q_r_row, rows[a:z], scale)
        frags.append((p @ rows[a:z, :d_c], lz))
    return frags


def combine_fragments(outs, lses):
    """Merge fragments by log-sum-exp.

    lse = ln sum_j exp(lse_j); out = sum_j exp(lse_j - lse) * out_j.  This is the
    whole-range softmax written as a weighted mean of per-range softmaxes.
    """
    lses = np.stack([np.asarray(v, dtype=np.float64) for v in lses])      # [k, ...]
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    tot = w.sum(axis=0)
    lse = m + np.log(tot)
    wn = w / tot
    out = sum(wn[j][..., None] * np.asarray(outs[j], dtype=np.float64) for j in range(len(outs)))
    return out, lse
