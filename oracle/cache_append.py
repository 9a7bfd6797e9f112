"""fp64 oracle for the cache-append step that precedes each MLA decode step:
latent down-projection, the decoupled RoPE key, and the write of the new row
into the paged cache; plus the matching rotation of the RoPE query.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU baseline, never by the library path.

What is computed (sources are the pages' own sections):

* Down-projection.  The hidden state x of a new token is compressed to the
  latent c = x . W_DKV, d -> d_c, with d = 7168 and d_c = 512 for DeepSeek
  ("DeepSeek的推理为什么比别人便宜一个数量级", leslieaibin.github.io, section "MLA",
  first step; "撕开 DeepSeek MLA 源码", sheratonhq.com, section 3, the
  ``mla_config.h`` constants ``kHiddenDim`` and ``kLatentKV``).
* What is cached.  Only c and a 64-value position branch k_R shared by all
  heads are stored, 576 values per token (sheratonhq.com section 1); after each
  decode step the new token's row is appended to the cache (leslieaibin.github.io,
  the decode-loop step of the closing summary).
* RoPE precision.  The rotary tables are precomputed in fp32 and applied with
  fp32 multiply-add; fp16 rotary tables cause a phase error
  (sheratonhq.com section 4, the verification paragraph; ``rope_compute_dtype``
  fp32 in the section 3 plugin JSON).
* Paging.  Token t of sequence b lives in row ``t mod 64`` of page
  ``block_table[b][t div 64]`` (sheratonhq.com section 3, ``page_size`` 64).

Readings where the pages are silent (each listed with its reason in the
design notes):

* k_R is the RoPE rotation of x . W_KR, W_KR of shape [d, 64], taken from the
  same hidden state as c (the decoupled-key construction of DeepSeek-V2, which
  the bjbfmj.com page names as the origin of this cache layout).  The two
  weights arrive as one matrix W_A = [W_DKV | W_KR] of shape [d, 576], so
  ``row = x . W_A`` and the last 64 values are rotated.
* No normalisation is applied to c (the pages define c = x . W_DKV only).
* The rotation acts on interleaved pairs (2i, 2i + 1), i = 0..31, by the angle
  p * theta_i with theta_i = base ** (-2 i / 64), base 10000.  A table row p
  holds [cos(p theta_0) .. cos(p theta_31) | sin(p theta_0) .. sin(p theta_31)];
  the angles and their cosines and sines are evaluated in fp64 and each entry
  is rounded once to fp32 (an fp32 angle p * theta would itself carry the phase
  error the pages warn about at long positions).
* New token i of sequence b (s_q new tokens) has position p = seqlens[b] - s_q + i,
  the same index the decode step uses for it, and is written to that position's
  slot.  A token whose slot or table row does not exist (p < 0, p >= max_pos,
  p beyond the block-table row, or a page id outside the pool) is not written.

Arithmetic on the bf16 inputs is exact fp64; the table is used at its fp32
values.  Rounding to bf16 happens only where a caller asks for cache bits.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import bf16_bits_to_f64, f64_to_bf16_bits


def _as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64, copy=False)


# --------------------------------------------------------------------------- RoPE


def rope_angles(max_pos: int, d_r: int = 64, base: float = 10000.0) -> np.ndarray:
    """Angles p * theta_i, theta_i = base ** (-2 i / d_r), as fp64 [max_pos, d_r / 2]."""
    i = np.arange(d_r // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d_r)
    p = np.arange(int(max_pos), dtype=np.float64)
    return p[:, None] * theta[None, :]


def rope_table(max_pos: int, d_r: int = 64, base: float = 10000.0, dtype=np.float32) -> np.ndarray:
    """Rotary table [max_pos, d_r]: cosines of the angles, then their sines.

    Evaluated in fp64 and rounded once to ``dtype`` (fp32 by default, the
    precision the pages prescribe for the precomputed table).
    """
    a = rope_angles(max_pos, d_r, base)
    return np.concatenate([np.cos(a), np.sin(a)], axis=1).astype(dtype)


def rope_rotate(v, table_rows) -> np.ndarray:
    """Rotate interleaved pairs of ``v [..., d_r]`` by table rows ``[..., d_r]``.

    Pair i, (v[2i], v[2i + 1]), turns by the angle whose cosine and sine are
    table_rows[i] and table_rows[d_r / 2 + i]:
        out[2i]     = v[2i] cos - v[2i + 1] sin
        out[2i + 1] = v[2i] sin + v[2i + 1] cos
    Exact fp64 on the given values.
    """
    v = _as_f64(v)
    t = np.asarray(table_rows, dtype=np.float64)
    half = v.shape[-1] // 2
    cos, sin = t[..., :half], t[..., half:]
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape, t.shape), dtype=np.float64)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


# --------------------------------------------------------------------------- append


def append_positions(seqlens, s_q: int) -> np.ndarray:
    """Position of new token i of sequence b: seqlens[b] - s_q + i, int64 [B, s_q]."""
    L = np.asarray(seqlens, dtype=np.int64)
    return L[:, None] - int(s_q) + np.arange(int(s_q), dtype=np.int64)[None, :]


def down_project(x, w_a) -> np.ndarray:
    """row = x . W_A over the hidden dimension, exact fp64; x [..., d], W_A [d, n]."""
    return np.matmul(_as_f64(x), _as_f64(w_a))


def append_rows(x, w_a, table, positions, d_c: int = 512) -> np.ndarray:
    """Exact new cache rows [..., d_c + d_r] for hidden states x [..., d].

    The first d_c values are the latent c = x . W_DKV; the last d_r are x . W_KR
    rotated to each token's position (``positions`` [...], rows of ``table``).
    Positions outside the table give NaN rows (such tokens are never written).
    """
    row = down_project(x, w_a)
    pos = np.asarray(positions, dtype=np.int64)
    tab = np.asarray(table, dtype=np.float64)
    ok = (pos >= 0) & (pos < tab.shape[0])
    rows_t = tab[np.where(ok, pos, 0)]
    rows_t[~ok] = np.nan
    out = row.copy()
    out[..., d_c:] = rope_rotate(row[..., d_c:], rows_t)
    return out


def slot_of(block_table, b: int, p: int, num_pages: int, page: int = 64):
    """(page id, row) of position p of sequence b, or None where that slot does not exist."""
    bt = np.asarray(block_table)
    if p < 0 or p // page >= bt.shape[1]:
        return None
    pg = int(bt[b, p // page])
    if pg < 0 or pg >= num_pages:
        return None
    return pg, p % page


def append_to_pool(pool_bits, rows_bits, block_table, seqlens, s_q: int, max_pos: int) -> np.ndarray:
    """Copy of the pool with new token i of sequence b written to its slot.

    ``rows_bits [B, s_q, row]`` are the bf16 rows; a token is skipped when its
    position is outside [0, max_pos) or its slot does not exist.
    """
    out = np.array(pool_bits, copy=True)
    num_pages, page = out.shape[0], out.shape[1]
    pos = append_positions(seqlens, s_q)
    for b in range(pos.shape[0]):
        for i in range(pos.shape[1]):
            p = int(pos[b, i])
            if p >= max_pos:
                continue
            s = slot_of(block_table, b, p, num_pages, page)
            if s is not None:
                out[s[0], s[1]] = rows_bits[b, i]
    return out


def append_kv(x_bits, w_a_bits, table, block_table, seqlens, pool_bits, s_q: int, d_c: int = 512):
    """The whole append step: returns (exact rows fp64 [B, s_q, row], new pool bits).

    The cached values are the rows rounded to bf16, nearest, ties to even.
    """
    pos = append_positions(seqlens, s_q)
    rows = append_rows(x_bits, w_a_bits, table, pos, d_c)
    ok = np.isfinite(rows).all(axis=-1, keepdims=True)
    bits = f64_to_bf16_bits(np.where(ok, rows, 0.0))
    return rows, append_to_pool(pool_bits, bits, block_table, seqlens, s_q, np.asarray(table).shape[0])


def rope_q(q_r, table, positions) -> np.ndarray:
    """RoPE query: q_r [B, s_q, H, d_r] rotated to the positions [B, s_q] (exact fp64).

    Every head of a token turns by the same angles, the ones its key uses.
    Tokens whose position is outside the table keep their values.
    """
    q = _as_f64(q_r)
    pos = np.asarray(positions, dtype=np.int64)
    tab = np.asarray(table, dtype=np.float64)
    ok = (pos >= 0) & (pos < tab.shape[0])
    rows_t = tab[np.where(ok, pos, 0)][:, :, None, :]
    out = rope_rotate(q, rows_t)
    out[~ok] = q[~ok]
    return out
