"""fp64 oracle for the decompress step of MLA prefill: the per-head keys and
values expanded from the cached latent.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU baseline, never by the library path.

Source: K = c . W_UK and V = c . W_UV, expanding each cached latent c into the
per-head keys and values ("DeepSeek的推理为什么比别人便宜一个数量级",
leslieaibin.github.io, section "MLA", second step); this is the "decompress"
branch that "撕开 DeepSeek MLA 源码" (sheratonhq.com, section 3 and the
section 6 measurement) takes for prefill chunks of at least
``kPrefillThresh`` = 256 query rows, while shorter ones use matrix absorption.
W_UK is laid out [H, d_hc, d_c] (sheratonhq.com section 4, ``w_uk``), so the
key of head h is K[t, d] = sum_c c[t, c] W_UK[h, d, c]; W_UV is [H, d_c, d_hc]
(the reading the decode oracle uses), V[t, e] = sum_c c[t, c] W_UV[h, c, e].
The attention that follows is ``decode_decompressed`` of the decode oracle with
s_q = the chunk length (query i of the chunk sees the first L - s_q + i + 1
tokens).  Exact fp64 on the bf16 inputs.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import bf16_bits_to_f64, gather_rows


def _as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64, copy=False)


def decompress_kv(pool, block_table, seqlens, w_uk, w_uv, max_len: int | None = None, d_c: int = 512):
    """Expanded keys and values of every cached token, fp64.

    Returns K, V of shape [B, H, max_len, d_hc] (max_len defaults to max seqlens);
    entries at t >= seqlens[b] are zero.
    """
    w_uk = _as_f64(w_uk)
    w_uv = _as_f64(w_uv)
    L = np.asarray(seqlens, dtype=np.int64)
    B, H, d_hc = L.shape[0], w_uk.shape[0], w_uk.shape[1]
    T = int(L.max()) if max_len is None else int(max_len)
    K = np.zeros((B, H, T, d_hc))
    V = np.zeros((B, H, T, w_uv.shape[2]))
    for b in range(B):
        n = int(L[b])
        c = _as_f64(gather_rows(pool, block_table, b, n))[:, :d_c]
        K[b, :, :n] = np.einsum("tc,hdc->htd", c, w_uk)
        V[b, :, :n] = np.einsum("tc,hce->hte", c, w_uv)
    return K, V
