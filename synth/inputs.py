"""Seeded input generator for absorbed MLA decode over a paged latent cache.

Shapes follow the kernel description on "撕开 DeepSeek MLA 源码" (sheratonhq.com,
section 3, the ``mla_config.h`` constants and the ``mla_plugin`` JSON): 128
heads, content head dim 128, latent 512, decoupled RoPE key 64, pages of 64
tokens, bf16 cache.  One cached row is ``c_KV[512] || k_R[64]``.

Recipe (all configurations), in draw order from ``numpy.random.default_rng(seed)``:

1. sequence lengths (only when drawn: ``integers(lo, hi + 1, B)``),
2. the physical page permutation (only when permuted),
3. ``q_c [B, s_q, H, 128]``, ``q_R [B, s_q, H, 64]``,
   ``W_UK [H, 128, 512]``, ``W_UV [H, 512, 128]``, the pool
   ``[num_pages, 64, 576]`` -- each ``standard_normal`` float32; the two weights
   are multiplied by ``float32(1/sqrt(512))`` so scores have unit scale,
4. every float32 value is rounded to bf16 with round-to-nearest-even.

The pool holds exactly ``sum_b ceil(L_b / 64)`` pages; sequence ``b`` owns the
logical pages ``offset_b .. offset_b + n_b - 1`` and its block table row is
``perm[offset_b + j]``.  Unused block-table entries are ``-1``.  Rows past
``L_b`` in a sequence's last page are ordinary random values unless the
caller poisons them.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

NUM_HEADS = 128
D_HC = 128
D_C = 512
D_R = 64
PAGE = 64
ROW = D_C + D_R

# Workloads: single-layer decode at batch 1 / 16 / 64, a 60-layer resident
# long-context cache, and a two-token speculative-verify step.
CONFIGS = {
    "c1": dict(batch=1, s_q=1, seqlen=2048, permute=False, seed=42, layers=1),
    "c2": dict(batch=16, s_q=1, seqlen=4096, permute=True, seed=43, layers=1),
    "c3": dict(batch=64, s_q=1, seqlen=(1024, 32768), permute=True, seed=44, layers=1),
    "c3max": dict(batch=64, s_q=1, seqlen=32768, permute=True, seed=47, layers=1),
    "c4": dict(batch=16, s_q=1, seqlen=65536, permute=True, seed=45, layers=60),
    "c5": dict(batch=4, s_q=2, seqlen=131072, permute=True, seed=46, layers=1),
}

_POOL_CHUNK_PAGES = 256


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Works on the raw IEEE bits: add 0x7FFF plus the lowest kept bit, then
    drop the low 16 bits.  NaNs are kept quiet NaNs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16), r)
    return r


def pages_per_seq(seqlens: np.ndarray, page: int = PAGE) -> np.ndarray:
    return (np.asarray(seqlens, dtype=np.int64) + page - 1) // page


@dataclasses.dataclass
class MlaInputs:
    """All tensors of one decode step, as host arrays (bf16 as uint16 bits)."""

    name: str
    seed: int
    batch: int
    s_q: int
    seqlens: np.ndarray          # int32 [B]
    block_table: np.ndarray      # int32 [B, max_blocks], -1 where unused
    q_c: np.ndarray              # uint16 [B, s_q, H, 128]
    q_r: np.ndarray              # uint16 [B, s_q, H, 64]
    w_uk: np.ndarray             # uint16 [H, 128, 512]
    w_uv: np.ndarray             # uint16 [H, 512, 128]
    pool: np.ndarray | None      # uint16 [num_pages, 64, 576] (None when generated elsewhere)
    num_pages: int
    scale: float = 1.0 / math.sqrt(D_HC + D_R)

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def cache_bytes(self) -> int:
        """Logical cache bytes read by one step: sum of L_b rows of 1152 B."""
        return int(np.asarray(self.seqlens, dtype=np.int64).sum()) * ROW * 2


def _draw_bf16(rng: np.random.Generator, shape, mul: float | None = None) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float32)
    if mul is not None:
        v *= np.float32(mul)
    return f32_to_bf16_bits(v)


def _draw_pool(rng: np.random.Generator, num_pages: int, page: int, row: int) -> np.ndarray:
    pool = np.empty((num_pages, page, row), dtype=np.uint16)
    for p0 in range(0, num_pages, _POOL_CHUNK_PAGES):
        p1 = min(num_pages, p0 + _POOL_CHUNK_PAGES)
        pool[p0:p1] = f32_to_bf16_bits(rng.standard_normal((p1 - p0, page, row), dtype=np.float32))
    return pool


def _build(name, seed, batch, s_q, seqlen, permute, *, num_heads=NUM_HEADS, d_hc=D_HC, d_c=D_C, d_r=D_R,
           page=PAGE, with_pool=True, extra_blocks=0) -> MlaInputs:
    rng = np.random.default_rng(seed)
    if isinstance(seqlen, tuple):
        lo, hi = seqlen
        seqlens = rng.integers(lo, hi + 1, batch).astype(np.int32)
    elif np.ndim(seqlen) == 1:
        seqlens = np.asarray(seqlen, dtype=np.int32)
        assert seqlens.shape == (batch,)
    else:
        seqlens = np.full(batch, int(seqlen), dtype=np.int32)
    n_b = pages_per_seq(seqlens, page)
    num_pages = int(n_b.sum())
    perm = rng.permutation(num_pages) if permute else np.arange(num_pages)
    max_blocks = int(n_b.max()) + extra_blocks if batch > 0 else 1
    bt = np.full((batch, max(max_blocks, 1)), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        bt[b, : n_b[b]] = perm[off: off + n_b[b]]
        off += int(n_b[b])
    wscale = 1.0 / math.sqrt(d_c)
    q_c = _draw_bf16(rng, (batch, s_q, num_heads, d_hc))
    q_r = _draw_bf16(rng, (batch, s_q, num_heads, d_r))
    w_uk = _draw_bf16(rng, (num_heads, d_hc, d_c), wscale)
    w_uv = _draw_bf16(rng, (num_heads, d_c, d_hc), wscale)
    pool = _draw_pool(rng, num_pages, page, d_c + d_r) if with_pool else None
    return MlaInputs(name=name, seed=seed, batch=batch, s_q=s_q, seqlens=seqlens, block_table=bt, q_c=q_c,
                     q_r=q_r, w_uk=w_uk, w_uv=w_uv, pool=pool, num_pages=num_pages,
                     scale=1.0 / math.sqrt(d_hc + d_r))


def make_inputs(name: str, *, with_pool: bool = True) -> MlaInputs:
    """Inputs of a named workload (see ``CONFIGS``).

    The 60-layer long-context pool is far too large for host memory; for it the
    pool is left to the caller (``with_pool`` is forced off) and only the
    table, lengths, queries and weights are drawn here.
    """
    cfg = CONFIGS[name]
    if cfg["layers"] > 1:
        with_pool = False
    return _build(name, cfg["seed"], cfg["batch"], cfg["s_q"], cfg["seqlen"], cfg["permute"], with_pool=with_pool)


def make_custom(seed: int, batch: int, s_q: int, seqlens, *, permute: bool = True, num_heads: int = NUM_HEADS,
                d_hc: int = D_HC, d_c: int = D_C, d_r: int = D_R, page: int = PAGE,
                extra_blocks: int = 0) -> MlaInputs:
    """Small ragged cases for parity tests (explicit per-sequence lengths)."""
    seqlens = np.asarray(seqlens, dtype=np.int32).reshape(batch)
    return _build(f"custom{seed}", seed, batch, s_q, seqlens, permute, num_heads=num_heads, d_hc=d_hc, d_c=d_c,
                  d_r=d_r, page=page, extra_blocks=extra_blocks)


def poison_unused(inp: MlaInputs, nan_bits: int = 0x7FC0) -> MlaInputs:
    """Fill every pool row that no sequence may read with a NaN pattern.

    Rows at or past ``L_b`` in a sequence's last page, and any page that no
    table entry covering ``[0, L_b)`` names, become NaN.  A correct decode
    never reads them, so its output stays finite.
    """
    assert inp.pool is not None
    used = np.zeros(inp.pool.shape[:2], dtype=bool)
    for b in range(inp.batch):
        L = int(inp.seqlens[b])
        t = np.arange(L)
        used[inp.block_table[b, t // PAGE], t % PAGE] = True
    inp.pool[~used] = np.uint16(nan_bits)
    return inp


D_MODEL = 7168   # hidden size d of DeepSeek ("撕开 DeepSeek MLA 源码", section 3, kHiddenDim)


def make_append_inputs(seed: int, batch: int, s_q: int, d_model: int = D_MODEL, row: int = ROW):
    """Hidden states of the new tokens and the joint down-projection weight.

    Draw order from ``numpy.random.default_rng(seed)``: ``x [B, s_q, d]`` then
    ``W_A [d, row]``, each ``standard_normal`` float32, the weight times
    ``float32(1/sqrt(d))`` so the projected values have unit scale, then
    rounded to bf16 bits (nearest, ties to even).
    """
    rng = np.random.default_rng(seed)
    x = _draw_bf16(rng, (batch, s_q, d_model))
    w_a = _draw_bf16(rng, (d_model, row), 1.0 / math.sqrt(d_model))
    return x, w_a
