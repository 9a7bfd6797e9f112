"""Plants plausible mistakes in a scratch copy of the oracle (CPU only) and
checks that the oracle's pins reject every one of them."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (oracle module, pin file) -> {name: (anchor, replacement)}
ATTENTION = ("mla_oracle.py", "test_oracle_attention.py")
APPEND = ("cache_append.py", "test_oracle_append.py")
PREFILL = ("prefill.py", "test_oracle_prefill.py")
FP8 = ("fp8_cache.py", "test_oracle_fp8.py")

MUTATIONS = {
    "dropped RoPE term": ("s = (K[:n] @ q_c[b, i, h] + r[:n] @ q_r[b, i, h]) * scale",
                          "s = (K[:n] @ q_c[b, i, h]) * scale"),
    "wrong sign of RoPE term": ("s = (K[:n] @ q_c[b, i, h] + r[:n] @ q_r[b, i, h]) * scale",
                                "s = (K[:n] @ q_c[b, i, h] - r[:n] @ q_r[b, i, h]) * scale"),
    "head index ignored": ("K = c @ w_uk[h].T", "K = c @ w_uk[0].T"),
    "visible count off by one": ("return int(L) - s_q + i + 1", "return int(L) - s_q + i"),
    "row within page shifted": ("return pool[pages, t % page]", "return pool[pages, (t + 1) % page]"),
    "scale dropped (absorbed)": ("s = (q_abs_row @ rows[:, :d_c].T + q_r_row @ rows[:, d_c:].T) * scale",
                                 "s = (q_abs_row @ rows[:, :d_c].T + q_r_row @ rows[:, d_c:].T)"),
    "max missing from lse": ("return e / z, (m + np.log(z))[..., 0]", "return e / z, (np.log(z))[..., 0]"),
    "latent columns shifted": ("out[bi, i] = p @ rows[:n, :d_c]", "out[bi, i] = p @ rows[:n, 1:d_c + 1]"),
    "W_UV heads reversed": ("y = np.matmul(x, w_uv)", "y = np.matmul(x, w_uv[::-1])"),
    "W_UK heads reversed": ("qa = np.matmul(q, w_uk)", "qa = np.matmul(q, w_uk[::-1])"),
    "merge weights unnormalised": ("wn = w / tot", "wn = w"),
}
MUTATIONS = {name: (ATTENTION, old, new) for name, (old, new) in MUTATIONS.items()}
MUTATIONS.update({name: (APPEND, old, new) for name, (old, new) in {
    "rotation sign flipped": ("out[..., 0::2] = a * cos - b * sin", "out[..., 0::2] = a * cos + b * sin"),
    "cosine and sine swapped": ("cos, sin = t[..., :half], t[..., half:]", "sin, cos = t[..., :half], t[..., half:]"),
    "pairs taken as halves": ("a, b = v[..., 0::2], v[..., 1::2]", "a, b = v[..., :half], v[..., half:]"),
    "frequency exponent halved": ("theta = base ** (-2.0 * i / d_r)", "theta = base ** (-1.0 * i / d_r)"),
    "table halves in the wrong order": ("np.concatenate([np.cos(a), np.sin(a)], axis=1)",
                                        "np.concatenate([np.sin(a), np.cos(a)], axis=1)"),
    "angle from an fp32 product": ("return p[:, None] * theta[None, :]",
                                   "return (p[:, None].astype(np.float32) * theta[None, :].astype(np.float32)).astype(np.float64)"),
    "new-token position off by one": ("return L[:, None] - int(s_q) + np.arange", "return L[:, None] - int(s_q) + 1 + np.arange"),
    "RoPE applied to the latent": ("out[..., d_c:] = rope_rotate(row[..., d_c:], rows_t)",
                                   "out[..., :64] = rope_rotate(row[..., :64], rows_t)"),
    "appended row within page shifted": ("return pg, p % page", "return pg, (p + 1) % page"),
    "invalid page written": ("if pg < 0 or pg >= num_pages:", "if pg >= num_pages:"),
    "query turned the other way": ("out = rope_rotate(q, rows_t)",
                                   "out = rope_rotate(q, np.concatenate([rows_t[..., :32], -rows_t[..., 32:]], -1))"),
}.items()})
MUTATIONS.update({name: (PREFILL, old, new) for name, (old, new) in {
    "decompress V heads reversed": ('V[b, :, :n] = np.einsum("tc,hce->hte", c, w_uv)',
                                    'V[b, :, :n] = np.einsum("tc,hce->hte", c, w_uv[::-1])'),
    "decompress latent columns shifted": ("c = _as_f64(gather_rows(pool, block_table, b, n))[:, :d_c]",
                                          "c = _as_f64(gather_rows(pool, block_table, b, n))[:, 1:d_c + 1]"),
    "decompress key transposed": ('K[b, :, :n] = np.einsum("tc,hdc->htd", c, w_uk)',
                                  'K[b, :, :n] = np.einsum("tc,hdc->htd", c[::-1], w_uk)'),
}.items()})
MUTATIONS.update({name: (FP8, old, new) for name, (old, new) in {
    "E4M3 exponent bias 8": ("np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)"),
    "E4M3 subnormal step halved": ("np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)"),
    "E4M3 ties away from zero": ("((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))", "(d_hi == d_lo)"),
    "E4M3 sign dropped": ("code = np.where(np.signbit(x), code | 0x80, code)", "code = code"),
    "MX scale clips like floor(log2 amax) - 8": ("x = np.where(amax > E4M3_MAX * np.ldexp(1.0, x0), x0 + 1, x0)",
                                                 "x = x0"),
    "MX scale from the block mean": ("np.abs(blocks).max(axis=-1)", "np.abs(blocks).mean(axis=-1)"),
    "MX scale bias off by one": ("np.ldexp(vals, (s - SCALE_BIAS)[..., None])",
                                 "np.ldexp(vals, (s - SCALE_BIAS - 1)[..., None])"),
    "MX blocks of 16": ("MX_BLOCK = 32", "MX_BLOCK = 16"),
    "k_R bytes big-endian": ('rope.astype("<u2").view(np.uint8)', 'rope.astype(">u2").view(np.uint8)'),
    "MXFP8 append ignores max_pos": ("if p < 0 or p >= max_pos:", "if p < 0:"),
}.items()})


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    (module, pins), old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", module), encoding="utf-8").read()
    assert old in src, "mutation anchor no longer present: " + name
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    (tmp_path / "oracle" / module).write_text(src.replace(old, new), encoding="utf-8")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/" + pins, "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins missed: {name}\n{r.stdout[-2000:]}"
