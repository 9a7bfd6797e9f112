"""Plants plausible mistakes in a scratch copy of the oracle (CPU only) and
checks that the oracle's pins reject every one of them."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

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


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "mla_oracle.py"), encoding="utf-8").read()
    old, new = MUTATIONS[name]
    assert old in src, "mutation anchor no longer present: " + name
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    (tmp_path / "oracle" / "mla_oracle.py").write_text(src.replace(old, new), encoding="utf-8")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_attention.py", "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins missed: {name}\n{r.stdout[-2000:]}"
