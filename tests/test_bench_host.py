"""Host-side logic of bench.py, on the CPU: the one-GPU contract, the split report
against hand-counted cases, the algorithmic flop counts against their closed forms,
and the source-hash gate that keeps counter summaries from describing other code."""

import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("seqlens,s_q,wgs,auto,expect", [
    # batch 1 x 2048: 64 tiles; an even split gives 1 tile per workgroup, the library's
    # choice raises it to 4, so 16 workgroups and 16 partials of the one unit
    ([2048], 1, 256, True, dict(workgroups_with_tiles=16, tiles_per_workgroup=4, fragments=16)),
    # an explicit split keeps the even share: 64 ranges of one tile
    ([2048], 1, 256, False, dict(workgroups_with_tiles=64, tiles_per_workgroup=1, fragments=64)),
    # batch 16 x 4096: 2048 tiles, 8 per workgroup, every unit cut into 16 ranges
    ([4096] * 16, 1, 256, True, dict(workgroups_with_tiles=256, tiles_per_workgroup=8, fragments=256)),
    # a unit inside one range leaves no partial
    ([100], 1, 256, True, dict(workgroups_with_tiles=1, tiles_per_workgroup=4, fragments=0)),
    # two queries over 64 tokens see 63 and 64 keys: 2 + 2 tiles; with 3 workgroups of
    # 2 tiles (ceil(4/3) = 2) each unit fills one range exactly
    ([64], 2, 3, False, dict(workgroups_with_tiles=2, tiles_per_workgroup=2, fragments=0)),
    # units of 5 and 3 tiles with ranges of 3: [0,3) [3,6) [6,8); unit 0 meets two
    # ranges, unit 1 meets two
    ([160, 96], 1, 3, False, dict(workgroups_with_tiles=3, tiles_per_workgroup=3, fragments=4)),
])
def test_split_summary_counts(seqlens, s_q, wgs, auto, expect):
    r = bench.split_summary(seqlens, s_q, wgs, auto)
    for k, v in expect.items():
        assert r[k] == v, (k, r)
    assert r["partial_bytes"] == r["fragments"] * 128 * 512 * 2
    assert r["partial_over_cache"] == round(r["partial_bytes"] / (sum(seqlens) * 1152), 4)


def test_decode_flops_closed_form():
    L = np.array([1024, 5000, 32768])
    # one query sees every cached token
    assert bench.decode_flops(L, 1) == 2 * 128 * 1088 * int(L.sum())
    # two queries see L - 1 and L tokens
    assert bench.decode_flops(L, 2) == 2 * 128 * 1088 * int((2 * L - 1).sum())


def test_prefill_flops_closed_form():
    B, L, M = 8, 4096, 4096
    expand, attn = bench.prefill_flops(B, L, M)
    assert expand == 2 * B * L * 512 * 128 * 128 * 2
    # a whole prompt: query i sees i + 1 keys, M (M + 1) / 2 in all
    assert attn == B * 128 * (M * (M + 1) // 2) * 320 * 2
    # a chunk of 256 queries over 4096 cached tokens: query i sees 3840 + i + 1 keys
    _, attn2 = bench.prefill_flops(1, 4096, 256)
    assert attn2 == 128 * sum(3840 + i + 1 for i in range(256)) * 320 * 2


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    """A copy of the decode sources and a profiles folder under a temporary root."""
    for rel in bench.TRAFFIC["decode"]["sources"]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_source_hash_ignores_comments_but_not_code(fake_root):
    h0 = bench.kernel_source_hash("decode")
    assert h0 == bench.kernel_source_hash("decode")
    src = fake_root / bench.TRAFFIC["decode"]["sources"][0]
    text = src.read_text()
    src.write_text("// a new comment line\n" + text.replace("\n", "\n\n", 3) + "\n/* block\ncomment */\n")
    assert bench.kernel_source_hash("decode") == h0
    src.write_text(text + "\nstatic int probe_variable = 1;\n")
    assert bench.kernel_source_hash("decode") != h0


def test_traffic_is_reported_only_for_the_code_it_was_taken_on(fake_root):
    f = fake_root / "profiles" / bench.TRAFFIC["decode"]["file"]
    good = bench.kernel_source_hash("decode")
    f.write_text(f"# summary\n\nsource_sha256: {good}\nfetch_bytes_per_launch: 123\nwrite_bytes_per_launch: 45\n")
    assert bench.load_traffic("decode") == {"fetch": 123.0, "write": 45.0}
    f.write_text(f"source_sha256: {'0' * 64}\nfetch_bytes_per_launch: 123\nwrite_bytes_per_launch: 45\n")
    assert bench.load_traffic("decode") is None
    f.unlink()
    assert bench.load_traffic("decode") is None


def test_committed_decode_traffic_matches_the_sources():
    """The committed summary was taken on the decode sources in the tree."""
    t = bench.load_traffic("decode")
    assert t is not None and t["fetch"] > 1.3e9


@pytest.mark.parametrize("kind", sorted(bench.TRAFFIC))
def test_every_committed_traffic_summary_matches_its_sources(kind):
    """Every kernel family's committed FETCH_SIZE/WRITE_SIZE summary was taken on the
    sources in the tree (a header shared by several families changes all their hashes)."""
    t = bench.load_traffic(kind)
    assert t is not None and t["fetch"] > 0 and t["write"] > 0, f"profiles/{bench.TRAFFIC[kind]['file']}"


def test_trace_summary_table(fake_root):
    d = fake_root / "trace"
    d.mkdir()
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp",
            '"void mla::(anonymous namespace)::decode_kernel<false>(mla::DecodeArgs)",1000,301000',
            '"void mla::(anonymous namespace)::decode_kernel<false>(mla::DecodeArgs)",400000,710000',
            '"mla::(anonymous namespace)::combine_kernel(mla::DecodeArgs, int)",720000,730000']
    (d / "run_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_trace(str(d), "t.md", ["cmd"], "test")
    text = (fake_root / "profiles" / "t.md").read_text()
    assert "| decode_kernel<false> | 2 | 305.0 | 305.0 | 300.0 | 310.0 | 98.4% |" in text
    assert "| combine_kernel | 1 | 10.0 | 10.0 | 10.0 | 10.0 | 1.6% |" in text
    assert f"source_sha256 (decode sources): {bench.kernel_source_hash('decode')}" in text


def _segments(ranges, tiles):
    """Per workgroup range: (tiles, units it meets)."""
    cum = np.concatenate([[0], np.cumsum(tiles)])
    out = []
    for _, a, b in ranges:
        out.append((b - a, sum(1 for u in range(len(tiles)) if tiles[u] > 0 and a < cum[u + 1] and b > cum[u])))
    return out


def test_segment_aware_split_hand_counted():
    """Units of 400, 100 and 300 tiles over 4 workgroups, library's own split.  The even
    split, 200 tiles each, meets 1, 1, 2 and 1 units: cost (tiles + 6 per unit met) 206,
    206, 212, 206.  The cost line puts 6 before each unit's tiles: [0,406) [406,512)
    [512,818), cut in ranges of ceil(818 / 4) = 205.  Cost 205 is tile 205 - 6 = 199 of
    unit 0, cost 410 tile 400 + max(0, 410 - 406 - 6) = 400, cost 615 tile 500 + 615 - 512
    - 6 = 597: ranges [0,199) [199,400) [400,597) [597,800), costs 205, 207, 209, 209."""
    ranges, seg, chunk = bench.split_plan([400, 100, 300], 4, True)
    assert seg == 6 and chunk == 205
    assert [(a, b) for _, a, b in ranges] == [(0, 199), (199, 400), (400, 597), (597, 800)]
    assert [t + 6 * s for t, s in _segments(ranges, [400, 100, 300])] == [205, 207, 209, 209]
    # the same units under an explicit split stay even
    ranges, seg, chunk = bench.split_plan([400, 100, 300], 4, False)
    assert seg == 0 and [(a, b) for _, a, b in ranges] == [(0, 200), (200, 400), (400, 600), (600, 800)]
    # ranges on unit starts already (every range inside one unit): no change
    ranges, seg, _ = bench.split_plan([256, 256, 512], 4, True)
    assert seg == 0


@pytest.mark.parametrize("seed", range(6))
def test_segment_aware_split_properties(seed):
    """Random workloads (zero-tile units included), 256 workgroups: the ranges tile the
    line without gaps; the merge's formulas (first and last workgroup of a unit, and whether
    the first fragment is a later segment of its workgroup) agree with the ranges; and the
    largest range cost, tiles + 6 per unit met, is never above the even split's."""
    rng = np.random.default_rng(seed)
    for _ in range(20):
        U = int(rng.integers(1, 150))
        tiles = np.where(rng.random(U) < 0.1, 0, rng.integers(1, 1200, size=U))
        for auto in (True, False):
            ranges, seg, chunk = bench.split_plan(tiles, 256, auto)
            if tiles.sum() == 0:
                assert ranges == []
                continue
            assert ranges[0][1] == 0 and ranges[-1][2] == tiles.sum()
            assert all(r[2] == s[1] for r, s in zip(ranges, ranges[1:]))
            cum = np.concatenate([[0], np.cumsum(tiles)])
            ccum = np.concatenate([[0], np.cumsum(np.where(tiles > 0, tiles + seg, 0))])
            for u in range(U):
                if tiles[u] == 0:
                    continue
                gs = [g for g, a, b in ranges if a < cum[u + 1] and b > cum[u]]
                g0, g1 = (ccum[u] + seg) // chunk, (ccum[u] + seg + tiles[u] - 1) // chunk
                assert gs == list(range(g0, g1 + 1))
                start0 = [a for g, a, b in ranges if g == g0][0]
                assert (start0 < cum[u]) == (g0 * chunk < ccum[u])
            if auto:
                cost = max(t + 6 * s for t, s in _segments(ranges, tiles))
                plain_chunk = max(-(-int(tiles.sum()) // 256), 4)
                plain = []
                for g in range(256):
                    a, b = g * plain_chunk, min(int(tiles.sum()), (g + 1) * plain_chunk)
                    if a < b:
                        plain.append((g, a, b))
                assert cost <= max(t + 6 * s for t, s in _segments(plain, tiles)) + 1
