#!/usr/bin/env python3
"""Benchmark of absorbed MLA paged decode on one MI355X.

One step = one ``mla_decode_paged`` call (plan + split-KV decode + LSE merge)
for one layer of the batch-64 workload: 64 sequences with lengths drawn
uniformly from [1024, 32768] (seed 44, 1 166 687 cached tokens, 18 261 pages of
64 tokens, 1.34 GB of bf16 latent cache), 128 heads, one query token each.
Inputs are resident in HBM before the timed region; the cache is five times
the 256 MiB last-level cache, so back-to-back steps stream it from HBM.

Prints ONE JSON line on stdout (value = achieved cache-read GB/s of a step).
"""

from __future__ import annotations

import os

for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(min(len(os.sched_getaffinity(0)), 16)))

import argparse  # noqa: E402
import json  # noqa: E402
import math  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

import numpy as np  # noqa: E402

METRIC = "decode attention µs/step + achieved HBM GB/s (% roofline), B=64 ctx=32K"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
ROW_BYTES = 1152               # one cached token of one layer: 576 bf16
COPY_BYTES = 512 << 20         # device copy of known size that calibrates the HBM byte counters
ROOT = os.path.dirname(os.path.abspath(__file__))
# Counter summaries (HBM bytes per launch): one per measured kernel family, each keyed
# by a hash of the sources its kernels are built from.
_CSRC = "mla_latent_kv_04_amd/csrc/"
TRAFFIC = {
    "decode": dict(file="decode_kernel_c3_b64_traffic.md", kernels=("decode_kernel",),
                   sources=(_CSRC + "decode.hip", _CSRC + "common.h", _CSRC + "mxfp8.h"),
                   title="decode_kernel: paged MLA decode, batch 64, seq_len U[1024,32768]"),
    "mxfp8": dict(file="decode_kernel_mxfp8_c3_b64_traffic.md", kernels=("decode_kernel",),
                  sources=(_CSRC + "decode.hip", _CSRC + "common.h", _CSRC + "mxfp8.h"),
                  title="decode_kernel over the MXFP8 cache: paged MLA decode, batch 64, seq_len U[1024,32768]"),
    "c5": dict(file="decode_kernel_c5_b4_sq2_traffic.md", kernels=("decode_kernel",),
               sources=(_CSRC + "decode.hip", _CSRC + "common.h", _CSRC + "mxfp8.h"),
               title="decode_kernel: two-token verify, batch 4, seq_len 131072"),
    "append": dict(file="append_kernel_c3_b64_traffic.md", kernels=("append_kernel", "append_finalize_kernel"),
                   sources=(_CSRC + "append.hip", _CSRC + "append.h", _CSRC + "common.h"),
                   title="cache append: 64 new tokens of the batch-64 workload, d = 7168 (both kernels of a call)"),
    "prefill": dict(file="prefill_attention_b8_4096_traffic.md", kernels=("prefill_attention_kernel",),
                    sources=(_CSRC + "prefill.hip", _CSRC + "prefill.h", _CSRC + "common.h"),
                    title="prefill_attention_kernel: 8 sequences x 4096-token prompt, one chunk"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", TRAFFIC["decode"]["file"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _dev_i32(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


WARM_SECONDS = 1.5   # untimed decode work before each timed region: the clock settles under the power cap
FLUSH_BYTES = 1 << 30   # written between cold calls: four times the 256 MiB last-level cache


def _warm(fn, warmup, torch):
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    t0 = time.time()
    while time.time() - t0 < WARM_SECONDS:
        for _ in range(10):
            fn(0)
        torch.cuda.synchronize()


def _per_call(fn, n, torch, flush=None):
    """GPU milliseconds of n calls, each between two stream events of its own.  With
    `flush`, a 1 GiB write runs before every call, outside its events, so the call
    finds neither its cache pages nor its queries in L2 or the last-level cache."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (e0, e1) in enumerate(ev):
        if flush is not None:
            flush()
        e0.record()
        fn(i)
        e1.record()
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) for e0, e1 in ev])


def _dist_us(ms):
    """median / p10 / p90 / mean of per-call times, in microseconds."""
    us = np.asarray(ms) * 1e3
    return {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2), "mean": round(float(us.mean()), 2), "calls": int(us.size)}


def _flusher(torch):
    """Evicts L2 and the last-level cache between cold calls: a 1 GiB write, then a 1 GiB
    read of another buffer, so the caches end up holding clean lines of neither the call's
    cache pages nor its queries, and no dirty lines are left to be written back during the
    timed call."""
    wbuf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    rbuf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    state = {"i": 0}

    def flush():
        state["i"] += 1
        wbuf.fill_(state["i"] & 0xFF)
        torch.amax(rbuf)
    return flush


REDO_SLOPE = 0.25   # k_R[t][0] = REDO_SLOPE * t in the redo leg


def run_redo(inp, pool_dev, torch, mla, steps, warmup, normal_ms):
    """The batch-64 step with scores that rise along every sequence: q_abs = 0, q_R = e_0 for
    every head, and the first RoPE component of token t's row set to REDO_SLOPE * t, so the score
    of token t is scale * REDO_SLOPE * t.  A decode range re-runs once with its true maximum when a
    later score leaves the first tile's maximum more than 64 log2 units behind; here that happens
    in every range spanning more than 64 ln 2 / (scale * REDO_SLOPE) tokens.  Reports the step time
    against the normal step's."""
    n_seq = inp.batch
    pages = np.full(int(pool_dev.shape[0]), -1, dtype=np.int64)
    ramp = np.zeros((int(pool_dev.shape[0]), 64), dtype=np.float32)
    for b in range(n_seq):
        n = (int(inp.seqlens[b]) + 63) // 64
        for j in range(n):
            ramp[inp.block_table[b, j]] = REDO_SLOPE * (64 * j + np.arange(64))
    pool2 = pool_dev.clone()
    pool2[:, :, 512] = torch.from_numpy(ramp).cuda().to(torch.bfloat16)
    del pages
    q_abs = torch.zeros((n_seq, 1, 128, 512), dtype=torch.bfloat16, device="cuda")
    q_r = torch.zeros((n_seq, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    q_r[..., 0] = 1.0
    sl, bt = _dev_i32(inp.seqlens, torch), _dev_i32(inp.block_table, torch)
    out = torch.empty(n_seq, 1, 128, 512, dtype=torch.bfloat16, device="cuda")
    params = mla.make_params(n_seq, 1, inp.max_blocks, int(pool2.shape[0]), inp.scale)
    ws = torch.empty(mla.workspace_size(params), dtype=torch.uint8, device="cuda")

    def step(i):
        mla.decode_paged(q_abs, q_r, pool2, bt, sl, scale=inp.scale, out_latent=out, want_lse=False, workspace=ws)
    ms, per, dist = _time_calls(step, steps, warmup, torch, mla)
    del pool2
    torch.cuda.empty_cache()
    span = 64 * math.log(2) / (inp.scale * REDO_SLOPE)
    return {"workload": "the batch-64 step with scores rising along every sequence (q_abs = 0, q_R = e_0, "
                        f"k_R[t][0] = {REDO_SLOPE} t): every decode range longer than {span:.0f} tokens is redone "
                        "once with its true maximum",
            "us_per_step": round(ms * 1e3, 2), "timing_us": dist,
            "kernels_us": {k: round(v * 1e3, 2) for k, v in per.items()},
            "step_time_vs_normal": round(ms / normal_ms, 4)}


def run_stream(inp, pool_dev, torch, mla, steps, warmup):
    """Time mla_stream_pages over a workload: the decode's page stream alone (same split,
    loads and LDS ring, no arithmetic), the stream-read ceiling the decode kernel is
    measured against."""
    bt, sl = _dev_i32(inp.block_table, torch), _dev_i32(inp.seqlens, torch)
    params = mla.make_params(inp.batch, inp.s_q, inp.max_blocks, int(pool_dev.shape[0]), inp.scale)
    ws = torch.empty(mla.workspace_size(params), dtype=torch.uint8, device="cuda")
    sums = torch.empty(mla.decode_num_workgroups(params) * 256, dtype=torch.int32, device="cuda")

    def step(i):
        mla.stream_pages(pool_dev, bt, sl, s_q=inp.s_q, sums=sums, workspace=ws)
    _warm(step, warmup, torch)
    ms = _per_call(step, steps, torch)
    cache_bytes = int(inp.seqlens.astype(np.int64).sum()) * ROW_BYTES
    med = float(np.median(ms))
    return {"kernel": "stream_kernel (mla_stream_pages)", "timing_us": _dist_us(ms),
            "GBps_median": round(cache_bytes / (med * 1e-3) / 1e9, 1),
            "frac_of_peak": round(cache_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def run_cache_resident(inp, pool_dev, torch, mla, steps, warmup, decode_ms):
    """The batch-64 step with every block-table entry mapped onto the first 32 pages of the
    pool (2.25 MiB, which every die's 4 MiB L2 holds): the same sequences, lengths, split and
    arithmetic as the real step, with the cache reads served from L2 instead of HBM.  The
    decode kernel's time here is its time when HBM bandwidth is not the limit."""
    bt = _dev_i32((inp.block_table.astype(np.int64) % 32).astype(np.int32), torch)
    sl = _dev_i32(inp.seqlens, torch)
    qa = torch.randn((inp.batch, 1, 128, 512), device="cuda").to(torch.bfloat16)
    qr = torch.randn((inp.batch, 1, 128, 64), device="cuda").to(torch.bfloat16)
    out = torch.empty(inp.batch, 1, 128, 512, dtype=torch.bfloat16, device="cuda")
    params = mla.make_params(inp.batch, 1, inp.max_blocks, int(pool_dev.shape[0]), inp.scale)
    ws = torch.empty(mla.workspace_size(params), dtype=torch.uint8, device="cuda")

    def step(i):
        mla.decode_paged(qa, qr, pool_dev, bt, sl, scale=inp.scale, out_latent=out, want_lse=False, workspace=ws)
    ms, per, dist = _time_calls(step, steps, warmup, torch, mla)
    return {"workload": "the batch-64 step (same lengths and split) with every page of every sequence mapped onto "
                        "the first 32 pages of the pool (2.25 MiB, resident in each die's L2)",
            "us_per_step": round(ms * 1e3, 2), "timing_us": dist,
            "kernels_us": {k: round(v * 1e3, 2) for k, v in per.items()},
            "decode_kernel_vs_hbm_resident": round(per["decode"] / decode_ms, 4)}


def _time_calls(fn, steps, warmup, torch, mla, flush=None):
    """Warm up (`warmup` calls, and at least WARM_SECONDS of calls so that the
    engine clock has settled), then time exactly `steps` calls between two
    synchronisations, without any other instrumentation; then the same number of
    calls each between its own events, back to back (warm) and, given `flush`,
    after a 1 GiB write each (cold); then `steps` more calls with the library's
    per-kernel events for the breakdown.  Returns (ms per call from the stream
    events around the first run, per-kernel ms per launch of the kernels that ran,
    {"warm": distribution, "cold": distribution or absent})."""
    _warm(fn, warmup, torch)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # the step time: nothing but the calls between the two events
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    dist = {"warm": _dist_us(_per_call(fn, steps, torch))}
    if flush is not None:
        dist["cold"] = _dist_us(_per_call(fn, steps, torch, flush))
        _warm(fn, 0, torch)
    # the per-kernel split: the same calls again with the library's per-kernel events
    with mla.KernelTimer() as kt:
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
    return ms, kt.per_launch_ms(), dist


def _workload_from_synth(name, torch, with_host_pool=True):
    from synth import make_inputs
    t0 = time.time()
    inp = make_inputs(name, with_pool=with_host_pool)
    log(f"[bench] {name}: generated on host in {time.time() - t0:.1f}s "
        f"(B={inp.batch} s_q={inp.s_q} tokens={int(inp.seqlens.sum())} pages={inp.num_pages})")
    return inp


def _device_pool(num_pages, seed, torch):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((num_pages, 64, 576), dtype=torch.bfloat16, device="cuda", generator=g)


MXFP8_ROW_BYTES = 656   # MXFP8 cache row: 512 E4M3 codes + 16 E8M0 scale bytes + 64 bf16 of k_R


def run_mxfp8(inp, pool_dev, torch, mla, steps, warmup):
    """Time the paged decode of a workload over its MXFP8 cache (made on the device from
    the bf16 cache); returns a result dict like run_paged's."""
    pool8 = mla.quantize_kv_mxfp8(pool_dev)
    q_abs = mla.absorb_q(_dev_bf16(inp.q_c, torch), _dev_bf16(inp.w_uk, torch))
    q_r = _dev_bf16(inp.q_r, torch)
    sl, bt = _dev_i32(inp.seqlens, torch), _dev_i32(inp.block_table, torch)
    B, s_q = inp.batch, inp.s_q
    out = torch.empty(B, s_q, 128, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, s_q, 128, dtype=torch.float32, device="cuda")
    params = mla.make_params(B, s_q, inp.max_blocks, int(pool8.shape[0]), inp.scale)
    ws = torch.empty(mla.workspace_size(params), dtype=torch.uint8, device="cuda")

    def step(i):
        mla.decode_paged_mxfp8(q_abs, q_r, pool8, bt, sl, scale=inp.scale, out_latent=out, lse=lse, workspace=ws)

    ms, per, dist = _time_calls(step, steps, warmup, torch, mla)
    del pool8
    cache_bytes = int(inp.seqlens.astype(np.int64).sum()) * MXFP8_ROW_BYTES
    return dict(ms=ms, per=per, dist=dist, cache_bytes=cache_bytes, tokens=int(inp.seqlens.sum()), queries=B * s_q)


def decode_flops(seqlens, s_q):
    """Algorithmic flops of one decode step: 2 x 128 heads x (576 + 512) per visible
    (key, query) pair -- the scores over the 576-wide row and P . c_KV over 512."""
    L = np.asarray(seqlens, dtype=np.int64)
    visible = int(sum(int(l) - s_q + i + 1 for l in L for i in range(s_q)))
    return 2 * 128 * (576 + 512) * visible


AUTO_MIN_CHUNK = 4    # fewest tiles per workgroup when the library sizes the split (num_splits = 0)


SEG_COST = 6          # tiles a segment start counts for in the library's own split
COST_SPLIT_MIN = 48   # fewest tiles per range for which that split applies


def unit_tiles(seqlens, s_q):
    """32-token tiles of each (sequence, query) unit: query i of a sequence of L tokens sees
    L - s_q + i + 1 keys."""
    out = []
    for L in np.asarray(seqlens, dtype=np.int64):
        for i in range(s_q):
            vis = max(int(L) - s_q + i + 1, 0)
            out.append((vis + 31) // 32)
    return np.asarray(out, dtype=np.int64)


def split_plan(tiles, workgroups, auto):
    """The decode's work split (the same rule as the kernels' work_range): the units' tiles
    laid end to end on a cost line where each unit with tiles also counts SEG_COST tiles for
    its segment start (only in the library's own split, with ranges of COST_SPLIT_MIN tiles or
    more, and when the even split's boundaries do not all fall on unit starts), cut evenly
    into ranges of ceil(cost / workgroups) (at least AUTO_MIN_CHUNK when auto). Returns the
    workgroups with work as (g, start, end), tiles [start, end), the segment cost used and
    the range length on the cost line."""
    tiles = np.asarray(tiles, dtype=np.int64)
    min_chunk = AUTO_MIN_CHUNK if auto else 1
    cum = np.concatenate([[0], np.cumsum(tiles)])
    total = int(cum[-1])
    chunk0 = max(-(-total // workgroups), min_chunk)
    aligned = all(cum[u] % chunk0 == 0 for u in range(len(tiles)) if tiles[u] > 0)
    seg = SEG_COST if (min_chunk > 1 and chunk0 >= COST_SPLIT_MIN and not aligned) else 0
    ccum = np.concatenate([[0], np.cumsum(np.where(tiles > 0, tiles + seg, 0))])
    T = int(ccum[-1])
    chunk = max(-(-T // workgroups), min_chunk)

    def tile_at(c):
        u = int(np.searchsorted(ccum[:-1], c, side="right")) - 1   # last unit with ccum <= c
        return int(cum[u]) + max(0, c - int(ccum[u]) - seg)

    ranges = []
    for g in range(workgroups):
        cs = g * chunk
        if cs >= T or total == 0:
            break
        ce = min(T, cs + chunk)
        start, end = tile_at(cs), (total if ce >= T else tile_at(ce))
        if end > start:
            ranges.append((g, start, end))
    return ranges, seg, chunk


def split_summary(seqlens, s_q, workgroups, auto):
    """The decode's split of a workload, for the report (split_plan); a unit cut by range
    boundaries leaves one bf16 partial output (128 heads x 512) per range it meets, which
    the merge reads back."""
    tiles = unit_tiles(seqlens, s_q)
    ranges, seg, _ = split_plan(tiles, workgroups, auto)
    cum = np.concatenate([[0], np.cumsum(tiles)])
    frags = 0
    for u in range(len(tiles)):
        if tiles[u] == 0:
            continue
        meet = sum(1 for _, a, b in ranges if a < cum[u + 1] and b > cum[u])
        if meet > 1:
            frags += meet
    part = frags * 128 * 512 * 2
    return {"workgroups_launched": workgroups, "workgroups_with_tiles": len(ranges), "tiles": int(cum[-1]),
            "tiles_per_workgroup": max((b - a for _, a, b in ranges), default=0), "segment_cost_tiles": seg,
            "fragments": frags, "partial_bytes": part,
            "partial_over_cache": round(part / (int(np.sum(seqlens)) * ROW_BYTES), 4)}


def run_split_sweep(names, values, steps, torch, mla, command):
    """Times the paged decode step of each named workload for each num_splits value (0 =
    the library's own choice), warm and HBM-cold, and writes the table to profiles/."""
    from synth import make_inputs
    flush = _flusher(torch)
    lines = [f"# Split sizing of the paged decode: workloads {', '.join(names)}", "",
             "Command (run from the repository root on one MI355X):", "", "```", *command, "```", "",
             "Per workload and `num_splits` (0 = the library's choice: one workgroup per compute unit, at least "
             f"{AUTO_MIN_CHUNK} tiles each): the split (tiles of 32 tokens per workgroup, units cut into "
             "fragments, bytes of bf16 partial outputs written and read back by the merge, as a share of the "
             "cache bytes), then the step time (decode + merge) median over back-to-back calls (warm) and over "
             "calls each after a 1 GiB write and a 1 GiB read of other buffers (cold), and the two kernels' "
             "durations from the library's per-kernel events (each includes about 2 us of event overhead).", "",
             "| workload | num_splits | workgroups | tiles each | fragments | partials / cache | warm us | "
             "cold us | decode us | merge us |", "|---|---|---|---|---|---|---|---|---|---|"]
    for name in names:
        oi = make_inputs(name, with_pool=False)
        pool = _device_pool(oi.num_pages, oi.seed, torch)
        q_abs = torch.randn((oi.batch, oi.s_q, 128, 512), device="cuda").to(torch.bfloat16)
        q_r = torch.randn((oi.batch, oi.s_q, 128, 64), device="cuda").to(torch.bfloat16)
        sl, bt = _dev_i32(oi.seqlens, torch), _dev_i32(oi.block_table, torch)
        out = torch.empty(oi.batch, oi.s_q, 128, 512, dtype=torch.bfloat16, device="cuda")
        for ns in values:
            params = mla.make_params(oi.batch, oi.s_q, oi.max_blocks, oi.num_pages, oi.scale, ns)
            ws = torch.empty(mla.workspace_size(params), dtype=torch.uint8, device="cuda")
            wgs = mla.decode_num_workgroups(params)

            def step(i):
                mla.decode_paged(q_abs, q_r, pool, bt, sl, scale=oi.scale, num_splits=ns, out_latent=out,
                                 want_lse=False, workspace=ws)
            ms, per, dist = _time_calls(step, steps, 5, torch, mla, flush)
            sp = split_summary(oi.seqlens, oi.s_q, wgs, ns == 0)
            lines.append(f"| {name} | {ns} | {wgs} | {sp['tiles_per_workgroup']} | {sp['fragments']} | "
                         f"{sp['partial_over_cache']:.1%} | {dist['warm']['median']:.1f} | "
                         f"{dist['cold']['median']:.1f} | {per.get('decode', 0) * 1e3:.1f} | "
                         f"{per.get('combine', 0) * 1e3:.1f} |")
            log(f"[bench] sweep {lines[-1]}")
        del pool
        torch.cuda.empty_cache()
    lines += ["", f"source_sha256 (decode sources): {kernel_source_hash('decode')}", ""]
    path = os.path.join(ROOT, "profiles", f"decode_split_sweep_{'_'.join(names)}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"[bench] wrote {path}")


def other_row(oi, orr, layers):
    """Report row of a workload other than the graded one: step time (back-to-back calls),
    per-call distributions warm and cold, the decode kernel's time and its roofline -- HBM
    for one query per sequence, MFMA when several queries share each cache byte."""
    dec_ms = orr["per"]["decode"]
    row = {"us_per_step": round(orr["ms"] * 1e3, 2),
           "cache_GBps": round(orr["cache_bytes"] / (orr["ms"] * 1e-3) / 1e9, 1),
           "timing_us": orr["dist"],
           "kernels_us": {k: round(v * 1e3, 2) for k, v in orr["per"].items()},
           "batch": oi.batch, "s_q": oi.s_q, "cached_tokens": orr["tokens"],
           "pool": "device-generated bf16 N(0,1)" + (", 60 layers, layer i%60 per call" if layers > 1 else ""),
           "split": split_summary(oi.seqlens, oi.s_q, orr["workgroups"], True)}
    cold = orr["dist"].get("cold")
    if cold is not None:
        row["cold_cache_GBps_median"] = round(orr["cache_bytes"] / (cold["median"] * 1e-6) / 1e9, 1)
    flops = decode_flops(oi.seqlens, oi.s_q)
    if oi.s_q > 1:
        tf = flops / (dec_ms * 1e-3) / 1e12
        row["roofline"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                           "kernel": "decode_kernel", "algorithmic_flops_per_launch": flops,
                           "hbm_GBps_of_cache": round(orr["cache_bytes"] / (dec_ms * 1e-3) / 1e9, 1)}
        # HBM bytes of this workload's launch, where a counter summary for it is committed
        t = load_traffic(oi.name) if oi.name in TRAFFIC else None
        row["roofline"]["traffic"] = int(t["fetch"] + t["write"]) if t else None
        row["roofline"]["traffic_split"] = t
    else:
        gb = orr["cache_bytes"] / (dec_ms * 1e-3) / 1e9
        row["roofline"] = {"bound": "hbm", "achieved": round(gb, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gb / HBM_PEAK_GBS, 4), "kernel": "decode_kernel",
                           "algorithmic_bytes_per_launch": orr["cache_bytes"]}
    return row


def mxfp8_row(inp, pool, torch, mla, steps, warmup, ms):
    """The graded workload over its MXFP8 cache: step time, kernels, roofline on 656-byte rows."""
    f8 = run_mxfp8(inp, pool, torch, mla, steps, warmup)
    f8_dec = f8["per"]["decode"]
    f8_ach = f8["cache_bytes"] / (f8_dec * 1e-3) / 1e9
    traffic8 = load_traffic("mxfp8")
    mx = {
        "workload": "the batch-64 workload above, cache in MXFP8 (E4M3 codes, one E8M0 scale per 32 latent "
                    "values, bf16 k_R: 656 B per token)",
        "us_per_step": round(f8["ms"] * 1e3, 2),
        "timing_us": f8["dist"],
        "kernels_us": {k: round(v * 1e3, 2) for k, v in f8["per"].items()},
        "cache_bytes_per_step": f8["cache_bytes"],
        "cache_GBps": round(f8["cache_bytes"] / (f8["ms"] * 1e-3) / 1e9, 1),
        "kv_tokens_per_s": round(f8["tokens"] / (f8["ms"] * 1e-3), 1),
        "step_speedup_vs_bf16_cache": round(ms / f8["ms"], 4),
        "roofline": {"bound": "hbm", "achieved": round(f8_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(f8_ach / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic8 is None else round(traffic8["fetch"] + traffic8["write"]),
                     "traffic_split": traffic8, "kernel": "decode_kernel (MXFP8 variant)",
                     "algorithmic_bytes_per_launch": f8["cache_bytes"]},
    }
    return mx


def run_paged(inp, pool_dev, torch, mla, steps, warmup, layers=1, pages_per_layer=None, flush=None):
    """Time the paged decode of one workload; returns a result dict."""
    q_abs = mla.absorb_q(_dev_bf16(inp.q_c, torch), _dev_bf16(inp.w_uk, torch))
    q_r = _dev_bf16(inp.q_r, torch)
    sl = _dev_i32(inp.seqlens, torch)
    bts = [_dev_i32(inp.block_table + (l * pages_per_layer if layers > 1 else 0), torch) for l in range(layers)]
    B, s_q = inp.batch, inp.s_q
    out = torch.empty(B, s_q, 128, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, s_q, 128, dtype=torch.float32, device="cuda")
    params = mla.make_params(B, s_q, inp.max_blocks, int(pool_dev.shape[0]), inp.scale)
    ws = torch.empty(mla.workspace_size(params), dtype=torch.uint8, device="cuda")

    def step(i):
        mla.decode_paged(q_abs, q_r, pool_dev, bts[i % layers], sl, scale=inp.scale, out_latent=out, lse=lse,
                         workspace=ws)

    ms, per, dist = _time_calls(step, steps, warmup, torch, mla, flush)
    cache_bytes = int(inp.seqlens.astype(np.int64).sum()) * ROW_BYTES
    return dict(ms=ms, per=per, dist=dist, cache_bytes=cache_bytes, tokens=int(inp.seqlens.sum()), queries=B * s_q,
                workgroups=mla.decode_num_workgroups(params))


D_MODEL = 7168                 # hidden size d of the appended tokens' states


def append_algorithmic_bytes(tokens, d=D_MODEL):
    """Bytes the cache append must move once: W_A [d, 576] bf16, x [T, d] bf16, the T new
    rows written, T fp32 table rows of 64, and one block-table entry and length per token."""
    return d * 576 * 2 + tokens * d * 2 + tokens * ROW_BYTES + tokens * 64 * 4 + tokens * 8


def run_append(inp, pool_dev, torch, mla, steps, warmup):
    """Time mla_append_kv (one new token per sequence of the workload, hidden size 7168),
    alone and with the query rotation fused in, and mla_rope_q on the same tokens.
    The GPU time per call comes from replaying a captured graph of calls (between
    stream events); the library's per-kernel HIP events and the per-call times of
    eager calls are reported too, but at this size they include event and Python
    binding overhead respectively."""
    from synth import make_append_inputs
    x_bits, w_bits = make_append_inputs(80, inp.batch, inp.s_q)
    x, w_a = _dev_bf16(x_bits, torch), _dev_bf16(w_bits, torch)
    table = mla.rope_table(131072)
    bt, sl = _dev_i32(inp.block_table, torch), _dev_i32(inp.seqlens, torch)
    params = mla.make_append_params(inp.batch, inp.s_q, D_MODEL, inp.max_blocks, int(pool_dev.shape[0]), 131072)
    ws = mla.append_workspace(params)
    q_r = _dev_bf16(inp.q_r, torch)

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with mla.KernelTimer() as kt:
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
        per = {k: v / max(kt.append_calls, 1) for k, v in kt.append_ms.items()}
        return e0.elapsed_time(e1) / n, per

    def graph_timed(fn, calls=20, replays=10):
        """GPU time per call from a captured graph of `calls` calls, replayed `replays`
        times (no host overhead between calls); every replay's rows are checked against
        the eager call's."""
        pos = inp.seqlens.astype(np.int64) - 1
        pages = torch.from_numpy(inp.block_table[np.arange(inp.batch), pos // 64].astype(np.int64)).cuda()
        rows = torch.from_numpy(pos % 64).cuda()
        fn()
        torch.cuda.synchronize()
        ref = pool_dev[pages, rows].clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                fn()
        times = []
        for _ in range(replays):
            pool_dev[pages, rows] = 0
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / calls)
            assert torch.equal(pool_dev[pages, rows], ref), "graph replay wrote other rows than the eager call"
        del g
        return float(np.median(times))

    graph_ms = graph_timed(lambda: mla.append_kv(x, w_a, table, pool_dev, bt, sl, workspace=ws))
    app_ms, app_k = timed(lambda: mla.append_kv(x, w_a, table, pool_dev, bt, sl, workspace=ws), steps)
    appq_ms, appq_k = timed(lambda: mla.append_kv(x, w_a, table, pool_dev, bt, sl, q_r=q_r, workspace=ws), steps)
    rope_ms, _ = timed(lambda: mla.rope_q(q_r, table, sl), steps)
    T = inp.batch * inp.s_q
    alg = append_algorithmic_bytes(T)
    proj_alg = D_MODEL * 576 * 2 + T * D_MODEL * 2          # W_A and x: what the projection kernel must read
    achieved = alg / (graph_ms * 1e-3) / 1e9
    traffic = load_traffic("append")
    return {
        "workload": f"{T} new tokens (one per sequence of the batch-64 workload), d={D_MODEL}, "
                    "W_A [7168, 576] bf16, fp32 RoPE table of 131072 rows, rows written into the shared pool",
        "gpu_us_per_call": round(graph_ms * 1e3, 2),
        "tokens_per_s": round(T / (graph_ms * 1e-3), 1),
        "event_bracketed_kernels_us": {k: round(v * 1e3, 2) for k, v in app_k.items()},
        "event_bracketed_kernels_with_q_rotation_us": {k: round(v * 1e3, 2) for k, v in appq_k.items()},
        "host_bound_us_per_call": {"append": round(app_ms * 1e3, 2), "append_with_q": round(appq_ms * 1e3, 2),
                                   "rope_q_alone": round(rope_ms * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic["fetch"] + traffic["write"]),
                     "traffic_split": traffic,
                     "kernel": "append_kernel<32> + append_finalize_kernel (one call, graph-replayed)",
                     "algorithmic_bytes_per_launch": alg},
        "projection_algorithmic_bytes": proj_alg,
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def prefill_flops(B, L, M):
    """Algorithmic flops of a decompress-branch prefill chunk (M queries over L cached tokens
    per sequence): the K and V expansion of every cached token (2 x 512 x 128 per head and
    tensor) and the causal attention (192-wide scores plus 128-wide P.V per visible key)."""
    expand = 2 * B * L * 512 * 128 * 128 * 2
    visible = sum(L - M + i + 1 for i in range(M))
    attn = B * 128 * visible * (192 + 128) * 2
    return expand, attn


def run_prefill(torch, mla, steps, warmup):
    """Prefill of an 8 x 4096-token prompt in one chunk (M = L = 4096, decompress branch),
    timed per kernel with the library's HIP events; then absorbed vs decompressed time for
    shorter chunks at the end of the same 4096-token sequences (the threshold check)."""
    from synth import make_custom
    B, L = 8, 4096
    base = make_custom(102, B, 1, [L] * B)
    pool = _dev_bf16(base.pool, torch)
    bt, sl = _dev_i32(base.block_table, torch), _dev_i32(base.seqlens, torch)
    w_uk, w_uv = _dev_bf16(base.w_uk, torch), _dev_bf16(base.w_uv, torch)
    g = torch.Generator(device="cuda")
    g.manual_seed(103)

    def inputs(M):
        q_c = torch.randn((B, M, 128, 128), device="cuda", generator=g).to(torch.bfloat16)
        q_r = torch.randn((B, M, 128, 64), device="cuda", generator=g).to(torch.bfloat16)
        return q_c, q_r

    def timed(M, mode, n, w):
        q_c, q_r = inputs(M)
        params = mla.make_prefill_params(B, M, base.max_blocks, base.num_pages, base.scale, mode)
        ws = torch.empty(mla.prefill_workspace_size(params), dtype=torch.uint8, device="cuda")
        out = torch.empty(B, M, 128, 128, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, M, 128, dtype=torch.float32, device="cuda")

        def call():
            mla.prefill(q_c, q_r, w_uk, w_uv, pool, bt, sl, scale=base.scale, mode=mode, out=out, lse=lse,
                        workspace=ws)
        for _ in range(w):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with mla.KernelTimer() as kt:
            e0.record()
            for _ in range(n):
                call()
            e1.record()
            torch.cuda.synchronize()
        per = {k: v / max(kt.prefill_calls, 1) for k, v in kt.prefill_ms.items()}
        return e0.elapsed_time(e1) / n, per

    ms, per = timed(L, 0, steps, warmup)
    traffic = load_traffic("prefill")
    expand, attn = prefill_flops(B, L, L)
    achieved = attn / (per["attention"] * 1e-3) / 1e12
    cross = {}
    for M in (64, 128, 256):
        a_ms, _ = timed(M, 1, max(steps // 2, 3), 2)
        d_ms, _ = timed(M, 2, max(steps // 2, 3), 2)
        cross[str(M)] = {"absorbed_us": round(a_ms * 1e3, 1), "decompressed_us": round(d_ms * 1e3, 1)}
    return {
        "workload": "prefill chunk, 8 sequences x 4096-token prompt (M = L = 4096, all rows cached), "
                    "128 heads, decompress branch (K/V expansion + causal attention), bf16",
        "us_per_call": round(ms * 1e3, 1),
        "kernels_us": {k: round(v * 1e3, 1) for k, v in per.items()},
        "tokens_per_s": round(B * L / (ms * 1e-3), 1),
        "tflops": {"expand": round(expand / (per["decompress"] * 1e-3) / 1e12, 1),
                   "attention": round(achieved, 1),
                   "whole_call": round((expand + attn) / (ms * 1e-3) / 1e12, 1)},
        "algorithmic_flops": {"expand": expand, "attention": attn},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None if traffic is None else round(traffic["fetch"] + traffic["write"]),
                     "traffic_split": traffic,
                     "kernel": "prefill_attention_kernel", "algorithmic_flops_per_launch": attn},
        "absorb_vs_decompress_at_L4096": cross,
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, seconds):
    """The fp64 oracle timed on host cores over the same workload's inputs: the absorbed
    form (what the kernels compute) on whole sequences until `seconds` have passed, and
    the decompressed form (the definition parity is checked against) on the shortest
    sequence, heads added until about `seconds` more have passed; both extrapolated to
    the whole step."""
    import oracle
    qa = oracle.absorb_q(inp.q_c, inp.w_uk)
    order = np.random.default_rng(0).permutation(inp.batch)
    done, toks = [], 0
    t0 = time.perf_counter()
    for b in order:
        oracle.decode_absorbed(qa, inp.q_r, inp.pool, inp.block_table, inp.seqlens, inp.s_q, inp.scale, batches=[b])
        done.append(int(b))
        toks += int(inp.seqlens[b])
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    total = int(inp.seqlens.sum())
    # decompressed: the shortest sequence, heads in blocks of 8 until the time is spent
    b = int(np.argmin(inp.seqlens))
    heads_done = 0
    t1 = time.perf_counter()
    while heads_done < 128:
        hs = list(range(heads_done, min(heads_done + 8, 128)))
        oracle.decode_decompressed(inp.q_c, inp.q_r, inp.w_uk, inp.w_uv, inp.pool, inp.block_table, inp.seqlens,
                                   inp.s_q, inp.scale, batches=[b], heads=hs)
        heads_done += len(hs)
        if time.perf_counter() - t1 >= seconds:
            break
    dd = time.perf_counter() - t1
    dd_step = dd * (128 / heads_done) * (total / int(inp.seqlens[b]))
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": toks * ROW_BYTES / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle.decode_absorbed (fp64) on {len(done)} of {inp.batch} sequences "
                      f"({toks} cached tokens) in {dt:.1f}s; seconds_per_step_extrapolated="
                      f"{dt * total / max(toks, 1):.1f}",
            "host_cores_available": len(os.sched_getaffinity(0)), "blas_threads": threads,
            "cpu_model": _cpu_model(),
            "decompressed": {"value": total * ROW_BYTES / dd_step / 1e9, "unit": "GB/s",
                             "seconds_per_step_extrapolated": round(dd_step, 1),
                             "sample": f"oracle.decode_decompressed (fp64, K and V expanded per head) on sequence "
                                       f"{b} ({int(inp.seqlens[b])} tokens), {heads_done} of 128 heads, "
                                       f"in {dd:.1f}s"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--extra", default="c1,c2,c3max,c4,c5",
                    help="comma list of other workloads timed for the report (c1,c2,c3max,c4,c5 or none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill chunk leg")
    ap.add_argument("--no-resident", action="store_true", help="skip the leg with the cache held in L2")
    ap.add_argument("--no-redo", action="store_true", help="skip the softmax-redo leg")
    ap.add_argument("--no-mxfp8", action="store_true", help="skip the MXFP8-cache leg")
    ap.add_argument("--no-append", action="store_true", help="skip the cache-append leg")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT_NAME"),
                    help="write a kernel-trace summary (rocprofv3 --kernel-trace --stats csv folder) to profiles/")
    ap.add_argument("--trace-title", default="", help="title line of --summarize-trace")
    ap.add_argument("--pmc-run", nargs="?", const="decode", default=None, choices=sorted(set(TRAFFIC) | {"c1", "c2", "resident"}),
                    help="only run launches of one kernel family (default decode) and the calibration copy "
                         "(target of rocprofv3 --pmc passes)")
    ap.add_argument("--settle", type=float, default=0.0,
                    help="with --pmc-run: seconds of untimed calls after the warm-up, before the counted ones")
    ap.add_argument("--flush", action="store_true",
                    help="with --pmc-run: flush L2 and the last-level cache before every call")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from the FETCH_SIZE and WRITE_SIZE pass output folders")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="write the decode kernel's cycle and instruction attribution from counter pass folders")
    ap.add_argument("--counters-kind", default="decode", choices=sorted(COUNTER_FILES),
                    help="kernel family of --summarize-counters (the --pmc-run the passes ran)")
    ap.add_argument("--summarize-clock", nargs="+", metavar="KIND=DIR",
                    help="write the engine clock and MFMA occupancy summary from counter passes "
                         "(SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE) over "
                         "--pmc-run KIND")
    ap.add_argument("--sweep-splits", metavar="WORKLOADS",
                    help="time the paged decode of these workloads (comma list) over --sweep-values num_splits "
                         "and write the table to profiles/")
    ap.add_argument("--sweep-values", default="0,16,32,64,128,256",
                    help="num_splits values of --sweep-splits (0 = the library's choice)")
    ap.add_argument("--pmc-kind", default="decode", choices=sorted(TRAFFIC),
                    help="kernel family of --summarize-pmc")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="command lines recorded in the traffic summary (repeatable)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.pmc_command, args.pmc_kind)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.pmc_command, args.counters_kind)
        return
    if args.summarize_clock:
        summarize_clock([x.split("=", 1) for x in args.summarize_clock], args.pmc_command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.pmc_command, args.trace_title)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(sequences shard across GPUs without exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    if args.pmc_run:
        pmc_run(args.steps, args.warmup, args.pmc_run, args.settle, args.flush)
        return
    if args.sweep_splits:
        import torch
        import mla_latent_kv_04_amd as mla
        cmd = [f"python3 bench.py --sweep-splits {args.sweep_splits} --sweep-values {args.sweep_values} "
               f"--steps {args.steps}"]
        run_split_sweep(args.sweep_splits.split(","), [int(x) for x in args.sweep_values.split(",")], args.steps,
                        torch, mla, cmd)
        return

    import torch
    import mla_latent_kv_04_amd as mla
    from synth import make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.cuda.get_device_properties(0)
    log(f"[bench] device {dev.name} CUs={dev.multi_processor_count}")

    # ---- graded workload: batch 64, lengths U[1024, 32768]
    inp = _workload_from_synth("c3", torch)
    pool = _dev_bf16(inp.pool, torch)
    flush = _flusher(torch)
    r = run_paged(inp, pool, torch, mla, args.steps, args.warmup, flush=flush)
    ms = r["ms"]
    gbs = r["cache_bytes"] / (ms * 1e-3) / 1e9
    dec_ms = r["per"]["decode"]
    achieved = r["cache_bytes"] / (dec_ms * 1e-3) / 1e9
    stream = run_stream(inp, pool, torch, mla, args.steps, args.warmup)
    log(f"[bench] c3 stream ceiling: {stream}")
    log(f"[bench] c3 paged: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s; kernels us: "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in r["per"].items() if v > 0))

    resident = None
    if not args.no_resident:
        resident = run_cache_resident(inp, pool, torch, mla, args.steps, args.warmup, dec_ms)
        log(f"[bench] c3 with the cache in L2: {resident}")

    # fused step (absorb + paged + merge + up-proj) on the same inputs
    d_qc, d_qr = _dev_bf16(inp.q_c, torch), _dev_bf16(inp.q_r, torch)
    d_wuk, d_wuv = _dev_bf16(inp.w_uk, torch), _dev_bf16(inp.w_uv, torch)
    d_bt, d_sl = _dev_i32(inp.block_table, torch), _dev_i32(inp.seqlens, torch)
    fout = torch.empty(inp.batch, 1, 128, 128, dtype=torch.bfloat16, device="cuda")
    fparams = mla.make_params(inp.batch, 1, inp.max_blocks, inp.num_pages, inp.scale)
    fws = torch.empty(mla.workspace_size(fparams, fused=True), dtype=torch.uint8, device="cuda")
    fms, fper, fdist = _time_calls(lambda i: mla.decode(d_qc, d_qr, d_wuk, d_wuv, pool, d_bt, d_sl,
                                                        scale=inp.scale, out=fout, workspace=fws, want_lse=False),
                                   args.steps, args.warmup, torch, mla)
    log(f"[bench] c3 fused: {fms * 1e3:.1f} us/step; kernels us: "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in fper.items()))

    # ---- the redo path of the fixed-reference softmax, made to fire in every long range
    redo = None
    if not args.no_redo:
        redo = run_redo(inp, pool, torch, mla, args.steps, args.warmup, ms)
        log(f"[bench] c3 redo: {redo}")

    # ---- the same workload over its MXFP8 cache
    mx = None
    if not args.no_mxfp8:
        mx = mxfp8_row(inp, pool, torch, mla, args.steps, args.warmup, ms)
        log(f"[bench] c3 mxfp8: {mx}")

    # ---- other workloads (timing only; parity is in the tests)
    others = {}
    for name in [x for x in args.extra.split(",") if x and x != "none"]:
        oi = make_inputs(name, with_pool=False)
        layers = 60 if name == "c4" else 1
        opool = _device_pool(oi.num_pages * layers, oi.seed, torch)
        # the 60-layer cache cycles through 72 GB, its own rotation; the others are flushed
        orr = run_paged(oi, opool, torch, mla, max(args.steps, 20), 3, layers=layers,
                        pages_per_layer=oi.num_pages, flush=None if layers > 1 else flush)
        others[name] = other_row(oi, orr, layers)
        log(f"[bench] {name}: {others[name]}")
        del opool
        torch.cuda.empty_cache()

    # ---- cache append of the same step's new tokens (timed after the decodes: it writes
    # one row per sequence into the pool)
    app = None
    if not args.no_append:
        app = run_append(inp, pool, torch, mla, args.steps, args.warmup)
        log(f"[bench] c3 append: {app}")

    pre = None
    if not args.no_prefill:
        pre = run_prefill(torch, mla, max(args.steps // 5, 5), 2)
        log(f"[bench] prefill: {pre}")

    cpu = None
    if not args.no_cpu:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f}s ...")
        cpu = cpu_baseline(inp, args.cpu_seconds)
        log(f"[bench] cpu baseline: {cpu}")

    traffic = load_traffic()
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "paged MLA decode, batch 64, seq_len U[1024,32768] (seed 44, sum 1166687), "
                               "1 query token, 128 heads, latent 512 + rope 64 bf16, page 64, permuted pages",
                   "batch": inp.batch, "cached_tokens": r["tokens"], "pages": inp.num_pages,
                   "num_splits": mla.decode_num_workgroups(mla.make_params(inp.batch, 1, inp.max_blocks,
                                                                           inp.num_pages, inp.scale)),
                   "cache_bytes_per_step": r["cache_bytes"]},
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "kv_tokens_per_s": round(r["tokens"] / (ms * 1e-3), 1),
        "query_tokens_per_s": round(r["queries"] / (ms * 1e-3), 1),
        "timing_us": r["dist"],
        "kernels_us": {k: round(v * 1e3, 2) for k, v in r["per"].items()},
        "fused_us_per_step": round(fms * 1e3, 2),
        "fused_timing_us": fdist,
        "fused_kernels_us": {k: round(v * 1e3, 2) for k, v in fper.items()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic["fetch"] + traffic["write"]),
                     "traffic_split": traffic,
                     "kernel": "decode_kernel", "algorithmic_bytes_per_launch": r["cache_bytes"],
                     "measured_stream_ceiling_GBps": stream["GBps_median"],
                     "frac_of_measured_stream_ceiling": round(achieved / stream["GBps_median"], 4)},
        "stream_ceiling": stream,
        "cache_resident": resident,
        "softmax_redo": redo,
        "cpu_baseline": cpu,
        "other_workloads": others,
        "cache_append": app,
        "prefill": pre,
        "mxfp8_cache": mx,
    }
    print(json.dumps(line), flush=True)


def kernel_source_hash(kind="decode"):
    """sha256 over the code of the sources a kernel family is compiled from (comments
    and blank space left out): counter readings taken with other code do not describe
    the kernels being timed."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in TRAFFIC[kind]["sources"]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def load_traffic(kind="decode"):
    """HBM bytes per launch (or per call, for the append) from the committed counter
    summary, or None when it is missing or was taken on other kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles", TRAFFIC[kind]["file"])) as f:
            kv = dict(line.split(":", 1) for line in f if line.startswith(("source_sha256:", "fetch_bytes_per_launch:",
                                                                             "write_bytes_per_launch:")))
    except OSError:
        return None
    if kv.get("source_sha256", "").strip() != kernel_source_hash(kind):
        return None
    return {"fetch": float(kv["fetch_bytes_per_launch"]), "write": float(kv["write_bytes_per_launch"])}


def _copy_for_calibration(torch):
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def pmc_run(steps, warmup, kind="decode", settle=0.0, flush=False):
    """Workload for the rocprofv3 --pmc passes and kernel traces: `warmup + steps` launches
    of one kernel family (decode: the batch-64 paged decode; c1, c2, c5: the paged decode
    of those workloads; resident: the batch-64 decode with every page mapped onto the pool's
    first 32 (held in L2); mxfp8: the batch-64 decode over the MXFP8 cache; append: the
    64-token cache append; prefill: the 8 x 4096-token prompt), then one device copy of
    COPY_BYTES bytes whose counter readings calibrate the kernels'.  settle: seconds of
    further untimed calls after the warm-up; flush: evict the caches before every call."""
    import torch
    import mla_latent_kv_04_amd as mla
    if kind == "decode":
        inp = _workload_from_synth("c3", torch, with_host_pool=False)
        pool = _device_pool(inp.num_pages, inp.seed, torch)
        qa = torch.randn((inp.batch, 1, 128, 512), device="cuda").to(torch.bfloat16)
        qr = torch.randn((inp.batch, 1, 128, 64), device="cuda").to(torch.bfloat16)
        bt, sl = _dev_i32(inp.block_table, torch), _dev_i32(inp.seqlens, torch)
        call = lambda: mla.decode_paged(qa, qr, pool, bt, sl, scale=inp.scale)
    elif kind == "resident":
        inp = _workload_from_synth("c3", torch, with_host_pool=False)
        pool = _device_pool(inp.num_pages, inp.seed, torch)
        qa = torch.randn((inp.batch, 1, 128, 512), device="cuda").to(torch.bfloat16)
        qr = torch.randn((inp.batch, 1, 128, 64), device="cuda").to(torch.bfloat16)
        bt = _dev_i32((inp.block_table.astype(np.int64) % 32).astype(np.int32), torch)
        sl = _dev_i32(inp.seqlens, torch)
        call = lambda: mla.decode_paged(qa, qr, pool, bt, sl, scale=inp.scale)
    elif kind in ("c1", "c2", "c5"):
        inp = _workload_from_synth(kind, torch, with_host_pool=False)
        pool = _device_pool(inp.num_pages, inp.seed, torch)
        qa = torch.randn((inp.batch, inp.s_q, 128, 512), device="cuda").to(torch.bfloat16)
        qr = torch.randn((inp.batch, inp.s_q, 128, 64), device="cuda").to(torch.bfloat16)
        bt, sl = _dev_i32(inp.block_table, torch), _dev_i32(inp.seqlens, torch)
        call = lambda: mla.decode_paged(qa, qr, pool, bt, sl, scale=inp.scale)
    elif kind == "mxfp8":
        inp = _workload_from_synth("c3", torch, with_host_pool=False)
        pool8 = mla.quantize_kv_mxfp8(_device_pool(inp.num_pages, inp.seed, torch))
        qa = torch.randn((inp.batch, 1, 128, 512), device="cuda").to(torch.bfloat16)
        qr = torch.randn((inp.batch, 1, 128, 64), device="cuda").to(torch.bfloat16)
        bt, sl = _dev_i32(inp.block_table, torch), _dev_i32(inp.seqlens, torch)
        call = lambda: mla.decode_paged_mxfp8(qa, qr, pool8, bt, sl, scale=inp.scale)
    elif kind == "append":
        from synth import make_append_inputs
        inp = _workload_from_synth("c3", torch, with_host_pool=False)
        pool = _device_pool(inp.num_pages, inp.seed, torch)
        x_bits, w_bits = make_append_inputs(80, inp.batch, inp.s_q)
        x, w_a = _dev_bf16(x_bits, torch), _dev_bf16(w_bits, torch)
        table = mla.rope_table(131072)
        bt, sl = _dev_i32(inp.block_table, torch), _dev_i32(inp.seqlens, torch)
        call = lambda: mla.append_kv(x, w_a, table, pool, bt, sl)
    elif kind == "prefill":
        from synth import make_custom
        B, L = 8, 4096
        base = make_custom(102, B, 1, [L] * B)
        q_c = torch.randn((B, L, 128, 128), device="cuda").to(torch.bfloat16)
        q_r = torch.randn((B, L, 128, 64), device="cuda").to(torch.bfloat16)
        args = (q_c, q_r, _dev_bf16(base.w_uk, torch), _dev_bf16(base.w_uv, torch), _dev_bf16(base.pool, torch),
                _dev_i32(base.block_table, torch), _dev_i32(base.seqlens, torch))
        call = lambda: mla.prefill(*args, scale=base.scale)
    else:
        raise SystemExit(f"unknown --pmc-run kind {kind!r}")
    if flush:
        # every call HBM-cold: the caches are flushed before it (the flush kernels show in a trace)
        flusher, plain = _flusher(torch), call

        def call():
            flusher()
            plain()
    for _ in range(warmup):
        call()
    # keep calling until the clock has settled under the power cap (the timed legs of the
    # report do the same before they time anything)
    t_end = time.perf_counter() + settle
    while time.perf_counter() < t_end:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    # marks the start of the steady launches (a power or clock sampler waits for it)
    log(f"[bench] pmc run ({kind}): warm-up done, {steps} calls follow")
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    _copy_for_calibration(torch)
    log(f"[bench] pmc run ({kind}): {warmup + steps} calls, copy of {COPY_BYTES} B")


def _csv_files(run_dir, kind):
    """rocprofv3 csv outputs of one kind under a run folder, plain or gzip-compressed."""
    import glob
    return sorted(glob.glob(os.path.join(run_dir, "**", f"*{kind}.csv"), recursive=True)
                  + glob.glob(os.path.join(run_dir, "**", f"*{kind}.csv.gz"), recursive=True))


def _open_text(path):
    import gzip
    return gzip.open(path, "rt") if path.endswith(".gz") else open(path)


def _pmc_per_dispatch(run_dir, counter):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 csv run."""
    import csv
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    for path in _csv_files(run_dir, "counter_collection"):
        with _open_text(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in vals.items()}


def _prefill_algorithmic_bytes():
    """HBM bytes the prefill attention kernel must move once (8 x 4096 tokens, 128 heads):
    expanded K and V read, q_c and q_R read, the output and lse written, k_R read."""
    B, L, M = 8, 4096, 4096
    return (2 * B * L * 128 * 128 * 2 + B * M * 128 * 192 * 2 + B * M * 128 * 128 * 2 + B * M * 128 * 4
            + B * L * 64 * 2)


COUNTER_FILES = {
    "decode": ("decode_kernel_c3_b64_counters.md", "decode_kernel",
               "paged MLA decode, batch 64, seq_len U[1024,32768]"),
    "mxfp8": ("decode_kernel_mxfp8_c3_b64_counters.md", "decode_kernel<true>",
              "paged MLA decode over the MXFP8 cache, batch 64, seq_len U[1024,32768]"),
}


def _c3_tiles():
    from synth import make_inputs
    inp = make_inputs("c3", with_pool=False)
    return int(((inp.seqlens.astype(np.int64) + 31) // 32).sum())


def summarize_counters(run_dirs, command, kind="decode"):
    """Writes the attribution summary of the decode kernel from rocprofv3 --pmc passes over
    `bench.py --pmc-run KIND` (decode: the bf16 cache, mxfp8: the MXFP8 cache): every counter
    averaged over the kernel's launches (the first, cold launch left out), then per tile per
    wave (instruction counts) and as shares of the waves' cycles (SQ_WAVE_CYCLES; the SQ cycle
    counters share its quad-cycle unit)."""
    out_name, kernel, what = COUNTER_FILES[kind]
    import csv
    vals = {}
    for d in run_dirs:
        names = set()
        for path in _csv_files(d, "counter_collection"):
            with _open_text(path) as f:
                for r in csv.DictReader(f):
                    names.add(r["Counter_Name"])
        for name in names:
            per = _pmc_per_dispatch(d, name)
            v = [x for k, xs in per.items() if kernel + "<" in k or kernel + "(" in k for x in xs]
            if v:
                vals.setdefault(name, []).append(sum(v[1:]) / max(len(v) - 1, 1) if len(v) > 1 else v[0])
    avg = {k: float(np.mean(v)) for k, v in vals.items()}
    tiles = _c3_tiles()
    wave_tiles = 4 * tiles
    lines = [
        f"# Cycle and instruction attribution of {kernel}: {what}",
        "",
        f"rocprofv3 counter passes (one per line, at most 8 SQ counters each) over `python3 bench.py --pmc-run "
        f"{kind}`, run from /tmp:",
        "",
        "```",
        *command,
        "```",
        "",
        f"Values are per launch of {kernel} (the first launch of each pass left out). The workload has "
        f"{tiles} tiles of 32 tokens; each is processed by all four waves of its workgroup, so per-tile-per-wave "
        f"figures divide by {wave_tiles}. Cycle counters are shares of SQ_WAVE_CYCLES (the SQ counts wave cycles "
        "in quad-cycle units, the same unit for all of them); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
        "(GRBM_GUI_ACTIVE / 8 dies x 1024 SIMDs).",
        "",
        "| counter | per launch | per tile per wave | share of wave cycles |",
        "|---|---|---|---|",
    ]
    wc = avg.get("SQ_WAVE_CYCLES")
    for k in sorted(avg):
        share = f"{avg[k] / wc:.3f}" if wc and (("CYCLES" in k or k.startswith(("SQ_WAIT", "SQ_ACTIVE", "SQ_BUSY")))
                                                and k.startswith("SQ_")) else ""
        lines.append(f"| {k} | {avg[k]:.4g} | {avg[k] / wave_tiles:.2f} | {share} |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (avg["GRBM_GUI_ACTIVE"] / 8 * 1024)
        lines += ["", f"MFMA busy share of the launch's cycles: {busy:.3f}."]
    lines += ["", f"source_sha256: {kernel_source_hash('decode')}", ""]
    path = os.path.join(ROOT, "profiles", out_name)
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"[bench] wrote {path}")


CLOCK_FILE = "mfma_busy_clock_decode_c3_prefill_b8_4096.md"
CLOCK_KINDS = {
    "decode": ("decode_kernel", "decode_kernel<false>: bf16 cache, batch 64 (c3)"),
    "resident": ("decode_kernel", "decode_kernel<false>: the same step with its pages held in L2"),
    "mxfp8": ("decode_kernel", "decode_kernel<true>: MXFP8 cache, batch 64 (c3)"),
    "prefill": ("prefill_attention_kernel", "prefill_attention_kernel: 8 x 4096 prompt"),
}


def summarize_clock(kind_dirs, command):
    """Writes the engine clock and matrix-pipe occupancy of the main kernel of each pass, per
    launch (the first launch of a pass left out): clock = GRBM_GUI_ACTIVE / 8 dies / launch
    duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8);
    wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES."""
    import csv
    rows_out = []
    for kind, d in kind_dirs:
        kern, label = CLOCK_KINDS[kind]
        per = {}
        for path in _csv_files(d, "counter_collection"):
            with _open_text(path) as f:
                for r in csv.DictReader(f):
                    if kern + "<" not in r["Kernel_Name"] and kern + "(" not in r["Kernel_Name"]:
                        continue
                    e = per.setdefault(int(r["Dispatch_Id"]), {"dur": (int(r["End_Timestamp"])
                                                                      - int(r["Start_Timestamp"])) * 1e-9})
                    e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        launches = [per[k] for k in sorted(per)][1:]
        if not launches:
            raise SystemExit(f"summarize-clock: no {kern} dispatches in {d}")
        dur = [x["dur"] * 1e6 for x in launches]
        clk = [x["GRBM_GUI_ACTIVE"] / 8 / x["dur"] / 1e9 for x in launches]
        busy = [x["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (x["GRBM_GUI_ACTIVE"] / 8) for x in launches]
        wait = [x["SQ_WAIT_INST_ANY"] / x["SQ_WAVE_CYCLES"] for x in launches]
        rng = lambda v, f: f"{f.format(min(v))}–{f.format(max(v))}"
        rows_out.append(f"| {label} | {len(launches)} | {rng(dur, '{:.0f}')} | {rng(clk, '{:.2f}')} | "
                        f"{rng(busy, '{:.3f}')} | {rng(wait, '{:.3f}')} |")
    lines = ["# Engine clock and MFMA occupancy per launch: decode (c3: bf16 cache, pages in L2, MXFP8 cache) "
             "and prefill attention (8 x 4096)", "",
             "rocprofv3 counter passes, one per kernel family, run from /tmp (`<repo>` is the repository root):", "",
             "```", *command, "```", "",
             "Per launch of the family's main kernel (the first launch of each pass left out): clock = "
             "GRBM_GUI_ACTIVE / 8 dies / launch duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / "
             "(GRBM_GUI_ACTIVE / 8) (a v_mfma_f32_32x32x16_bf16 keeps its SIMD's matrix pipe busy 32 cycles); "
             "wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave cycles spent waiting on a dependency). Under --pmc "
             "the launches are serialised one by one, so their durations spread more than the benchmark's.", "",
             "| kernel | launches | duration us | clock GHz | MFMA busy | wait |", "|---|---|---|---|---|---|",
             *rows_out, "",
             f"source_sha256 (decode sources): {kernel_source_hash('decode')}",
             f"source_sha256 (prefill sources): {kernel_source_hash('prefill')}", ""]
    path = os.path.join(ROOT, "profiles", CLOCK_FILE)
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"[bench] wrote {path}")


def summarize_trace(trace_dir, out_name, command, title):
    """Writes a kernel-trace summary to profiles/OUT_NAME: per kernel, the number of dispatches
    and their duration (average, median, min, max) from a rocprofv3 --kernel-trace csv folder."""
    import csv
    import statistics
    rows = []
    for path in _csv_files(trace_dir, "kernel_trace"):
        with _open_text(path) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"summarize-trace: no kernel_trace.csv under {trace_dir}")
    by = {}
    for r in rows:
        name = r["Kernel_Name"]
        short = name.replace("(anonymous namespace)::", "").replace("void ", "").replace("mla::", "").split("(")[0]
        by.setdefault(short, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    total = sum(sum(v) for v in by.values())
    lines = [f"# Kernel trace: {title}", "", "Command (run from /tmp; `<repo>` is the repository root):", "", "```",
             *command, "```", "",
             "| kernel | dispatches | avg us | median us | min us | max us | share of traced kernel time |",
             "|---|---|---|---|---|---|---|"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {len(v)} | {statistics.mean(v):.1f} | {statistics.median(v):.1f} | {min(v):.1f} | "
                     f"{max(v):.1f} | {sum(v) / total:.1%} |")
    lines += ["", f"source_sha256 (decode sources): {kernel_source_hash('decode')}", ""]
    path = os.path.join(ROOT, "profiles", out_name)
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"[bench] wrote {path}")


def summarize_pmc(fetch_dir, write_dir, command, kind="decode"):
    """Writes the traffic summary of a kernel family: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of its kernels, each scaled by COPY_BYTES over what the same counter reads
    for the copy (the copy fetches and writes COPY_BYTES exactly).  For a family of two
    kernels per call (the append) the per-call bytes are the sum of their averages."""
    t = TRAFFIC[kind]
    out = {}
    per_kernel = {}
    for name, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _pmc_per_dispatch(run_dir, name)
        # the calibration copy is the runtime's blit kernel (torch's dtype conversions are "copy" kernels too)
        cop = [v for k, vs in per.items() if "rocclr_copyBuffer" in k for v in vs]
        if not cop:
            raise SystemExit(f"summarize-pmc: no copy dispatches with {name} in {run_dir}: {list(per)}")
        cop_kib = max(cop)
        factor = COPY_BYTES / (cop_kib * 1024.0)
        total = 0.0
        for kern in t["kernels"]:
            vals = [v for k, vs in per.items() if (kern + "(" in k or kern + "<" in k) for v in vs]
            if not vals:
                raise SystemExit(f"summarize-pmc: no {kern} dispatches with {name} in {run_dir}: {list(per)}")
            kib = sum(vals[1:]) / max(len(vals) - 1, 1) if len(vals) > 1 else vals[0]   # first launch is cold
            per_kernel.setdefault(kern, {})[name] = (kib, len(vals))
            total += kib
        out[name] = {"kib": total, "copy_kib": cop_kib, "factor": factor, "bytes": total * 1024.0 * factor}
    if kind == "decode":
        alg, alg_note = 1166687 * ROW_BYTES, "cache rows read once"
    elif kind == "mxfp8":
        alg, alg_note = 1166687 * MXFP8_ROW_BYTES, "MXFP8 cache rows read once"
    elif kind == "c5":
        alg, alg_note = 4 * 131072 * ROW_BYTES, "cache rows read once (both queries of a sequence share them)"
    elif kind == "append":
        alg, alg_note = append_algorithmic_bytes(64), "W_A, x, rows written, table rows, table entries and lengths"
    else:
        alg, alg_note = _prefill_algorithmic_bytes(), "expanded K and V, q_c and q_R read once, output and lse written"
    fetch, write = out["FETCH_SIZE"]["bytes"], out["WRITE_SIZE"]["bytes"]
    lines = [
        f"# HBM traffic of {t['title']}",
        "",
        f"Two rocprofv3 counter passes over `python3 bench.py --pmc-run {kind}` ({kind} calls, then a",
        f"device copy of {COPY_BYTES} B that calibrates the counters), run from /tmp:",
        "",
        "```",
        *command,
        "```",
        "",
        "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | dispatches |",
        "|---|---|---|---|",
        *[f"| {k} | {v['FETCH_SIZE'][0]:.0f} | {v['WRITE_SIZE'][0]:.0f} | {v['FETCH_SIZE'][1]} |"
          for k, v in per_kernel.items()],
        "",
        "| counter | KiB per launch | copy KiB | calibration (copy bytes / copy reading) | bytes per launch |",
        "|---|---|---|---|---|",
        *[f"| {n} | {v['kib']:.0f} | {v['copy_kib']:.0f} | {v['factor']:.4f} | {v['bytes']:.0f} |"
          for n, v in out.items()],
        "",
        f"Algorithmic bytes per launch ({alg_note}): {alg}; fetched / algorithmic = {fetch / alg:.4f};"
        f" fetched + written / algorithmic = {(fetch + write) / alg:.4f}.",
        "",
        f"source_sha256: {kernel_source_hash(kind)}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        "",
    ]
    path = os.path.join(ROOT, "profiles", t["file"])
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"[bench] wrote {path}: fetch {fetch:.0f} B, write {write:.0f} B per launch")


if __name__ == "__main__":
    main()
