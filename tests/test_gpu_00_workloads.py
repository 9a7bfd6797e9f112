"""GPU parity on the five named workloads at full size, every sequence checked.

Each workload runs in the launch configuration the benchmark times (one split-KV
workgroup per compute unit).  Two outputs are compared with the fp64 oracle:

* ``out_latent`` and ``lse`` of ``mla_decode_paged`` against the absorbed form
  fed the same bf16 q_abs (RNE of the exact q_c . W_UK), for every sequence and
  every query token, all 128 heads;
* ``out`` and ``lse`` of the fused ``mla_decode`` against the decompress
  definition (K = c . W_UK, V = c . W_UV expanded per head, standard softmax),
  for every sequence and query token, on a fixed sample of heads that covers
  both ends of each wave's 32-head block (the decompress oracle costs two
  512 x 128 expansions per head and token, so all heads at these lengths would
  take minutes).

The path-A vs path-B equivalence check of "撕开 DeepSeek MLA 源码" (sheratonhq.com,
section 4) is what the fused comparison extends to whole workloads.  Bar:
max|gpu - ref| <= 1e-2 max|ref| + 2e-3 per output tensor; lse within 2e-3 when
both sides use the same bf16 q_abs, within the derived bf16-rounding bound
against the unrounded definition."""

import numpy as np
import pytest

import oracle
from synth import make_inputs

from ._gpu import (LSE_ATOL, absorbed_inputs, assert_close, dev_bf16, dev_i32, host_bits, host_f64, require_gpu,
                   upload)

pytestmark = pytest.mark.gpu

# heads 0/31 and 32/63 are the ends of the first two waves' score blocks; 64 and 127
# the start of the third and the last head
HEADS = [0, 31, 32, 63, 64, 127]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    _CACHE.clear()


import mla_latent_kv_04_amd as mla  # noqa: E402

_CACHE = {}


def _workload(name):
    """Host inputs and their device copies, made once per module."""
    if name not in _CACHE:
        inp = make_inputs(name)
        print(f"[case] {name} seed={inp.seed} B={inp.batch} s_q={inp.s_q} tokens={int(inp.seqlens.sum())} "
              f"pages={inp.num_pages}", flush=True)
        _CACHE[name] = (inp, upload(inp))
    return _CACHE[name]


def _rows_f64(pool_bits, block_table, b, L):
    return oracle.bf16_bits_to_f64(oracle.gather_rows(pool_bits, block_table, b, L))


def lse_bound(qa_exact, rows, L, s_q, scale, heads):
    """[s_q, len(heads)] bound on |lse_gpu - lse_def| when the GPU scores with q_abs rounded
    to bf16: each score moves by at most scale * 2^-8 * sum_c |q_abs_c c_c| (one bf16 ulp of
    every q_abs value, which also covers the fp32 sum), so lse moves by at most the
    largest such shift over the visible tokens; plus LSE_ATOL for fp32 exp2/log2."""
    lat = np.abs(rows[:, :512])
    out = np.zeros((s_q, len(heads)))
    for i in range(s_q):
        n = L - s_q + i + 1
        out[i] = scale * 2.0 ** -8 * (np.abs(qa_exact[i][heads]) @ lat[:n].T).max(axis=1)
    return out + LSE_ATOL


def _check_paged(inp, qa_bits, ol, lse, batches, what):
    """out_latent and lse of the listed sequences against the absorbed oracle, one by one."""
    got_ol, got_lse = host_f64(ol), lse.double().cpu().numpy()
    refs, gots = [], []
    worst_lse = 0.0
    for b in batches:
        ref_ol, ref_lse = oracle.decode_absorbed(qa_bits, inp.q_r, inp.pool, inp.block_table, inp.seqlens,
                                                 inp.s_q, inp.scale, batches=[b])
        refs.append(ref_ol)
        gots.append(got_ol[b:b + 1])
        worst_lse = max(worst_lse, float(np.max(np.abs(got_lse[b:b + 1] - ref_lse))))
    err = assert_close(np.concatenate(gots), np.concatenate(refs), f"{what} out_latent")
    print(f"[{what}] out_latent max err {err:.3e} over {len(batches)} sequences; lse max err {worst_lse:.3e}",
          flush=True)
    assert worst_lse <= LSE_ATOL, f"{what}: lse err {worst_lse:.3e} > {LSE_ATOL}"


def _check_fused(inp, out, lse, batches, what):
    """out and lse of the listed sequences (sampled heads) against the decompress definition."""
    got_out, got_lse = host_f64(out), lse.double().cpu().numpy()
    qa = oracle.absorb_q(inp.q_c, inp.w_uk)
    refs, gots = [], []
    for b in batches:
        ref, ref_lse = oracle.decode_decompressed(inp.q_c, inp.q_r, inp.w_uk, inp.w_uv, inp.pool, inp.block_table,
                                                  inp.seqlens, inp.s_q, inp.scale, batches=[b], heads=HEADS)
        refs.append(ref)
        gots.append(got_out[b:b + 1][:, :, HEADS])
        L = int(inp.seqlens[b])
        bound = lse_bound(qa[b], _rows_f64(inp.pool, inp.block_table, b, L), L, inp.s_q, inp.scale, HEADS)
        dl = np.abs(got_lse[b][:, HEADS] - ref_lse[0])
        assert np.all(dl <= bound), f"{what} seq {b}: lse err {float(dl.max()):.3e} beyond the derived bound"
    err = assert_close(np.concatenate(gots), np.concatenate(refs), f"{what} out")
    print(f"[{what}] out max err {err:.3e} over {len(batches)} sequences x heads {HEADS}", flush=True)


# ------------------------------------------------------------------ paged decode, every sequence

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_paged_every_sequence(name):
    inp, d = _workload(name)
    qa = absorbed_inputs(inp)
    ol, lse = mla.decode_paged(dev_bf16(qa), d["q_r"], d["pool"], d["bt"], d["sl"], scale=inp.scale)
    import torch
    torch.cuda.synchronize()
    _check_paged(inp, qa, ol, lse, list(range(inp.batch)), f"{name} paged")


# ------------------------------------------------------------------ fused step vs the decompress definition

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_fused_every_sequence(name):
    inp, d = _workload(name)
    out, lse = mla.decode(d["q_c"], d["q_r"], d["w_uk"], d["w_uv"], d["pool"], d["bt"], d["sl"], scale=inp.scale)
    import torch
    torch.cuda.synchronize()
    _check_fused(inp, out, lse, list(range(inp.batch)), f"{name} fused")


# ------------------------------------------------------------------ the 60-layer long-context cache

C4_LAYERS = 60


@pytest.fixture(scope="module")
def c4_pool():
    """The 60 layers' caches of the long-context workload in one 72 GB device pool (later
    layers at byte offsets beyond 2^36), drawn on the device from a seeded generator."""
    import torch
    _CACHE.clear()
    inp = make_inputs("c4")
    P = inp.num_pages
    print(f"[case] c4 (60 layers) seed={inp.seed} B={inp.batch} L={int(inp.seqlens[0])} pages/layer={P}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(inp.seed)
    pool = torch.empty((C4_LAYERS * P, 64, 576), dtype=torch.bfloat16, device="cuda")
    for i in range(C4_LAYERS):
        pool[i * P:(i + 1) * P].normal_(generator=g)
    yield inp, pool
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", [0, 37, C4_LAYERS - 1])
def test_c4_every_sequence(c4_pool, layer):
    """16 sequences x 65536 tokens of one layer, decoded as a model runs it (one call per
    layer on that layer's slice of the pool).  Every sequence's out_latent and lse (paged
    call) and out and lse (fused call, sampled heads) are checked against the oracle on
    host copies of exactly the pages that sequence reads."""
    import torch
    inp, pool = c4_pool
    P = inp.num_pages
    qa_bits = absorbed_inputs(inp)
    qa_exact = oracle.absorb_q(inp.q_c, inp.w_uk)
    d_qa, d_qr = dev_bf16(qa_bits), dev_bf16(inp.q_r)
    d_qc, d_wuk, d_wuv = dev_bf16(inp.q_c), dev_bf16(inp.w_uk), dev_bf16(inp.w_uv)
    d_bt, d_sl = dev_i32(inp.block_table), dev_i32(inp.seqlens)
    lp = pool[layer * P:(layer + 1) * P]
    ol, lse = mla.decode_paged(d_qa, d_qr, lp, d_bt, d_sl, scale=inp.scale)
    out, flse = mla.decode(d_qc, d_qr, d_wuk, d_wuv, lp, d_bt, d_sl, scale=inp.scale)
    torch.cuda.synchronize()
    got_ol, got_lse = host_f64(ol), lse.double().cpu().numpy()
    got_out, got_flse = host_f64(out), flse.double().cpu().numpy()
    e_ol = e_out = e_lse = 0.0
    for b in range(inp.batch):
        L = int(inp.seqlens[b])
        n = (L + 63) // 64
        pages = inp.block_table[b, :n].astype(np.int64)
        sub = host_bits(lp[torch.from_numpy(pages).cuda()])
        bt1 = np.arange(n, dtype=np.int32).reshape(1, n)
        sl1 = inp.seqlens[b:b + 1]
        ref_ol, ref_lse = oracle.decode_absorbed(qa_bits[b:b + 1], inp.q_r[b:b + 1], sub, bt1, sl1, 1, inp.scale)
        e_ol = max(e_ol, assert_close(got_ol[b:b + 1], ref_ol, f"out_latent layer {layer} seq {b}"))
        dl = float(np.max(np.abs(got_lse[b:b + 1] - ref_lse)))
        assert dl <= LSE_ATOL, f"layer {layer} seq {b}: lse err {dl:.3e}"
        e_lse = max(e_lse, dl)
        ref, ref_flse = oracle.decode_decompressed(inp.q_c[b:b + 1], inp.q_r[b:b + 1], inp.w_uk, inp.w_uv, sub, bt1,
                                                   sl1, 1, inp.scale, heads=HEADS)
        e_out = max(e_out, assert_close(got_out[b:b + 1][:, :, HEADS], ref, f"out layer {layer} seq {b}"))
        bound = lse_bound(qa_exact[b], _rows_f64(sub, bt1, 0, L), L, 1, inp.scale, HEADS)
        dfl = np.abs(got_flse[b][:, HEADS] - ref_flse[0])
        assert np.all(dfl <= bound), f"layer {layer} seq {b}: fused lse beyond the derived bound"
    print(f"[c4] layer {layer}: 16 sequences, out_latent err {e_ol:.3e}, lse err {e_lse:.3e}, "
          f"fused out err {e_out:.3e}", flush=True)
