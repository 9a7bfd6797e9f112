"""The allocation-free paged decode (mla_decode_paged_noalloc) against mla_decode_paged:
same parameters, same kernels and split plan, so the outputs must agree bit for bit; and
against the fp64 oracle at the output tolerance.  Two calls in a row share the library's
device array, the second with a smaller input (fewer sequences and workgroups), so a
stale value left by the first call would show."""

import ctypes

import numpy as np
import pytest

import oracle
from synth import make_custom

from ._gpu import LSE_ATOL, absorbed_inputs, assert_close, dev_bf16, host_bits, host_f64, require_gpu, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _noalloc(inp, d, qa, num_splits):
    import torch
    import mla_latent_kv_04_amd as mla
    from mla_latent_kv_04_amd import _lib
    lib = _lib.load()
    B, s_q = inp.batch, inp.s_q
    out = torch.full((B, s_q, 128, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, s_q, 128), float("nan"), dtype=torch.float32, device="cuda")
    p = mla.make_params(B, s_q, inp.max_blocks, inp.num_pages, inp.scale, num_splits)
    st = lib.mla_decode_paged_noalloc(
        ctypes.c_void_p(qa.data_ptr()), ctypes.c_void_p(d["q_r"].data_ptr()), ctypes.c_void_p(d["pool"].data_ptr()),
        ctypes.c_void_p(d["bt"].data_ptr()), ctypes.c_void_p(d["sl"].data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), ctypes.byref(p),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st, "mla_decode_paged_noalloc")
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("num_splits", [0, 40])
def test_noalloc_matches_workspace_decode_twice(num_splits):
    import torch
    import mla_latent_kv_04_amd as mla
    rng = np.random.default_rng(90 + num_splits)
    # largest first, each later call smaller: 70 long sequences (the plan kernel; with the
    # library's own split the ranges are cut on the segment-aware cost line), 70 short ones,
    # then 3 sequences of two queries
    cases = [make_custom(93, 70, 1, [int(x) for x in rng.integers(1, 24000, size=70)], extra_blocks=1),
             make_custom(91, 70, 1, [int(x) for x in rng.integers(1, 3000, size=70)], extra_blocks=1),
             make_custom(92, 3, 2, [2, 65, 700], extra_blocks=1)]
    for inp in cases:
        print(f"[case] noalloc splits={num_splits} B={inp.batch} s_q={inp.s_q}", flush=True)
        d = upload(inp)
        qa_bits = absorbed_inputs(inp)
        qa = dev_bf16(qa_bits)
        got, got_lse = _noalloc(inp, d, qa, num_splits)
        ref, ref_lse = mla.decode_paged(qa, d["q_r"], d["pool"], d["bt"], d["sl"], scale=inp.scale,
                                        num_splits=num_splits)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(got), host_bits(ref))
        assert np.array_equal(got_lse.cpu().numpy().view(np.uint32), ref_lse.cpu().numpy().view(np.uint32))
        o_ol, o_lse = oracle.decode_absorbed(qa_bits, inp.q_r, inp.pool, inp.block_table, inp.seqlens, inp.s_q,
                                             inp.scale)
        assert_close(host_f64(got), o_ol, "out_latent")
        assert np.max(np.abs(got_lse.double().cpu().numpy() - o_lse)) <= LSE_ATOL
