"""Helpers shared by the GPU tests: host <-> device copies of bf16 bit arrays and
the output tolerance.  No attention arithmetic lives here."""

from __future__ import annotations

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import mla_latent_kv_04_amd._lib as L
    L.load()      # fails loudly if the HIP library is missing


def dev_bf16(bits: np.ndarray):
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).cuda().view(torch.bfloat16)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_bits(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return oracle.bf16_bits_to_f64(host_bits(t))
    return t.double().cpu().numpy()


def tol(ref: np.ndarray) -> float:
    """max |gpu - ref| allowed for an output tensor (bf16 in, fp32 accumulate)."""
    return 1e-2 * float(np.max(np.abs(ref))) + 2e-3


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    err = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    t = tol(ref) if ref.size else 0.0
    assert err <= t, f"{what}: max err {err:.3e} > tol {t:.3e}"
    return err


# lse is fp32 on the GPU (exp2/log2 hardware approximations, fp32 sums) vs fp64 here.
LSE_ATOL = 2e-3


def lse_bound_for_rounded_q(inp, batches=None, heads=None):
    """Per (b, i, h) bound on how far lse can move when q_abs is rounded to bf16
    before the scores: each score moves by at most scale * 2^-8 * sum_c |q_abs_c c_c|
    (one bf16 ulp per factor, which also covers the fp32 sum), so lse moves by at
    most the largest such shift over the visible tokens; plus LSE_ATOL."""
    qa = oracle.absorb_q(inp.q_c, inp.w_uk)
    batches = range(inp.batch) if batches is None else batches
    heads = list(range(qa.shape[2])) if heads is None else heads
    out = np.zeros((len(batches), inp.s_q, len(heads)))
    for bi, b in enumerate(batches):
        L = int(inp.seqlens[b])
        rows = np.abs(oracle.bf16_bits_to_f64(oracle.gather_rows(inp.pool, inp.block_table, b, L))[:, :512])
        for i in range(inp.s_q):
            n = L - inp.s_q + i + 1
            m = (np.abs(qa[b, i][heads]) @ rows[:n].T).max(axis=1)
            out[bi, i] = inp.scale * 2.0 ** -8 * m
    return out + LSE_ATOL


def absorbed_inputs(inp):
    """The bf16 q_abs both sides use for paged-decode parity: RNE of the exact product."""
    return oracle.f64_to_bf16_bits(oracle.absorb_q(inp.q_c, inp.w_uk))


def upload(inp):
    return dict(q_c=dev_bf16(inp.q_c), q_r=dev_bf16(inp.q_r), w_uk=dev_bf16(inp.w_uk), w_uv=dev_bf16(inp.w_uv),
                pool=dev_bf16(inp.pool), bt=dev_i32(inp.block_table), sl=dev_i32(inp.seqlens))


# ---------------------------------------------------------------------------- bf16 results with a derived bound

U = 2.0 ** -24


def assert_bf16_match(got_bits, exact, err, what, max_frac=1e-2):
    """|gpu - exact| <= err + 2^-8 (|exact| + err) everywhere (err: the fp32 error bound of the
    computation, 2^-8 (|exact| + err): one bf16 rounding); bits equal to RNE(exact) but for max_frac."""
    ref_bits = oracle.f64_to_bf16_bits(exact)
    assert got_bits.shape == ref_bits.shape
    got = oracle.bf16_bits_to_f64(got_bits)
    bound = err + 2.0 ** -8 * (np.abs(exact) + err)
    over = np.abs(got - exact) > bound
    assert not over.any(), f"{what}: {int(over.sum())} elements beyond the bound, worst excess " \
        f"{float(np.max(np.abs(got - exact) - bound)):.3e}"
    frac = float(np.count_nonzero(got_bits != ref_bits)) / max(got_bits.size, 1)
    assert frac <= max_frac, f"{what}: {frac:.2%} of elements differ from the rounded oracle"
    return frac


# ---------------------------------------------------------------------------- cache-append rows


def rotation_err(a, b, cos, sin):
    """fp32 rounding bound of out = (a cos - b sin, a sin + b cos) on pairs (a, b)."""
    m = np.abs(a) * np.abs(cos) + np.abs(b) * np.abs(sin)
    n = np.abs(a) * np.abs(sin) + np.abs(b) * np.abs(cos)
    out = np.empty(np.broadcast_shapes(a.shape, cos.shape)[:-1] + (2 * a.shape[-1],))
    out[..., 0::2], out[..., 1::2] = 4 * U * m, 4 * U * n
    return out


def projection_err(x, w_a, table, positions):
    """Error bound E of the appended rows [..., 576] before their final rounding: the
    split fp32 sum of d products with 16x16x32 MFMAs (each output a chain of d/32
    four-term dot products, and the partial-sum additions) is within
    (d/32 + 64) * 2^-24 * sum|x w| of the exact sum; the k_R pairs add the fp32 rotation's
    error, two products and a sum per output."""
    d = x.shape[-1]
    S = np.abs(oracle.bf16_bits_to_f64(x)) @ np.abs(oracle.bf16_bits_to_f64(w_a))
    k = (d / 32 + 64) * U
    pre = np.abs(oracle.down_project(x, w_a))[..., 512:]
    t = np.asarray(table, dtype=np.float64)[np.asarray(positions)]
    cos, sin = np.abs(t[..., :32]), np.abs(t[..., 32:])
    E = k * S
    sa, sb = S[..., 512::2], S[..., 513::2]
    E[..., 512::2] = k * (sa * cos + sb * sin)
    E[..., 513::2] = k * (sa * sin + sb * cos)
    E[..., 512:] += rotation_err(pre[..., 0::2], pre[..., 1::2], cos, sin)
    return E
