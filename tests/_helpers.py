"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np

from mhc_inputs import bf16_bits_to_f32

# Tolerances stated for the method: fp32 mixes within 1e-5 absolute; bf16
# outputs within 2^-7 * |ref| + 1e-3 of the unrounded fp64 reference.
MIX_ATOL = 1e-5
BF16_RTOL = 2.0 ** -7
BF16_ATOL = 1e-3


def to_dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev_f32(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def bits_of(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_of(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def assert_bf16_close(got_bits: np.ndarray, ref: np.ndarray, what: str):
    got = bf16_bits_to_f32(got_bits).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    tol = BF16_RTOL * np.abs(ref) + BF16_ATOL
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; max err {err.max():.3e}; "
                             f"first at {idx.tolist()}: got {got[bad][:5]} ref {ref[bad][:5]}")


def assert_f32_close(got: np.ndarray, ref: np.ndarray, what: str, atol: float = MIX_ATOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= atol)
    if bad.any():
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside {atol}; max err {err.max():.3e}")


def sample_tokens(T: int, n: int, seed: int = 123) -> np.ndarray:
    """First/last tokens, tile edges (multiples of 64 +/- 1) and random ones."""
    g = np.random.default_rng(seed)
    fixed = [0, 1, 15, 16, 63, 64, 65, 127, T // 2, T - 2, T - 1]
    pick = set(t for t in fixed if 0 <= t < T)
    while len(pick) < min(n, T):
        pick.add(int(g.integers(0, T)))
    return np.array(sorted(pick))


def oracle_threads() -> int:
    import os
    return max(1, min(os.cpu_count() or 1, 16))


# fp32 outputs of an fp32 multiply-add chain (the fp32-stream post-map): within 2^-21 of
# the sum of the absolute terms (five roundings of at most 2^-24 of it each, with margin).
F32_CHAIN_REL = 2.0 ** -21


def assert_f32_chain_close(got, ref, scale, what, rel: float = F32_CHAIN_REL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    tol = rel * np.asarray(scale, dtype=np.float64) + 1e-30
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {idx.tolist()}; "
                             f"max err/tol {(err / tol).max():.3e}")


def post_f32s_scale(x_bits, res, post, comb):
    """Sum of the absolute terms of each fp32-stream post-map output: |x post| + sum_o |res comb|."""
    xa = np.abs(bf16_bits_to_f32(x_bits).astype(np.float64))
    ra = np.abs(np.asarray(res, np.float64))
    pa = np.abs(np.asarray(post, np.float64)).reshape(ra.shape[0], 4)
    ca = np.abs(np.asarray(comb, np.float64)).reshape(ra.shape[0], 4, 4)
    return xa[:, None, :] * pa[:, :, None] + np.einsum("toh,ton->tnh", ra, ca)


def check_pre_all_tokens(inp, got, what, params=None, chunk=256, x=None, out=None):
    """Every token of a pre-map call (y, post, comb, pre) against the oracle, and with `x`/`out`
    the post-map that followed it.  The oracle runs on token chunks over threads (its ctypes
    calls release the GIL), comparing each chunk as it finishes, so memory stays bounded.
    fp32 streams (inp.res float32) are checked against the fp32-stream oracle; their post-map
    against the oracle on the kernel's own post and comb (fp32), within F32_CHAIN_REL."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    y, post, comb, pre = got
    p = dict(inp.params)
    if params:
        p.update(params)
    T = inp.res.shape[0]
    f32 = inp.res.dtype == np.float32
    pre_fn = oracle.pre_f32s if f32 else oracle.pre

    def one(t0):
        t1 = min(T, t0 + chunk)
        r = inp.res[t0:t1]
        ref = pre_fn(r, inp.hc_fn, inp.hc_scale, inp.hc_base, rms_eps=p["rms_eps"], pre_eps=p["pre_eps"],
                     sinkhorn_eps=p["sinkhorn_eps"], post_mult=p["post_mult"], num_iters=p["num_iters"])
        if pre is not None:
            assert_f32_close(pre[t0:t1], ref["pre"], f"{what} pre [{t0}:{t1}]")
        assert_f32_close(post[t0:t1], ref["post"], f"{what} post [{t0}:{t1}]")
        assert_f32_close(comb[t0:t1], ref["comb"], f"{what} comb [{t0}:{t1}]")
        assert_bf16_close(y[t0:t1], ref["y"], f"{what} y [{t0}:{t1}]")
        if out is not None and f32:
            gp, gc = post[t0:t1].astype(np.float64), comb[t0:t1].astype(np.float64)
            ref_out = oracle.post_f32s(x[t0:t1], r, gp, gc)
            assert_f32_chain_close(out[t0:t1], ref_out, post_f32s_scale(x[t0:t1], r, gp, gc),
                                   f"{what} out [{t0}:{t1}]")
        elif out is not None:
            ref_out = oracle.post(x[t0:t1], r, ref["post"], ref["comb"])
            assert_bf16_close(out[t0:t1], ref_out, f"{what} out [{t0}:{t1}]")

    with ThreadPoolExecutor(oracle_threads()) as ex:
        list(ex.map(one, range(0, T, chunk)))
