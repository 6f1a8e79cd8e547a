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
