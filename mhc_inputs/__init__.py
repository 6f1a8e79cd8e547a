"""Seeded synthetic inputs for the mHC residual-mixing path.

This module only draws random numbers and packs them into the dtypes the
method consumes (bf16 streams as uint16 bit patterns, fp32 mixes).  It holds
none of the method's arithmetic, so both the CPU oracle (``oracle/``) and the
HIP library consume the same arrays without sharing any computation.

Recipe (one generator per tensor, so adding a tensor never shifts another):
``numpy.random.default_rng([seed, cfg_id, tensor_id])`` draws float32
``standard_normal`` (or ``uniform``) values, scales them, and bf16 tensors are
rounded to nearest-even from those float32 values.

Workloads follow the shapes the pages name: HC is fixed at 4 and the 24-logit
projection is pre(4)+post(4)+comb(16) (FlashInfer mHC article, section 1);
H=4096 and H=7168 are the DeepSeek-V4 shapes the post kernel is specialised
for (same article, section 2.3) and H=127 is its non-multiple-of-8 case
(section 5.3).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HC = 4
MIX = HC * (2 + HC)  # 24 logits per token: pre(4) + post(4) + comb(16)

# Tensor ids: fixed per tensor name so that each draw has its own stream.
_TID = {
    "res": 1,
    "x": 2,
    "hc_fn": 3,
    "hc_base": 4,
    "post": 5,
    "comb_logits": 6,
    "logits": 7,
    "hc_scale": 8,
    "grad": 9,
    "d_out": 10,
    "dy": 11,
    "d_post": 12,
    "d_comb": 13,
    "dots": 14,
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, cfg: int, tensor: str) -> np.random.Generator:
    return np.random.default_rng([seed, cfg, _TID[tensor]])


def normal_f32(seed: int, cfg: int, tensor: str, shape, std: float) -> np.ndarray:
    g = _rng(seed, cfg, tensor)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def device_normal_bf16(seed: int, cfg: int, tensor: str, shape, device="cuda", std: float = 1.0):
    """A large seeded bf16 tensor drawn directly on the device (torch's generator, fp32
    normals rounded to bf16 nearest-even), for shapes too big to draw on the host.  The
    caller copies the rows it checks back to the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + cfg) * 1_000_003 + _TID[tensor])
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def device_normal_f32(seed: int, cfg: int, tensor: str, shape, device="cuda", std: float = 1.0):
    """A large seeded fp32 tensor drawn directly on the device (torch's generator), as
    device_normal_bf16 without the rounding."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + cfg) * 1_000_003 + _TID[tensor])
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def normal_bf16(seed: int, cfg: int, tensor: str, shape, std: float = 1.0) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, cfg, tensor, shape, std))


def uniform_f32(seed: int, cfg: int, tensor: str, shape, lo: float, hi: float) -> np.ndarray:
    g = _rng(seed, cfg, tensor)
    return g.uniform(lo, hi, size=shape).astype(np.float32)


@dataclass
class LayerInputs:
    """Inputs of one pre-map + post-map call (all host numpy arrays)."""

    T: int
    H: int
    res: np.ndarray  # [T, 4, H] uint16 (bf16 bits)
    x: np.ndarray  # [T, H] uint16 (bf16 bits), plays the sublayer output
    hc_fn: np.ndarray  # [24, 4H] float32
    hc_scale: np.ndarray  # [3] float32: pre, post, comb
    hc_base: np.ndarray  # [24] float32
    params: dict = field(default_factory=dict)


# Numeric parameters used by every layer workload: the defaults the FlashInfer
# mHC article lists for mhc_pre_big_fuse (section 3.2).
DEFAULT_PARAMS = dict(rms_eps=1e-6, pre_eps=1e-6, sinkhorn_eps=1e-6, post_mult=1.0, num_iters=20)

# Workloads.  cfg ids are stable: they seed the generators.
LAYER_SHAPES = {
    "tiny": (1, 16, 256),  # (cfg id, T, H): CPU-seconds full layer
    "post_h4096": (2, 4096, 4096),  # post-map only, persistent-kernel shape
    "layer_h7168": (3, 8192, 7168),  # full pre+post at large hidden size
    "decode_h7168": (5, 32, 7168),  # launch-latency bound decode
    "ragged_h1000": (6, 3000, 1000),  # H not a multiple of 32 / 64*8
    "tail_h127": (7, 40, 127),  # H % 8 != 0: scalar path
    "tail_h1001": (8, 24, 1001),  # H % 8 != 0, odd
}


def layer_inputs(T: int, H: int, cfg: int, seed: int = 0, *, hc_fn_std: float = 0.02,
                 base_std: float = 0.1, scale=(1.0, 1.0, 1.0)) -> LayerInputs:
    """Streams and x ~ N(0,1) in bf16, hc_fn ~ N(0, hc_fn_std), hc_base ~ N(0, base_std)."""
    res = normal_bf16(seed, cfg, "res", (T, HC, H))
    x = normal_bf16(seed, cfg, "x", (T, H))
    hc_fn = normal_f32(seed, cfg, "hc_fn", (MIX, HC * H), hc_fn_std)
    hc_base = normal_f32(seed, cfg, "hc_base", (MIX,), base_std)
    hc_scale = np.asarray(scale, dtype=np.float32)
    return LayerInputs(T, H, res, x, hc_fn, hc_scale, hc_base, dict(DEFAULT_PARAMS))


def f32_streams(T: int, H: int, cfg: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """FP32 residual streams [T, 4, H] ~ N(0, std): full fp32 values (almost none are bf16
    values), for the fp32-stream entry points."""
    return normal_f32(seed, cfg, "res", (T, HC, H), std)


def layer_inputs_f32s(T: int, H: int, cfg: int, seed: int = 0, *, hc_fn_std: float = 0.02,
                      base_std: float = 0.1, scale=(1.0, 1.0, 1.0)) -> LayerInputs:
    """layer_inputs with FP32 streams (res float32 [T, 4, H] ~ N(0,1)); x stays bf16."""
    res = f32_streams(T, H, cfg, seed)
    x = normal_bf16(seed, cfg, "x", (T, H))
    hc_fn = normal_f32(seed, cfg, "hc_fn", (MIX, HC * H), hc_fn_std)
    hc_base = normal_f32(seed, cfg, "hc_base", (MIX,), base_std)
    hc_scale = np.asarray(scale, dtype=np.float32)
    return LayerInputs(T, H, res, x, hc_fn, hc_scale, hc_base, dict(DEFAULT_PARAMS))


def named_layer(name: str, seed: int = 0) -> LayerInputs:
    cfg, T, H = LAYER_SHAPES[name]
    return layer_inputs(T, H, cfg, seed)


def post_inputs(T: int, H: int, cfg: int = 2, seed: int = 0):
    """Post-map inputs: res, x ~ N(0,1) bf16, post ~ U(0,2) fp32 and N(0,1) comb logits.

    The comb matrix itself is the Sinkhorn projection of ``comb_logits``; the
    caller computes it (row softmax of N(0,1) logits equals row-normalising
    exp(N(0,1)), so this is the same projection applied to those logits).
    """
    res = normal_bf16(seed, cfg, "res", (T, HC, H))
    x = normal_bf16(seed, cfg, "x", (T, H))
    post = uniform_f32(seed, cfg, "post", (T, HC), 0.0, 2.0)
    comb_logits = normal_f32(seed, cfg, "comb_logits", (T, HC, HC), 1.0)
    return res, x, post, comb_logits


SINKHORN_CFG = 4
SINKHORN_N = 1 << 20


def stress_logits() -> np.ndarray:
    """Eight fixed 4x4 logit matrices that stress the exp range (|logit| <= 8)."""
    m = np.zeros((8, HC, HC), dtype=np.float32)
    # 0: all zeros
    m[1] = np.where(np.eye(HC, dtype=bool), 8.0, -8.0)  # +8 diagonal, -8 elsewhere
    m[2, 0, :] = 8.0  # one row at +8 ...
    m[2, 3, :] = -8.0  # ... and one row at -8
    m[3] = -8.0
    m[3, [0, 1, 2, 3], [2, 0, 3, 1]] = 8.0  # permutation pattern at +8
    # 4: log of a doubly-stochastic matrix (a mix of two permutation matrices)
    d = 0.7 * np.eye(HC) + 0.3 * np.roll(np.eye(HC), 1, axis=1)
    m[4] = np.log(d + 1e-30).clip(-8.0, 8.0)
    a = np.array([3.0, -2.0, 0.5, -7.0])
    b = np.array([-1.0, 4.0, 2.5, -3.5])
    m[5] = (a[:, None] + b[None, :]).clip(-8.0, 8.0)  # separable a_i + b_j
    m[6] = np.where((np.arange(HC)[:, None] + np.arange(HC)[None, :]) % 2 == 0, 8.0, -8.0)
    m[7, 1, 2] = 8.0  # a single +8 entry
    return m.astype(np.float32)


def sinkhorn_logits(n: int = SINKHORN_N, seed: int = 0, cfg: int = SINKHORN_CFG) -> np.ndarray:
    """[n, 4, 4] fp32 logits ~ N(0, 2) clamped to [-8, 8]; entries 0..7 are stress_logits()."""
    lg = normal_f32(seed, cfg, "logits", (n, HC, HC), 2.0)
    np.clip(lg, -8.0, 8.0, out=lg)
    k = min(n, 8)
    lg[:k] = stress_logits()[:k]
    return lg


def sinkhorn_grad(n: int = SINKHORN_N, seed: int = 0, cfg: int = SINKHORN_CFG) -> np.ndarray:
    """[n, 4, 4] fp32 output gradients ~ N(0, 1) for the Sinkhorn reverse mode."""
    return normal_f32(seed, cfg, "grad", (n, HC, HC), 1.0)


def post_grad(T: int, H: int, cfg: int = 2, seed: int = 0) -> np.ndarray:
    """[T, 4, H] bf16 gradients ~ N(0, 1) of the post-map output."""
    return normal_bf16(seed, cfg, "d_out", (T, HC, H))


def pre_grads(T: int, H: int, cfg: int = 3, seed: int = 0):
    """Output gradients of the pre-map: dy [T, H] bf16 ~ N(0, 1), d_post [T, 4] and
    d_comb [T, 4, 4] fp32 ~ N(0, 1)."""
    dy = normal_bf16(seed, cfg, "dy", (T, H))
    d_post = normal_f32(seed, cfg, "d_post", (T, HC), 1.0)
    d_comb = normal_f32(seed, cfg, "d_comb", (T, HC, HC), 1.0)
    return dy, d_post, d_comb


def external_dots(T: int, H: int, cfg: int = 3, seed: int = 0, splits: int = 1, hc_fn_std: float = 0.02):
    """[splits, T, 24] fp32 partial dots with the spread of the layer workload's projection:
    the full dot of N(0, 1) streams with N(0, hc_fn_std) weights has std hc_fn_std * sqrt(4H),
    shared evenly between the splits."""
    std = hc_fn_std * (HC * H) ** 0.5 / splits ** 0.5
    return normal_f32(seed, cfg, "dots", (splits, T, MIX), std)


def algorithmic_bytes_pre(T: int, H: int) -> int:
    """Bytes the pre-map must move: res read, y written, post/comb written, hc_fn + scale/base read once."""
    return T * (8 * H + 2 * H + 16 + 64) + 384 * H + 108


def algorithmic_bytes_pre_bf16(T: int, H: int) -> int:
    """The pre-map with bf16 weights: as algorithmic_bytes_pre, with 192 H bytes of weights."""
    return T * (8 * H + 2 * H + 16 + 64) + 192 * H + 108


def algorithmic_bytes_pre_f32(T: int, H: int) -> int:
    """The pre-map over fp32 streams: 16 H bytes of streams read per token, the rest as
    algorithmic_bytes_pre."""
    return T * (16 * H + 2 * H + 16 + 64) + 384 * H + 108


def algorithmic_bytes_post_f32(T: int, H: int) -> int:
    """The post-map over fp32 streams: x (bf16) and res (fp32) read, 80 B of mixes, out (fp32) written."""
    return T * (2 * H + 16 * H + 80 + 16 * H)


def algorithmic_bytes_expand_f32(T: int, H: int) -> int:
    """Model entry onto fp32 streams: the hidden row read, 4 fp32 streams written."""
    return T * (2 * H + 16 * H)


def algorithmic_bytes_head_mean_f32(T: int, H: int) -> int:
    """Unweighted head over fp32 streams: 4 fp32 streams read, one bf16 row written."""
    return T * (16 * H + 2 * H)


def algorithmic_bytes_expand(T: int, H: int) -> int:
    """Model entry: the hidden row read, 4 streams written."""
    return T * (2 * H + 8 * H)


def algorithmic_bytes_head_mean(T: int, H: int) -> int:
    """Unweighted head: 4 streams read, one row written."""
    return T * (8 * H + 2 * H)


def algorithmic_bytes_head(T: int, H: int) -> int:
    """Weighted head: 4 streams read, one row written, 4 x 4H fp32 weights and 5 scalars read once."""
    return T * (8 * H + 2 * H) + 64 * H + 20


def algorithmic_bytes_post(T: int, H: int) -> int:
    """Bytes the post-map must move: x and res read, 80 B of mixes, out written."""
    return T * (2 * H + 8 * H + 80 + 8 * H)


def algorithmic_bytes_post_project(T: int, H: int) -> int:
    """The post-map fused with the next projection: the post-map's bytes, the next fp32
    weights read once, and 24 dots and a sum of squares written (100 B per token)."""
    return algorithmic_bytes_post(T, H) + 384 * H + T * 100


def algorithmic_bytes_pre_dots(T: int, H: int, splits: int = 1, sqrsum: bool = False) -> int:
    """Bytes the pre-map from external dots must move: the dot partials (and sum-of-squares
    partials) read, res read, y written, post/comb written, scale/base read once."""
    return T * (splits * 96 + (splits * 4 if sqrsum else 0) + 8 * H + 2 * H + 16 + 64) + 108


def algorithmic_bytes_sinkhorn(n: int) -> int:
    return n * 64 * 2


def algorithmic_bytes_post_backward(T: int, H: int) -> int:
    """Bytes the post-map reverse mode must move: d_out, x and res read, 80 B of mixes read,
    d_x and d_res written, 80 B of mix gradients written."""
    return T * (8 * H + 2 * H + 8 * H + 80 + 2 * H + 8 * H + 80)


def algorithmic_bytes_pre_dots_backward(T: int, H: int, splits: int = 1, sqrsum: bool = False) -> int:
    """Bytes the pre-map reverse mode (external dots) must move: dy, res, d_post, d_comb and the
    dot partials read, d_res and d_dot written (plus the sum-of-squares partial and its gradient)."""
    return T * (2 * H + 8 * H + 16 + 64 + splits * 96 + 8 * H + 96 + (splits * 4 + 4 if sqrsum else 0))


def algorithmic_bytes_pre_backward(T: int, H: int) -> int:
    """Bytes the whole pre-map's reverse mode must move: dy, res, d_post and d_comb read,
    d_res written, the fp32 weights read and their gradient written."""
    return T * (2 * H + 8 * H + 80 + 8 * H) + 2 * 384 * H + 108


def algorithmic_bytes_sinkhorn_backward(n: int) -> int:
    """grad and logits read, d_logits written: 64 B each per matrix."""
    return n * 64 * 3
