"""Python binding over libmhc, the MI355X (gfx950) mHC residual-mixing library.

The functions below carry the names of the C entry points declared in
``include/mhc.h`` and only marshal arguments: shape/dtype checks, output and
workspace allocation through PyTorch, device pointers and the current HIP
stream.  Every step of the computation runs in the library's HIP kernels; if
``libmhc.so`` is missing or cannot be loaded, every call raises.

Shapes follow the FlashInfer mHC API ("FlashInfer mHC 模块深度解析", sections
2.2 and 3.1): leading token dimensions are flattened, HC is fixed at 4,
streams/activations are bf16 and mixing coefficients fp32.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

HC = 4
MIX = 24
LIB_PATH = Path(__file__).resolve().parent / "libmhc.so"

MHC_SUCCESS = 0
MHC_ERROR_INVALID_VALUE = 1
MHC_ERROR_WORKSPACE = 2
MHC_ERROR_LAUNCH = 3
MHC_PRE_FUSED_NOALLOC_MAX_BYTES = 16 << 20  # the static scratch of mhc_pre_fused_noalloc

_lib = None


class MHCError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libmhc.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m mhc_hyper_connection_amd.build`")
    L = ctypes.CDLL(str(LIB_PATH))
    P, I64, I32, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.mhc_abi_version.argtypes = []
    L.mhc_abi_version.restype = ctypes.c_int
    L.mhc_status_string.argtypes = [ctypes.c_int]
    L.mhc_status_string.restype = ctypes.c_char_p
    L.mhc_launch_plan.argtypes = [ctypes.c_char_p, I64, I64, I32, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                  ctypes.POINTER(I64)]
    L.mhc_launch_plan.restype = ctypes.c_int
    L.mhc_sinkhorn.argtypes = [P, P, I64, I32, F, P]
    L.mhc_sinkhorn.restype = ctypes.c_int
    L.mhc_pre_fused_workspace_bytes.argtypes = [I64, I64]
    L.mhc_pre_fused_workspace_bytes.restype = SZ
    L.mhc_pre_fused.argtypes = [P, P, P, P, I64, I64, F, F, F, F, I32, P, P, P, P, P, SZ, P]
    L.mhc_pre_fused.restype = ctypes.c_int
    L.mhc_post.argtypes = [P, P, P, P, I64, I64, P, P]
    L.mhc_post.restype = ctypes.c_int
    L.mhc_pre_from_dots.argtypes = [P, P, I32, P, P, P, I64, I64, F, F, F, F, F, I32, P, P, P, P, P]
    L.mhc_pre_from_dots.restype = ctypes.c_int
    L.mhc_sinkhorn_backward.argtypes = [P, P, I64, I32, F, P, P]
    L.mhc_sinkhorn_backward.restype = ctypes.c_int
    L.mhc_post_backward.argtypes = [P, P, P, P, P, I64, I64, P, P, P, P, P]
    L.mhc_post_backward.restype = ctypes.c_int
    L.mhc_pre_fused_bf16.argtypes = [P, P, P, P, I64, I64, F, F, F, F, I32, P, P, P, P, P, SZ, P]
    L.mhc_pre_fused_bf16.restype = ctypes.c_int
    L.mhc_pre_fused_noalloc.argtypes = [P, P, P, P, I64, I64, F, F, F, F, I32, P, P, P, P, P]
    L.mhc_pre_fused_noalloc.restype = ctypes.c_int
    L.mhc_pre_split_bytes.argtypes = [I64]
    L.mhc_pre_split_bytes.restype = SZ
    L.mhc_pre_split_weights.argtypes = [P, I64, P, SZ, P]
    L.mhc_pre_split_weights.restype = ctypes.c_int
    L.mhc_pre_fused_presplit.argtypes = [P, P, P, P, I64, I64, F, F, F, F, I32, P, P, P, P, P, SZ, P]
    L.mhc_pre_fused_presplit.restype = ctypes.c_int
    L.mhc_pre_fused_f32.argtypes = [P, P, P, P, I64, I64, F, F, F, F, I32, P, P, P, P, P, SZ, P]
    L.mhc_pre_fused_f32.restype = ctypes.c_int
    L.mhc_post_f32.argtypes = [P, P, P, P, I64, I64, P, P]
    L.mhc_post_f32.restype = ctypes.c_int
    L.mhc_expand_f32.argtypes = [P, I64, I64, P, P]
    L.mhc_expand_f32.restype = ctypes.c_int
    L.mhc_head_mean_f32.argtypes = [P, I64, I64, P, P]
    L.mhc_head_mean_f32.restype = ctypes.c_int
    L.mhc_expand.argtypes = [P, I64, I64, P, P]
    L.mhc_expand.restype = ctypes.c_int
    L.mhc_head_mean.argtypes = [P, I64, I64, P, P]
    L.mhc_head_mean.restype = ctypes.c_int
    L.mhc_head.argtypes = [P, P, P, P, I64, I64, F, F, P, P, P, SZ, P]
    L.mhc_head.restype = ctypes.c_int
    L.mhc_pre_fused_backward_workspace_bytes.argtypes = [I64, I64]
    L.mhc_pre_fused_backward_workspace_bytes.restype = SZ
    L.mhc_pre_fused_backward.argtypes = [P, P, P, P, P, P, P, I64, I64, F, F, F, F, I32, P, P, P, P, P, SZ, P]
    L.mhc_pre_fused_backward.restype = ctypes.c_int
    L.mhc_pre_backward_workspace_bytes.argtypes = [I64]
    L.mhc_pre_backward_workspace_bytes.restype = SZ
    L.mhc_pre_from_dots_backward.argtypes = [P, P, P, P, P, I32, P, P, P, I64, I64, F, F, F, F, F, I32, P, P, P, P,
                                             P, P, SZ, P]
    L.mhc_pre_from_dots_backward.restype = ctypes.c_int
    L.mhc_post_project_workspace_bytes.argtypes = [I64, I64]
    L.mhc_post_project_workspace_bytes.restype = SZ
    L.mhc_post_project.argtypes = [P, P, P, P, P, I64, I64, P, P, P, P, SZ, P]
    L.mhc_post_project.restype = ctypes.c_int
    L.mhc_post_pre_fused.argtypes = [P, P, P, P, P, P, P, I64, I64, F, F, F, F, I32, P, P, P, P, P, P, SZ, P]
    L.mhc_post_pre_fused.restype = ctypes.c_int
    L.mhc_set_exchange_test_hooks.argtypes = [I32, ctypes.c_uint32]
    L.mhc_set_exchange_test_hooks.restype = None
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().mhc_status_string(int(status)).decode()


def launch_plan(entry: str, T: int, H: int, vec8: bool = True) -> dict:
    """How `entry` (an entry point's name without the mhc_ prefix) splits a call at these
    sizes into launches of its token-parallel kernel (host arithmetic only, no GPU call)."""
    n, per, items = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("mhc_launch_plan", lib().mhc_launch_plan(entry.encode(), int(T), int(H), int(bool(vec8)),
                                                    ctypes.byref(n), ctypes.byref(per), ctypes.byref(items)))
    return {"launches": n.value, "tokens_per_launch": per.value, "max_items": items.value}


def abi_version() -> int:
    return lib().mhc_abi_version()


def _check(fn: str, status: int):
    if status != MHC_SUCCESS:
        raise MHCError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


def mhc_sinkhorn(logits: torch.Tensor, out: torch.Tensor | None = None, num_iters: int = 20,
                 eps: float = 1e-6) -> torch.Tensor:
    """Fixed-count Sinkhorn-Knopp projection of [..., 4, 4] fp32 logits (``out`` may be ``logits``)."""
    _need(logits, "logits", torch.float32)
    if logits.dim() < 2 or tuple(logits.shape[-2:]) != (HC, HC):
        raise ValueError(f"logits must be [..., 4, 4], got {tuple(logits.shape)}")
    if out is None:
        out = torch.empty_like(logits)
    _need(out, "out", torch.float32)
    if out.shape != logits.shape:
        raise ValueError("out must have the shape of logits")
    _same_device(logits, out)
    n = logits.numel() // (HC * HC)
    _check("mhc_sinkhorn", lib().mhc_sinkhorn(_ptr(logits), _ptr(out), n, int(num_iters), float(eps),
                                              _stream(logits.device)))
    return out


def mhc_pre_fused_workspace_bytes(T: int, H: int) -> int:
    return int(lib().mhc_pre_fused_workspace_bytes(int(T), int(H)))


def mhc_pre_fused(res: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                  rms_eps: float = 1e-6, pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6,
                  post_mult: float = 1.0, num_iters: int = 20, *, y=None, post=None, comb=None, pre=None,
                  return_pre: bool = False, workspace: torch.Tensor | None = None):
    """The pre-map.  res [..., 4, H] bf16 -> (y [..., H] bf16, post [..., 4] fp32, comb [..., 4, 4] fp32
    [, pre [..., 4] fp32]).  Outputs may be passed in (contiguous, right shape) to be written in place."""
    return _pre_fused("mhc_pre_fused", torch.float32, res, hc_fn, hc_scale, hc_base, rms_eps, pre_eps,
                      sinkhorn_eps, post_mult, num_iters, y, post, comb, pre, return_pre, workspace)


def mhc_pre_fused_bf16(res: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                       rms_eps: float = 1e-6, pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6,
                       post_mult: float = 1.0, num_iters: int = 20, *, y=None, post=None, comb=None, pre=None,
                       return_pre: bool = False, workspace: torch.Tensor | None = None):
    """:func:`mhc_pre_fused` with hc_fn [24, 4H] in bf16."""
    return _pre_fused("mhc_pre_fused_bf16", torch.bfloat16, res, hc_fn, hc_scale, hc_base, rms_eps, pre_eps,
                      sinkhorn_eps, post_mult, num_iters, y, post, comb, pre, return_pre, workspace)


def mhc_pre_fused_noalloc(res: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                          rms_eps: float = 1e-6, pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6,
                          post_mult: float = 1.0, num_iters: int = 20, *, y=None, post=None, comb=None, pre=None,
                          return_pre: bool = False):
    """:func:`mhc_pre_fused` with the library's static scratch instead of a workspace (for callers
    that cannot allocate device memory).  Outputs given here are written in place; ones left as
    None are allocated by this Python wrapper, not by the library."""
    return _pre_fused("mhc_pre_fused_noalloc", torch.float32, res, hc_fn, hc_scale, hc_base, rms_eps, pre_eps,
                      sinkhorn_eps, post_mult, num_iters, y, post, comb, pre, return_pre, None, noalloc=True)


def mhc_pre_split_bytes(H: int) -> int:
    return int(lib().mhc_pre_split_bytes(int(H)))


def mhc_pre_split_weights(hc_fn: torch.Tensor, workspace: torch.Tensor) -> torch.Tensor:
    """Split hc_fn [24, 4H] fp32 into the start of a pre-map workspace (uint8, device), for
    :func:`mhc_pre_fused_presplit` calls with the same weights.  Returns the workspace."""
    _need(hc_fn, "hc_fn", torch.float32)
    if hc_fn.dim() != 2 or hc_fn.shape[0] != MIX or hc_fn.shape[1] % HC != 0:
        raise ValueError(f"hc_fn must be [24, 4H], got {tuple(hc_fn.shape)}")
    H = hc_fn.shape[1] // HC
    _need(workspace, "workspace", torch.uint8)
    _same_device(hc_fn, workspace)
    _check("mhc_pre_split_weights", lib().mhc_pre_split_weights(_ptr(hc_fn), H, _ptr(workspace), workspace.numel(),
                                                                _stream(hc_fn.device)))
    return workspace


def mhc_pre_fused_presplit(res: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                           rms_eps: float = 1e-6, pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6,
                           post_mult: float = 1.0, num_iters: int = 20, *, workspace: torch.Tensor, y=None,
                           post=None, comb=None, pre=None, return_pre: bool = False):
    """:func:`mhc_pre_fused` on a workspace that :func:`mhc_pre_split_weights` prepared with
    this hc_fn (the two-pass form skips its weight split)."""
    return _pre_fused("mhc_pre_fused_presplit", torch.float32, res, hc_fn, hc_scale, hc_base, rms_eps, pre_eps,
                      sinkhorn_eps, post_mult, num_iters, y, post, comb, pre, return_pre, workspace)


def mhc_pre_fused_f32(res: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                      rms_eps: float = 1e-6, pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6,
                      post_mult: float = 1.0, num_iters: int = 20, *, y=None, post=None, comb=None, pre=None,
                      return_pre: bool = False, workspace: torch.Tensor | None = None):
    """:func:`mhc_pre_fused` over fp32 streams: res [..., 4, H] float32 -> (y [..., H] bf16,
    post [..., 4], comb [..., 4, 4] [, pre [..., 4]])."""
    return _pre_fused("mhc_pre_fused_f32", torch.float32, res, hc_fn, hc_scale, hc_base, rms_eps, pre_eps,
                      sinkhorn_eps, post_mult, num_iters, y, post, comb, pre, return_pre, workspace,
                      res_dtype=torch.float32)


def _pre_fused(name, fn_dtype, res, hc_fn, hc_scale, hc_base, rms_eps, pre_eps, sinkhorn_eps, post_mult, num_iters,
               y, post, comb, pre, return_pre, workspace, noalloc=False, res_dtype=torch.bfloat16):
    _need(res, "res", res_dtype)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"res must be [..., 4, H], got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(hc_fn, "hc_fn", fn_dtype)
    if tuple(hc_fn.shape) != (MIX, HC * H):
        raise ValueError(f"hc_fn must be [24, 4H] = [24, {HC * H}], got {tuple(hc_fn.shape)}")
    _need(hc_scale, "hc_scale", torch.float32)
    if tuple(hc_scale.shape) != (3,):
        raise ValueError("hc_scale must be [3] (pre, post, comb)")
    _need(hc_base, "hc_base", torch.float32)
    if tuple(hc_base.shape) != (MIX,):
        raise ValueError("hc_base must be [24]")
    dev = res.device
    if y is None:
        y = torch.empty(outer + (H,), dtype=torch.bfloat16, device=dev)
    if post is None:
        post = torch.empty(outer + (HC,), dtype=torch.float32, device=dev)
    if comb is None:
        comb = torch.empty(outer + (HC, HC), dtype=torch.float32, device=dev)
    if pre is None and return_pre:
        pre = torch.empty(outer + (HC,), dtype=torch.float32, device=dev)
    _need(y, "y", torch.bfloat16)
    _need(post, "post", torch.float32)
    _need(comb, "comb", torch.float32)
    if y.numel() != T * H or post.numel() != T * HC or comb.numel() != T * HC * HC:
        raise ValueError("output sizes do not match res")
    if pre is not None:
        _need(pre, "pre", torch.float32)
        if pre.numel() != T * HC:
            raise ValueError("pre must hold [T, 4] values")
    _same_device(res, hc_fn, hc_scale, hc_base, y, post, comb, pre)
    if noalloc:
        _check(name, getattr(lib(), name)(
            _ptr(res), _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), T, H, float(rms_eps), float(pre_eps),
            float(sinkhorn_eps), float(post_mult), int(num_iters), _ptr(y), _ptr(post), _ptr(comb), _ptr(pre),
            _stream(dev)))
        return (y, post, comb, pre) if return_pre else (y, post, comb)
    need = mhc_pre_fused_workspace_bytes(T, H)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    _check(name, getattr(lib(), name)(
        _ptr(res), _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), T, H, float(rms_eps), float(pre_eps),
        float(sinkhorn_eps), float(post_mult), int(num_iters), _ptr(y), _ptr(post), _ptr(comb), _ptr(pre),
        _ptr(workspace), workspace.numel(), _stream(dev)))
    if return_pre:
        return y, post, comb, pre
    return y, post, comb


def mhc_pre_from_dots(dot_mix: torch.Tensor, res: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                      sqrsum: torch.Tensor | None = None, k: float | None = None, rms_eps: float = 1e-6,
                      pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6, post_mult: float = 1.0,
                      num_iters: int = 20, *, y=None, post=None, comb=None, pre=None, return_pre: bool = False):
    """The pre-map from an external projection.  dot_mix [..., 24] or [splits, ..., 24] fp32, res [..., 4, H]
    bf16, sqrsum None (computed from res), [...] or [splits, ...] fp32, k the RMS denominator (default 4H)
    -> (y [..., H], post [..., 4], comb [..., 4, 4] [, pre [..., 4]])."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"res must be [..., 4, H], got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(dot_mix, "dot_mix", torch.float32)
    if tuple(dot_mix.shape) == outer + (MIX,):
        splits = 1
    elif dot_mix.dim() == len(outer) + 2 and tuple(dot_mix.shape[1:]) == outer + (MIX,):
        splits = dot_mix.shape[0]
    else:
        raise ValueError(f"dot_mix must be {outer + (MIX,)} or [splits, *{outer + (MIX,)}], "
                         f"got {tuple(dot_mix.shape)}")
    if sqrsum is not None:
        _need(sqrsum, "sqrsum", torch.float32)
        if sqrsum.numel() != splits * T:
            raise ValueError(f"sqrsum must hold [splits, T] = [{splits}, {T}] values")
    _need(hc_scale, "hc_scale", torch.float32)
    if tuple(hc_scale.shape) != (3,):
        raise ValueError("hc_scale must be [3] (pre, post, comb)")
    _need(hc_base, "hc_base", torch.float32)
    if tuple(hc_base.shape) != (MIX,):
        raise ValueError("hc_base must be [24]")
    dev = res.device
    if y is None:
        y = torch.empty(outer + (H,), dtype=torch.bfloat16, device=dev)
    if post is None:
        post = torch.empty(outer + (HC,), dtype=torch.float32, device=dev)
    if comb is None:
        comb = torch.empty(outer + (HC, HC), dtype=torch.float32, device=dev)
    if pre is None and return_pre:
        pre = torch.empty(outer + (HC,), dtype=torch.float32, device=dev)
    _need(y, "y", torch.bfloat16)
    _need(post, "post", torch.float32)
    _need(comb, "comb", torch.float32)
    if y.numel() != T * H or post.numel() != T * HC or comb.numel() != T * HC * HC:
        raise ValueError("output sizes do not match res")
    if pre is not None:
        _need(pre, "pre", torch.float32)
        if pre.numel() != T * HC:
            raise ValueError("pre must hold [T, 4] values")
    _same_device(dot_mix, sqrsum, res, hc_scale, hc_base, y, post, comb, pre)
    kk = float(HC * H) if k is None else float(k)
    _check("mhc_pre_from_dots", lib().mhc_pre_from_dots(
        _ptr(dot_mix), _ptr(sqrsum), int(splits), _ptr(res), _ptr(hc_scale), _ptr(hc_base), T, H, kk,
        float(rms_eps), float(pre_eps), float(sinkhorn_eps), float(post_mult), int(num_iters), _ptr(y), _ptr(post),
        _ptr(comb), _ptr(pre), _stream(dev)))
    if return_pre:
        return y, post, comb, pre
    return y, post, comb


def mhc_post(x: torch.Tensor, res: torch.Tensor, post: torch.Tensor, comb: torch.Tensor,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """The post-map.  x [..., H] bf16, res [..., 4, H] bf16, post [..., 4] or [..., 4, 1] fp32,
    comb [..., 4, 4] fp32 -> out [..., 4, H] bf16 (``out`` may be ``res`` for an in-place update)."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"residual.shape[-2] / HC must be 4, got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(x, "x", torch.bfloat16)
    if tuple(x.shape) != outer + (H,):
        raise ValueError(f"x must be {outer + (H,)}, got {tuple(x.shape)}")
    _need(post, "post", torch.float32)
    if tuple(post.shape) not in (outer + (HC,), outer + (HC, 1)):
        raise ValueError(f"post must be {outer + (HC,)} or {outer + (HC, 1)}, got {tuple(post.shape)}")
    _need(comb, "comb", torch.float32)
    if tuple(comb.shape) != outer + (HC, HC):
        raise ValueError(f"comb must be {outer + (HC, HC)}, got {tuple(comb.shape)}")
    if out is None:
        out = torch.empty_like(res)
    _need(out, "out", torch.bfloat16)
    if out.shape != res.shape:
        raise ValueError("out must have the shape of res")
    _same_device(x, res, post, comb, out)
    _check("mhc_post", lib().mhc_post(_ptr(x), _ptr(res), _ptr(post), _ptr(comb), T, H, _ptr(out),
                                      _stream(res.device)))
    return out


def mhc_post_f32(x: torch.Tensor, res: torch.Tensor, post: torch.Tensor, comb: torch.Tensor,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """:func:`mhc_post` over fp32 streams: x [..., H] bf16, res [..., 4, H] float32 ->
    out [..., 4, H] float32 (``out`` may be ``res``)."""
    _need(res, "res", torch.float32)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"res must be [..., 4, H], got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(x, "x", torch.bfloat16)
    if tuple(x.shape) != outer + (H,):
        raise ValueError(f"x must be {outer + (H,)}, got {tuple(x.shape)}")
    _need(post, "post", torch.float32)
    if tuple(post.shape) not in (outer + (HC,), outer + (HC, 1)):
        raise ValueError(f"post must be {outer + (HC,)} or {outer + (HC, 1)}, got {tuple(post.shape)}")
    _need(comb, "comb", torch.float32)
    if tuple(comb.shape) != outer + (HC, HC):
        raise ValueError(f"comb must be {outer + (HC, HC)}, got {tuple(comb.shape)}")
    if out is None:
        out = torch.empty_like(res)
    _need(out, "out", torch.float32)
    if out.shape != res.shape:
        raise ValueError("out must have the shape of res")
    _same_device(x, res, post, comb, out)
    _check("mhc_post_f32", lib().mhc_post_f32(_ptr(x), _ptr(res), _ptr(post), _ptr(comb), T, H, _ptr(out),
                                              _stream(res.device)))
    return out


def mhc_post_project_workspace_bytes(T: int, H: int) -> int:
    return int(lib().mhc_post_project_workspace_bytes(int(T), int(H)))


def mhc_post_project(x: torch.Tensor, res: torch.Tensor, post: torch.Tensor, comb: torch.Tensor,
                     hc_fn_next: torch.Tensor, *, out: torch.Tensor | None = None,
                     dot_mix: torch.Tensor | None = None, sqrsum: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None):
    """The post-map fused with the next sublayer's projection: out as :func:`mhc_post`
    writes it, and the next pre-map's dots and sum of squares over out, dot_mix [..., 24]
    and sqrsum [...] fp32.  Returns (out, dot_mix, sqrsum); pass them to
    :func:`mhc_pre_from_dots` with res=out.  H must be a multiple of 8; ``out`` may be
    ``res``."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"residual.shape[-2] / HC must be 4, got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    if H % 8 != 0:
        raise ValueError(f"H must be a multiple of 8, got {H}")
    _need(x, "x", torch.bfloat16)
    if tuple(x.shape) != outer + (H,):
        raise ValueError(f"x must be {outer + (H,)}, got {tuple(x.shape)}")
    _need(post, "post", torch.float32)
    if tuple(post.shape) not in (outer + (HC,), outer + (HC, 1)):
        raise ValueError(f"post must be {outer + (HC,)} or {outer + (HC, 1)}, got {tuple(post.shape)}")
    _need(comb, "comb", torch.float32)
    if tuple(comb.shape) != outer + (HC, HC):
        raise ValueError(f"comb must be {outer + (HC, HC)}, got {tuple(comb.shape)}")
    _need(hc_fn_next, "hc_fn_next", torch.float32)
    if tuple(hc_fn_next.shape) != (MIX, HC * H):
        raise ValueError(f"hc_fn_next must be {(MIX, HC * H)}, got {tuple(hc_fn_next.shape)}")
    dev = res.device
    if out is None:
        out = torch.empty_like(res)
    _need(out, "out", torch.bfloat16)
    if out.shape != res.shape:
        raise ValueError("out must have the shape of res")
    if dot_mix is None:
        dot_mix = torch.empty(outer + (MIX,), dtype=torch.float32, device=dev)
    _need(dot_mix, "dot_mix", torch.float32)
    if tuple(dot_mix.shape) != outer + (MIX,):
        raise ValueError(f"dot_mix must be {outer + (MIX,)}, got {tuple(dot_mix.shape)}")
    if sqrsum is None:
        sqrsum = torch.empty(outer, dtype=torch.float32, device=dev)
    _need(sqrsum, "sqrsum", torch.float32)
    if tuple(sqrsum.shape) != outer:
        raise ValueError(f"sqrsum must be {outer}, got {tuple(sqrsum.shape)}")
    need = mhc_post_project_workspace_bytes(T, H)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _same_device(x, res, post, comb, hc_fn_next, out, dot_mix, sqrsum, workspace)
    _check("mhc_post_project", lib().mhc_post_project(_ptr(x), _ptr(res), _ptr(post), _ptr(comb), _ptr(hc_fn_next),
                                                      T, H, _ptr(out), _ptr(dot_mix), _ptr(sqrsum), _ptr(workspace),
                                                      workspace.numel(), _stream(dev)))
    return out, dot_mix, sqrsum


def mhc_post_pre_fused(x: torch.Tensor, res: torch.Tensor, post: torch.Tensor, comb: torch.Tensor,
                       hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor, rms_eps: float = 1e-6,
                       pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6, post_mult: float = 1.0,
                       num_iters: int = 20, *, out: torch.Tensor | None = None, y=None, post_next=None,
                       comb_next=None, pre_next=None, return_pre: bool = False,
                       workspace: torch.Tensor | None = None):
    """The post-map of one sublayer and the next sublayer's pre-map in one call: out as
    :func:`mhc_post` writes it (``out`` may be ``res``), then what :func:`mhc_pre_fused`
    computes over ``out`` with the next weights.  Returns (out, y, post_next, comb_next
    [, pre_next])."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"res must be [..., 4, H], got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(x, "x", torch.bfloat16)
    if tuple(x.shape) != outer + (H,):
        raise ValueError(f"x must be {outer + (H,)}, got {tuple(x.shape)}")
    _need(post, "post", torch.float32)
    if tuple(post.shape) not in (outer + (HC,), outer + (HC, 1)):
        raise ValueError(f"post must be {outer + (HC,)} or {outer + (HC, 1)}, got {tuple(post.shape)}")
    _need(comb, "comb", torch.float32)
    if tuple(comb.shape) != outer + (HC, HC):
        raise ValueError(f"comb must be {outer + (HC, HC)}, got {tuple(comb.shape)}")
    _need(hc_fn, "hc_fn", torch.float32)
    if tuple(hc_fn.shape) != (MIX, HC * H):
        raise ValueError(f"hc_fn must be [24, 4H] = [24, {HC * H}], got {tuple(hc_fn.shape)}")
    _need(hc_scale, "hc_scale", torch.float32)
    if tuple(hc_scale.shape) != (3,):
        raise ValueError("hc_scale must be [3] (pre, post, comb)")
    _need(hc_base, "hc_base", torch.float32)
    if tuple(hc_base.shape) != (MIX,):
        raise ValueError("hc_base must be [24]")
    dev = res.device
    if out is None:
        out = torch.empty_like(res)
    _need(out, "out", torch.bfloat16)
    if out.shape != res.shape:
        raise ValueError("out must have the shape of res")
    if y is None:
        y = torch.empty(outer + (H,), dtype=torch.bfloat16, device=dev)
    if post_next is None:
        post_next = torch.empty(outer + (HC,), dtype=torch.float32, device=dev)
    if comb_next is None:
        comb_next = torch.empty(outer + (HC, HC), dtype=torch.float32, device=dev)
    if pre_next is None and return_pre:
        pre_next = torch.empty(outer + (HC,), dtype=torch.float32, device=dev)
    _need(y, "y", torch.bfloat16)
    _need(post_next, "post_next", torch.float32)
    _need(comb_next, "comb_next", torch.float32)
    if y.numel() != T * H or post_next.numel() != T * HC or comb_next.numel() != T * HC * HC:
        raise ValueError("output sizes do not match res")
    if pre_next is not None:
        _need(pre_next, "pre_next", torch.float32)
        if pre_next.numel() != T * HC:
            raise ValueError("pre_next must hold [T, 4] values")
    need = mhc_pre_fused_workspace_bytes(T, H)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    _same_device(x, res, post, comb, hc_fn, hc_scale, hc_base, out, y, post_next, comb_next, pre_next, workspace)
    _check("mhc_post_pre_fused", lib().mhc_post_pre_fused(
        _ptr(x), _ptr(res), _ptr(post), _ptr(comb), _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), T, H,
        float(rms_eps), float(pre_eps), float(sinkhorn_eps), float(post_mult), int(num_iters), _ptr(out), _ptr(y),
        _ptr(post_next), _ptr(comb_next), _ptr(pre_next), _ptr(workspace), workspace.numel(), _stream(dev)))
    if return_pre:
        return out, y, post_next, comb_next, pre_next
    return out, y, post_next, comb_next


def set_exchange_test_hooks(max_retry: int = -1, tag_skew: int = 0) -> None:
    """Test hooks of the one-read pre-map's exchange (process-wide; tests of its failure
    path only): reloads of a missing record before the step's outputs become NaN (-1: the
    default) and a value mixed into the expected tags (nonzero: every record looks
    missing).  (-1, 0) restores normal operation."""
    lib().mhc_set_exchange_test_hooks(int(max_retry), int(tag_skew) & 0xFFFFFFFF)


SINKHORN_BWD_MAX_ITERS = 255


def mhc_sinkhorn_backward(grad: torch.Tensor, logits: torch.Tensor, num_iters: int = 20, eps: float = 1e-6,
                          d_logits: torch.Tensor | None = None) -> torch.Tensor:
    """Gradient of :func:`mhc_sinkhorn` with respect to its logits, for the output gradient
    ``grad``; both [..., 4, 4] fp32.  ``d_logits`` may be ``grad`` or ``logits``."""
    _need(logits, "logits", torch.float32)
    if logits.dim() < 2 or tuple(logits.shape[-2:]) != (HC, HC):
        raise ValueError(f"logits must be [..., 4, 4], got {tuple(logits.shape)}")
    _need(grad, "grad", torch.float32)
    if grad.shape != logits.shape:
        raise ValueError("grad must have the shape of logits")
    if d_logits is None:
        d_logits = torch.empty_like(logits)
    _need(d_logits, "d_logits", torch.float32)
    if d_logits.shape != logits.shape:
        raise ValueError("d_logits must have the shape of logits")
    _same_device(grad, logits, d_logits)
    n = logits.numel() // (HC * HC)
    _check("mhc_sinkhorn_backward",
           lib().mhc_sinkhorn_backward(_ptr(grad), _ptr(logits), n, int(num_iters), float(eps), _ptr(d_logits),
                                       _stream(logits.device)))
    return d_logits


def mhc_post_backward(d_out: torch.Tensor, x: torch.Tensor, res: torch.Tensor, post: torch.Tensor,
                      comb: torch.Tensor, *, d_x: torch.Tensor | None = None, d_res: torch.Tensor | None = None,
                      d_post: torch.Tensor | None = None, d_comb: torch.Tensor | None = None):
    """Gradients of :func:`mhc_post` for the output gradient ``d_out`` [..., 4, H] bf16:
    returns (d_x [..., H] bf16, d_res [..., 4, H] bf16, d_post [..., 4] fp32, d_comb [..., 4, 4] fp32).
    ``d_res`` may be ``d_out``; ``post`` may be [..., 4] or [..., 4, 1] (d_post takes its shape)."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"residual.shape[-2] / HC must be 4, got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(d_out, "d_out", torch.bfloat16)
    if d_out.shape != res.shape:
        raise ValueError("d_out must have the shape of res")
    _need(x, "x", torch.bfloat16)
    if tuple(x.shape) != outer + (H,):
        raise ValueError(f"x must be {outer + (H,)}, got {tuple(x.shape)}")
    _need(post, "post", torch.float32)
    if tuple(post.shape) not in (outer + (HC,), outer + (HC, 1)):
        raise ValueError(f"post must be {outer + (HC,)} or {outer + (HC, 1)}, got {tuple(post.shape)}")
    _need(comb, "comb", torch.float32)
    if tuple(comb.shape) != outer + (HC, HC):
        raise ValueError(f"comb must be {outer + (HC, HC)}, got {tuple(comb.shape)}")
    if d_x is None:
        d_x = torch.empty_like(x)
    if d_res is None:
        d_res = torch.empty_like(res)
    if d_post is None:
        d_post = torch.empty_like(post)
    if d_comb is None:
        d_comb = torch.empty_like(comb)
    for t, name, dt, shape in ((d_x, "d_x", torch.bfloat16, x.shape), (d_res, "d_res", torch.bfloat16, res.shape),
                               (d_post, "d_post", torch.float32, post.shape),
                               (d_comb, "d_comb", torch.float32, comb.shape)):
        _need(t, name, dt)
        if t.shape != shape:
            raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")
    _same_device(d_out, x, res, post, comb, d_x, d_res, d_post, d_comb)
    _check("mhc_post_backward",
           lib().mhc_post_backward(_ptr(d_out), _ptr(x), _ptr(res), _ptr(post), _ptr(comb), T, H, _ptr(d_x),
                                   _ptr(d_res), _ptr(d_post), _ptr(d_comb), _stream(res.device)))
    return d_x, d_res, d_post, d_comb


def mhc_expand(hidden: torch.Tensor, streams: torch.Tensor | None = None) -> torch.Tensor:
    """Model entry: hidden [..., H] bf16 -> streams [..., 4, H] bf16, each stream a copy of the row."""
    _need(hidden, "hidden", torch.bfloat16)
    if hidden.dim() < 1:
        raise ValueError("hidden must be [..., H]")
    H = hidden.shape[-1]
    outer = tuple(hidden.shape[:-1])
    T = hidden.numel() // H if H > 0 else 0
    if streams is None:
        streams = torch.empty(outer + (HC, H), dtype=torch.bfloat16, device=hidden.device)
    _need(streams, "streams", torch.bfloat16)
    if tuple(streams.shape) != outer + (HC, H):
        raise ValueError(f"streams must be {outer + (HC, H)}, got {tuple(streams.shape)}")
    _same_device(hidden, streams)
    _check("mhc_expand", lib().mhc_expand(_ptr(hidden), T, H, _ptr(streams), _stream(hidden.device)))
    return streams


def mhc_head_mean(res: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """Model exit, unweighted: res [..., 4, H] bf16 -> the mean of the 4 streams [..., H] bf16."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"res must be [..., 4, H], got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    if y is None:
        y = torch.empty(outer + (H,), dtype=torch.bfloat16, device=res.device)
    _need(y, "y", torch.bfloat16)
    if tuple(y.shape) != outer + (H,):
        raise ValueError(f"y must be {outer + (H,)}, got {tuple(y.shape)}")
    _same_device(res, y)
    _check("mhc_head_mean", lib().mhc_head_mean(_ptr(res), T, H, _ptr(y), _stream(res.device)))
    return y


def mhc_expand_f32(hidden: torch.Tensor, streams: torch.Tensor | None = None) -> torch.Tensor:
    """Model entry onto fp32 streams: hidden [..., H] bf16 -> streams [..., 4, H] float32."""
    _need(hidden, "hidden", torch.bfloat16)
    if hidden.dim() < 1:
        raise ValueError("hidden must be [..., H]")
    H = hidden.shape[-1]
    outer = tuple(hidden.shape[:-1])
    T = hidden.numel() // H if H > 0 else 0
    if streams is None:
        streams = torch.empty(outer + (HC, H), dtype=torch.float32, device=hidden.device)
    _need(streams, "streams", torch.float32)
    if tuple(streams.shape) != outer + (HC, H):
        raise ValueError(f"streams must be {outer + (HC, H)}, got {tuple(streams.shape)}")
    _same_device(hidden, streams)
    _check("mhc_expand_f32", lib().mhc_expand_f32(_ptr(hidden), T, H, _ptr(streams), _stream(hidden.device)))
    return streams


def mhc_head_mean_f32(res: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """Model exit, unweighted, over fp32 streams: res [..., 4, H] float32 -> y [..., H] bf16."""
    _need(res, "res", torch.float32)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"res must be [..., 4, H], got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    if y is None:
        y = torch.empty(outer + (H,), dtype=torch.bfloat16, device=res.device)
    _need(y, "y", torch.bfloat16)
    if tuple(y.shape) != outer + (H,):
        raise ValueError(f"y must be {outer + (H,)}, got {tuple(y.shape)}")
    _same_device(res, y)
    _check("mhc_head_mean_f32", lib().mhc_head_mean_f32(_ptr(res), T, H, _ptr(y), _stream(res.device)))
    return y


def mhc_head(res: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
             norm_eps: float = 1e-6, hc_eps: float = 1e-6, *, y: torch.Tensor | None = None,
             pre: torch.Tensor | None = None, return_pre: bool = False,
             workspace: torch.Tensor | None = None):
    """Model exit, weighted: res [..., 4, H] bf16, hc_fn [4, 4H], hc_scale [1], hc_base [4] fp32 ->
    y [..., H] bf16 (and pre [..., 4] fp32 with ``return_pre``)."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"res must be [..., 4, H], got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(hc_fn, "hc_fn", torch.float32)
    if tuple(hc_fn.shape) != (HC, HC * H):
        raise ValueError(f"hc_fn must be [4, 4H] = [4, {HC * H}], got {tuple(hc_fn.shape)}")
    _need(hc_scale, "hc_scale", torch.float32)
    _need(hc_base, "hc_base", torch.float32)
    if hc_scale.numel() != 1 or hc_base.numel() != HC:
        raise ValueError("hc_scale must hold 1 value and hc_base 4")
    dev = res.device
    if y is None:
        y = torch.empty(outer + (H,), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16)
    if y.numel() != T * H:
        raise ValueError("y must hold [T, H] values")
    if pre is None and return_pre:
        pre = torch.empty(outer + (HC,), dtype=torch.float32, device=dev)
    if pre is not None:
        _need(pre, "pre", torch.float32)
        if pre.numel() != T * HC:
            raise ValueError("pre must hold [T, 4] values")
    need = mhc_pre_fused_workspace_bytes(T, H)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    _same_device(res, hc_fn, hc_scale, hc_base, y, pre, workspace)
    _check("mhc_head", lib().mhc_head(_ptr(res), _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), T, H, float(norm_eps),
                                      float(hc_eps), _ptr(y), _ptr(pre), _ptr(workspace), workspace.numel(),
                                      _stream(dev)))
    return (y, pre) if return_pre else y


def mhc_pre_backward_workspace_bytes(T: int) -> int:
    return int(lib().mhc_pre_backward_workspace_bytes(int(T)))


def mhc_pre_from_dots_backward(dy: torch.Tensor, d_post: torch.Tensor, d_comb: torch.Tensor,
                               dot_mix: torch.Tensor, res: torch.Tensor, hc_scale: torch.Tensor,
                               hc_base: torch.Tensor, sqrsum: torch.Tensor | None = None, k: float | None = None,
                               rms_eps: float = 1e-6, pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6,
                               post_mult: float = 1.0, num_iters: int = 20, *, d_res: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None) -> dict:
    """Gradients of :func:`mhc_pre_from_dots` for the output gradients dy [..., H] bf16,
    d_post [..., 4] (or [..., 4, 1]) and d_comb [..., 4, 4] fp32.  dot_mix and sqrsum as in
    the forward.  Returns a dict: d_res [..., 4, H] bf16, d_dot [..., 24] fp32 (the gradient
    of every split's partial dots), d_sqrsum [...] fp32 or None, d_hc_scale [3], d_hc_base [24].
    ``d_res`` may be ``res``."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"residual.shape[-2] / HC must be 4, got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(dy, "dy", torch.bfloat16)
    if tuple(dy.shape) != outer + (H,):
        raise ValueError(f"dy must be {outer + (H,)}, got {tuple(dy.shape)}")
    _need(d_post, "d_post", torch.float32)
    if tuple(d_post.shape) not in (outer + (HC,), outer + (HC, 1)):
        raise ValueError(f"d_post must be {outer + (HC,)} or {outer + (HC, 1)}, got {tuple(d_post.shape)}")
    _need(d_comb, "d_comb", torch.float32)
    if tuple(d_comb.shape) != outer + (HC, HC):
        raise ValueError(f"d_comb must be {outer + (HC, HC)}, got {tuple(d_comb.shape)}")
    _need(dot_mix, "dot_mix", torch.float32)
    if tuple(dot_mix.shape) == outer + (MIX,):
        splits = 1
    elif dot_mix.dim() == len(outer) + 2 and tuple(dot_mix.shape[1:]) == outer + (MIX,):
        splits = dot_mix.shape[0]
    else:
        raise ValueError(f"dot_mix must be {outer + (MIX,)} or [S, *{outer + (MIX,)}], got {tuple(dot_mix.shape)}")
    if sqrsum is not None:
        _need(sqrsum, "sqrsum", torch.float32)
        if sqrsum.numel() != splits * T:
            raise ValueError(f"sqrsum must hold num_splits * T = {splits * T} values, got {sqrsum.numel()}")
    _need(hc_scale, "hc_scale", torch.float32)
    _need(hc_base, "hc_base", torch.float32)
    if hc_scale.numel() != 3 or hc_base.numel() != MIX:
        raise ValueError("hc_scale must have 3 values and hc_base 24")
    if d_res is None:
        d_res = torch.empty_like(res)
    _need(d_res, "d_res", torch.bfloat16)
    if d_res.shape != res.shape:
        raise ValueError("d_res must have the shape of res")
    dev = res.device
    d_dot = torch.empty(outer + (MIX,), dtype=torch.float32, device=dev)
    d_sq = torch.empty(outer, dtype=torch.float32, device=dev) if sqrsum is not None else None
    d_scale = torch.empty(3, dtype=torch.float32, device=dev)
    d_base = torch.empty(MIX, dtype=torch.float32, device=dev)
    need = mhc_pre_backward_workspace_bytes(T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _same_device(dy, d_post, d_comb, dot_mix, sqrsum, res, hc_scale, hc_base, d_res, workspace)
    kk = float(HC * H) if k is None else float(k)
    _check("mhc_pre_from_dots_backward",
           lib().mhc_pre_from_dots_backward(_ptr(dy), _ptr(d_post), _ptr(d_comb), _ptr(dot_mix), _ptr(sqrsum),
                                            int(splits), _ptr(res), _ptr(hc_scale), _ptr(hc_base), T, H, kk,
                                            float(rms_eps), float(pre_eps), float(sinkhorn_eps), float(post_mult),
                                            int(num_iters), _ptr(d_res), _ptr(d_dot), _ptr(d_sq), _ptr(d_scale),
                                            _ptr(d_base), _ptr(workspace), workspace.numel(), _stream(dev)))
    return dict(d_res=d_res, d_dot=d_dot, d_sqrsum=d_sq, d_hc_scale=d_scale, d_hc_base=d_base)


def mhc_pre_fused_backward_workspace_bytes(T: int, H: int) -> int:
    return int(lib().mhc_pre_fused_backward_workspace_bytes(int(T), int(H)))


def mhc_pre_fused_backward(dy: torch.Tensor, d_post: torch.Tensor, d_comb: torch.Tensor, res: torch.Tensor,
                           hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                           rms_eps: float = 1e-6, pre_eps: float = 1e-6, sinkhorn_eps: float = 1e-6,
                           post_mult: float = 1.0, num_iters: int = 20, *, d_res: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None) -> dict:
    """Gradients of :func:`mhc_pre_fused` for dy [..., H] bf16, d_post [..., 4] and d_comb [..., 4, 4]
    fp32: a dict with d_res [..., 4, H] bf16, d_hc_fn [24, 4H], d_hc_scale [3], d_hc_base [24] fp32.
    ``d_res`` may be ``res``.  H must be a multiple of 8."""
    _need(res, "res", torch.bfloat16)
    if res.dim() < 2 or res.shape[-2] != HC:
        raise ValueError(f"res must be [..., 4, H], got {tuple(res.shape)}")
    H = res.shape[-1]
    outer = tuple(res.shape[:-2])
    T = res.numel() // (HC * H) if H > 0 else 0
    _need(dy, "dy", torch.bfloat16)
    if tuple(dy.shape) != outer + (H,):
        raise ValueError(f"dy must be {outer + (H,)}, got {tuple(dy.shape)}")
    _need(d_post, "d_post", torch.float32)
    if d_post.numel() != T * HC:
        raise ValueError("d_post must hold [T, 4] values")
    _need(d_comb, "d_comb", torch.float32)
    if tuple(d_comb.shape) != outer + (HC, HC):
        raise ValueError(f"d_comb must be {outer + (HC, HC)}, got {tuple(d_comb.shape)}")
    _need(hc_fn, "hc_fn", torch.float32)
    if tuple(hc_fn.shape) != (MIX, HC * H):
        raise ValueError(f"hc_fn must be [24, 4H] = [24, {HC * H}], got {tuple(hc_fn.shape)}")
    _need(hc_scale, "hc_scale", torch.float32)
    _need(hc_base, "hc_base", torch.float32)
    if hc_scale.numel() != 3 or hc_base.numel() != MIX:
        raise ValueError("hc_scale must have 3 values and hc_base 24")
    dev = res.device
    if d_res is None:
        d_res = torch.empty_like(res)
    _need(d_res, "d_res", torch.bfloat16)
    if d_res.shape != res.shape:
        raise ValueError("d_res must have the shape of res")
    d_fn = torch.empty(MIX, HC * H, dtype=torch.float32, device=dev)
    d_scale = torch.empty(3, dtype=torch.float32, device=dev)
    d_base = torch.empty(MIX, dtype=torch.float32, device=dev)
    need = mhc_pre_fused_backward_workspace_bytes(T, H)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _same_device(dy, d_post, d_comb, res, hc_fn, hc_scale, hc_base, d_res, workspace)
    _check("mhc_pre_fused_backward",
           lib().mhc_pre_fused_backward(_ptr(dy), _ptr(d_post), _ptr(d_comb), _ptr(res), _ptr(hc_fn), _ptr(hc_scale),
                                        _ptr(hc_base), T, H, float(rms_eps), float(pre_eps), float(sinkhorn_eps),
                                        float(post_mult), int(num_iters), _ptr(d_res), _ptr(d_fn), _ptr(d_scale),
                                        _ptr(d_base), _ptr(workspace), workspace.numel(), _stream(dev)))
    return dict(d_res=d_res, d_hc_fn=d_fn, d_hc_scale=d_scale, d_hc_base=d_base)


__all__ = ["mhc_sinkhorn", "mhc_pre_fused", "mhc_pre_fused_noalloc", "mhc_pre_fused_bf16", "mhc_pre_fused_f32",
           "mhc_pre_split_bytes", "mhc_pre_split_weights", "mhc_pre_fused_presplit",
           "mhc_post_f32", "mhc_expand_f32", "mhc_head_mean_f32", "mhc_expand", "mhc_head_mean", "mhc_head",
           "mhc_pre_fused_workspace_bytes", "mhc_pre_from_dots", "mhc_post",
           "mhc_sinkhorn_backward", "mhc_post_backward", "mhc_pre_from_dots_backward",
           "mhc_pre_backward_workspace_bytes", "mhc_pre_fused_backward", "mhc_pre_fused_backward_workspace_bytes",
           "mhc_post_project", "mhc_post_project_workspace_bytes", "mhc_post_pre_fused",
           "set_exchange_test_hooks",
           "lib", "abi_version", "status_string", "launch_plan", "MHCError", "HC",
           "MIX", "SINKHORN_BWD_MAX_ITERS", "MHC_PRE_FUSED_NOALLOC_MAX_BYTES"]
