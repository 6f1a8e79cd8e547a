"""ctypes shim over the fp64 CPU oracle (``mhc_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product library never imports
it, and it imports nothing from the product package.

All results are returned as unrounded float64 numpy arrays; callers round them
(``round_bf16``, ``np.float32``) where a comparison needs the rounded value.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_DIR = Path(__file__).resolve().parent
_SRC = _DIR / "mhc_oracle.c"
_LIB_PATH = _DIR / "libmhc_oracle.so"
_lib = None

HC = 4
MIX = 24


def build(verbose: bool = False) -> Path:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-o", str(_LIB_PATH) + ".tmp", str(_SRC), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(str(_LIB_PATH) + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # MHC_ORACLE_LIB names another build of this source to load instead: the planted-mistake
    # test builds mutated copies and runs the pins against each.
    alt = os.environ.get("MHC_ORACLE_LIB")
    if alt:
        lib = ctypes.CDLL(alt)
    else:
        if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        lib = ctypes.CDLL(str(_LIB_PATH))
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    lib.orc_f64_to_bf16.argtypes = [D]
    lib.orc_f64_to_bf16.restype = ctypes.c_uint16
    lib.orc_round_bf16.argtypes = [P, I64, P]
    lib.orc_rms.argtypes = [P, I64, I64, D, P, P]
    lib.orc_project.argtypes = [P, P, I64, I64, P]
    lib.orc_mix_activation.argtypes = [P, P, P, P, I64, D, D, P, P, P]
    lib.orc_sinkhorn.argtypes = [P, I64, ctypes.c_int, D, P]
    lib.orc_collapse.argtypes = [P, P, I64, I64, P]
    lib.orc_post.argtypes = [P, P, P, P, I64, I64, P]
    lib.orc_pre.argtypes = [P, P, P, P, I64, I64, D, D, D, D, ctypes.c_int, P, P, P, P, P, P]
    lib.orc_pre_from_dots.argtypes = [P, P, I64, P, P, P, I64, I64, D, D, D, D, D, ctypes.c_int, P, P, P, P]
    lib.orc_sinkhorn_backward.argtypes = [P, P, I64, ctypes.c_int, D, P]
    lib.orc_post_backward.argtypes = [P, P, P, P, P, I64, I64, P, P, P, P]
    lib.orc_pre_from_dots_backward.argtypes = [P, P, P, P, P, P, P, P, I64, I64, D, D, D, D, D, ctypes.c_int,
                                               P, P, P, P, P]
    lib.orc_expand.argtypes = [P, I64, I64, P]
    lib.orc_head_mean.argtypes = [P, I64, I64, P]
    lib.orc_head.argtypes = [P, P, P, P, I64, I64, D, D, P, P]
    lib.orc_pre_backward.argtypes = [P, P, P, P, P, P, P, I64, I64, D, D, D, D, ctypes.c_int, P, P, P, P, P]
    lib.orc_rms_f32s.argtypes = [P, I64, I64, D, P, P]
    lib.orc_project_f32s.argtypes = [P, P, I64, I64, P]
    lib.orc_collapse_f32s.argtypes = [P, P, I64, I64, P]
    lib.orc_pre_f32s.argtypes = [P, P, P, P, I64, I64, D, D, D, D, ctypes.c_int, P, P, P, P]
    lib.orc_post_f32s.argtypes = [P, P, P, P, I64, I64, P]
    lib.orc_expand_f32s.argtypes = [P, I64, I64, P]
    lib.orc_head_mean_f32s.argtypes = [P, I64, I64, P]
    for f in ("orc_round_bf16", "orc_rms", "orc_project", "orc_mix_activation", "orc_sinkhorn",
              "orc_collapse", "orc_post", "orc_pre", "orc_pre_from_dots", "orc_sinkhorn_backward",
              "orc_post_backward", "orc_rms_f32s", "orc_project_f32s", "orc_collapse_f32s", "orc_pre_f32s",
              "orc_post_f32s", "orc_expand_f32s", "orc_head_mean_f32s"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 bit patterns (nearest, ties to even), directly from fp64."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_round_bf16(_p(v), v.size, _p(out))
    return out


def rms(res: np.ndarray, rms_eps: float):
    """Step A1: (sqsum [T], rstd [T]) of res [T,4,H] (bf16 bits)."""
    res = _c(res, np.uint16)
    T, hc, H = res.shape
    assert hc == HC
    sq = np.empty(T)
    rstd = np.empty(T)
    _load().orc_rms(_p(res), T, H, rms_eps, _p(sq), _p(rstd))
    return sq, rstd


def project(res: np.ndarray, hc_fn: np.ndarray) -> np.ndarray:
    """Step A2: dot [T,24] = res_flat @ hc_fn^T in fp64."""
    res = _c(res, np.uint16)
    hc_fn = _c(hc_fn, np.float32)
    T, hc, H = res.shape
    assert hc == HC and hc_fn.shape == (MIX, HC * H)
    dot = np.empty((T, MIX))
    _load().orc_project(_p(res), _p(hc_fn), T, H, _p(dot))
    return dot


def mix_activation(dot, rstd, hc_scale, hc_base, pre_eps, post_mult):
    """Step A3: (pre [T,4], post [T,4], comb_logits [T,4,4])."""
    dot = _c(dot, np.float64)
    rstd = _c(rstd, np.float64)
    hc_scale = _c(hc_scale, np.float32)
    hc_base = _c(hc_base, np.float32)
    T = dot.shape[0]
    pre = np.empty((T, HC))
    post = np.empty((T, HC))
    logits = np.empty((T, HC, HC))
    _load().orc_mix_activation(_p(dot), _p(rstd), _p(hc_scale), _p(hc_base), T, pre_eps, post_mult,
                               _p(pre), _p(post), _p(logits))
    return pre, post, logits


def sinkhorn(logits: np.ndarray, num_iters: int = 20, eps: float = 1e-6) -> np.ndarray:
    """Step A4: [n,4,4] logits -> [n,4,4] Sinkhorn projection (fp64)."""
    lg = _c(logits, np.float64)
    shape = lg.shape
    assert shape[-2:] == (HC, HC)
    n = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    out = np.empty(shape)
    _load().orc_sinkhorn(_p(lg), n, int(num_iters), eps, _p(out))
    return out


def collapse(res: np.ndarray, pre: np.ndarray) -> np.ndarray:
    """Step A5: y [T,H] = sum_i pre[:,i] * res[:,i,:]."""
    res = _c(res, np.uint16)
    pre = _c(pre, np.float64)
    T, hc, H = res.shape
    y = np.empty((T, H))
    _load().orc_collapse(_p(res), _p(pre), T, H, _p(y))
    return y


def post(x: np.ndarray, res: np.ndarray, post: np.ndarray, comb: np.ndarray) -> np.ndarray:
    """Step A6: out [T,4,H] (fp64, unrounded)."""
    x = _c(x, np.uint16)
    res = _c(res, np.uint16)
    post_ = _c(post, np.float64).reshape(-1, HC)
    comb = _c(comb, np.float64).reshape(-1, HC, HC)
    T, hc, H = res.shape
    assert x.shape == (T, H) and post_.shape[0] == T and comb.shape[0] == T
    out = np.empty((T, HC, H))
    _load().orc_post(_p(x), _p(res), _p(post_), _p(comb), T, H, _p(out))
    return out


def pre(res, hc_fn, hc_scale, hc_base, rms_eps=1e-6, pre_eps=1e-6, sinkhorn_eps=1e-6, post_mult=1.0,
        num_iters=20):
    """Whole pre-map.  Returns dict of fp64 arrays: y, post, comb, pre, dot, rstd."""
    res = _c(res, np.uint16)
    hc_fn = _c(hc_fn, np.float32)
    hc_scale = _c(hc_scale, np.float32)
    hc_base = _c(hc_base, np.float32)
    T, hc, H = res.shape
    assert hc == HC and hc_fn.shape == (MIX, HC * H) and hc_scale.shape == (3,) and hc_base.shape == (MIX,)
    y = np.empty((T, H))
    post_ = np.empty((T, HC))
    comb = np.empty((T, HC, HC))
    pre_ = np.empty((T, HC))
    dot = np.empty((T, MIX))
    rstd = np.empty(T)
    _load().orc_pre(_p(res), _p(hc_fn), _p(hc_scale), _p(hc_base), T, H, rms_eps, pre_eps, sinkhorn_eps,
                    post_mult, int(num_iters), _p(y), _p(post_), _p(comb), _p(pre_), _p(dot), _p(rstd))
    return dict(y=y, post=post_, comb=comb, pre=pre_, dot=dot, rstd=rstd)


def pre_from_dots(dot_mix, res, hc_scale, hc_base, sqrsum=None, k=None, rms_eps=1e-6, pre_eps=1e-6,
                  sinkhorn_eps=1e-6, post_mult=1.0, num_iters=20):
    """Pre-map from an external projection.  dot_mix [T,24] or [S,T,24] fp32, sqrsum None, [T] or [S,T]
    fp32, k the RMS denominator (default 4H).  Returns dict of fp64 arrays: y, post, comb, pre."""
    res = _c(res, np.uint16)
    T, hc, H = res.shape
    assert hc == HC
    dm = _c(dot_mix, np.float32)
    if dm.ndim == 2:
        dm = dm.reshape(1, T, MIX)
    S = dm.shape[0]
    assert dm.shape == (S, T, MIX)
    sq = None
    if sqrsum is not None:
        sq = _c(sqrsum, np.float32).reshape(S, T)
    k = float(HC * H) if k is None else float(k)
    y = np.empty((T, H))
    post_ = np.empty((T, HC))
    comb = np.empty((T, HC, HC))
    pre_ = np.empty((T, HC))
    _load().orc_pre_from_dots(_p(dm), _p(sq) if sq is not None else None, S, _p(res),
                              _p(_c(hc_scale, np.float32)), _p(_c(hc_base, np.float32)), T, H, k, rms_eps,
                              pre_eps, sinkhorn_eps, post_mult, int(num_iters), _p(y), _p(post_), _p(comb),
                              _p(pre_))
    return dict(y=y, post=post_, comb=comb, pre=pre_)


def sinkhorn_backward(grad, logits, num_iters=20, eps=1e-6):
    """d_logits [n,4,4] of the fixed-count Sinkhorn for the output gradient grad [n,4,4] (fp64)."""
    g = _c(grad, np.float64)
    lg = _c(logits, np.float64)
    assert g.shape == lg.shape and lg.shape[-2:] == (HC, HC)
    assert 1 <= int(num_iters) <= 1024
    n = int(np.prod(lg.shape[:-2])) if lg.ndim > 2 else 1
    out = np.empty(lg.shape)
    _load().orc_sinkhorn_backward(_p(g), _p(lg), n, int(num_iters), eps, _p(out))
    return out


def post_backward(d_out, x, res, post, comb):
    """Reverse mode of the post-map: (d_x [T,H], d_res [T,4,H], d_post [T,4], d_comb [T,4,4]), fp64."""
    d_out = _c(d_out, np.uint16)
    x = _c(x, np.uint16)
    res = _c(res, np.uint16)
    T, hc, H = res.shape
    assert hc == HC and d_out.shape == res.shape and x.shape == (T, H)
    post_ = _c(post, np.float64).reshape(T, HC)
    comb = _c(comb, np.float64).reshape(T, HC, HC)
    d_x = np.empty((T, H))
    d_res = np.empty((T, HC, H))
    d_post = np.empty((T, HC))
    d_comb = np.empty((T, HC, HC))
    _load().orc_post_backward(_p(d_out), _p(x), _p(res), _p(post_), _p(comb), T, H, _p(d_x), _p(d_res),
                              _p(d_post), _p(d_comb))
    return d_x, d_res, d_post, d_comb



def pre_from_dots_backward(dy, d_post, d_comb, dot, res, hc_scale, hc_base, sqrsum=None, k=None, rms_eps=1e-6,
                           pre_eps=1e-6, sinkhorn_eps=1e-6, post_mult=1.0, num_iters=20):
    """Reverse mode of the pre-map from external dots (one split).  dy [T,H] bf16 bits, d_post [T,4],
    d_comb [T,4,4], dot [T,24] and sqrsum [T] or None (real values).  Returns dict of fp64 arrays:
    d_res [T,4,H], d_dot [T,24], d_sqrsum [T] (None when sqrsum is None), d_hc_scale [3], d_hc_base [24]."""
    res = _c(res, np.uint16)
    T, hc, H = res.shape
    assert hc == HC
    dy = _c(dy, np.uint16)
    assert dy.shape == (T, H)
    d_post = _c(d_post, np.float64).reshape(T, HC)
    d_comb = _c(d_comb, np.float64).reshape(T, HC, HC)
    dot = _c(dot, np.float64).reshape(T, MIX)
    sq = None if sqrsum is None else _c(sqrsum, np.float64).reshape(T)
    hc_scale = _c(hc_scale, np.float32)
    hc_base = _c(hc_base, np.float32)
    assert 1 <= int(num_iters) <= 1024
    k = float(HC * H) if k is None else float(k)
    d_res = np.empty((T, HC, H))
    d_dot = np.empty((T, MIX))
    d_sq = np.empty(T) if sq is not None else None
    d_scale = np.empty(3)
    d_base = np.empty(MIX)
    _load().orc_pre_from_dots_backward(_p(dy), _p(d_post), _p(d_comb), _p(dot), _p(sq) if sq is not None else None,
                                       _p(res), _p(hc_scale), _p(hc_base), T, H, k, rms_eps, pre_eps, sinkhorn_eps,
                                       post_mult, int(num_iters), _p(d_res), _p(d_dot),
                                       _p(d_sq) if d_sq is not None else None, _p(d_scale), _p(d_base))
    return dict(d_res=d_res, d_dot=d_dot, d_sqrsum=d_sq, d_hc_scale=d_scale, d_hc_base=d_base)


def pre_backward(dy, d_post, d_comb, res, hc_fn, hc_scale, hc_base, rms_eps=1e-6, pre_eps=1e-6, sinkhorn_eps=1e-6,
                 post_mult=1.0, num_iters=20):
    """Reverse mode of the whole pre-map (projection inside).  Returns dict of fp64 arrays:
    d_res [T,4,H], d_hc_fn [24,4H], d_hc_scale [3], d_hc_base [24]."""
    res = _c(res, np.uint16)
    T, hc, H = res.shape
    assert hc == HC
    dy = _c(dy, np.uint16)
    assert dy.shape == (T, H)
    d_post = _c(d_post, np.float64).reshape(T, HC)
    d_comb = _c(d_comb, np.float64).reshape(T, HC, HC)
    hc_fn = _c(hc_fn, np.float32)
    assert hc_fn.shape == (MIX, HC * H)
    hc_scale = _c(hc_scale, np.float32)
    hc_base = _c(hc_base, np.float32)
    assert 1 <= int(num_iters) <= 1024
    d_res = np.empty((T, HC, H))
    d_fn = np.empty((MIX, HC * H))
    d_scale = np.empty(3)
    d_base = np.empty(MIX)
    scratch = np.empty(2 * MIX * max(T, 1))
    _load().orc_pre_backward(_p(dy), _p(d_post), _p(d_comb), _p(res), _p(hc_fn), _p(hc_scale), _p(hc_base), T, H,
                             rms_eps, pre_eps, sinkhorn_eps, post_mult, int(num_iters), _p(d_res), _p(d_fn),
                             _p(d_scale), _p(d_base), _p(scratch))
    return dict(d_res=d_res, d_hc_fn=d_fn, d_hc_scale=d_scale, d_hc_base=d_base)


def expand(hidden):
    """Model entry: [T,H] bf16 bits -> [T,4,H] bf16 bits, each stream a copy of the row."""
    hidden = _c(hidden, np.uint16)
    T, H = hidden.shape
    out = np.empty((T, HC, H), np.uint16)
    _load().orc_expand(_p(hidden), T, H, _p(out))
    return out


def head_mean(res):
    """Model exit, unweighted: the mean of the 4 streams, [T,H] fp64 (unrounded)."""
    res = _c(res, np.uint16)
    T, hc, H = res.shape
    assert hc == HC
    y = np.empty((T, H))
    _load().orc_head_mean(_p(res), T, H, _p(y))
    return y


def head(res, hc_fn, hc_scale, hc_base, norm_eps=1e-6, hc_eps=1e-6):
    """Model exit, weighted: hc_fn [4,4H], hc_scale [1], hc_base [4] fp32.  Returns dict of fp64
    arrays y [T,H], pre [T,4]."""
    res = _c(res, np.uint16)
    T, hc, H = res.shape
    assert hc == HC
    hc_fn = _c(hc_fn, np.float32)
    assert hc_fn.shape == (HC, HC * H)
    hc_scale = _c(hc_scale, np.float32).reshape(-1)
    hc_base = _c(hc_base, np.float32).reshape(-1)
    assert hc_scale.shape == (1,) and hc_base.shape == (HC,)
    y = np.empty((T, H))
    pre_ = np.empty((T, HC))
    _load().orc_head(_p(res), _p(hc_fn), _p(hc_scale), _p(hc_base), T, H, norm_eps, hc_eps, _p(y), _p(pre_))
    return dict(y=y, pre=pre_)


# ---------------------------------------------------------------- fp32 residual streams
# The same steps on FP32 [T, 4, H] streams (metrale hyper_connection_dispatch.rs, module
# header; glm5next_mhc.rs, glm_hc_expand / glm_hc_pre / glm_hc_post).  res is float32.

def rms_f32s(res: np.ndarray, rms_eps: float):
    """Step A1 on fp32 streams: (sqsum [T], rstd [T])."""
    res = _c(res, np.float32)
    T, hc, H = res.shape
    assert hc == HC
    sq = np.empty(T)
    rstd = np.empty(T)
    _load().orc_rms_f32s(_p(res), T, H, float(rms_eps), _p(sq), _p(rstd))
    return sq, rstd


def project_f32s(res: np.ndarray, hc_fn: np.ndarray) -> np.ndarray:
    """Step A2 on fp32 streams: dot [T,24]."""
    res = _c(res, np.float32)
    T, hc, H = res.shape
    assert hc == HC
    hc_fn = _c(hc_fn, np.float32)
    assert hc_fn.shape == (MIX, HC * H)
    dot = np.empty((T, MIX))
    _load().orc_project_f32s(_p(res), _p(hc_fn), T, H, _p(dot))
    return dot


def collapse_f32s(res: np.ndarray, pre: np.ndarray) -> np.ndarray:
    """Step A5 on fp32 streams: y [T,H] fp64 (unrounded)."""
    res = _c(res, np.float32)
    T, hc, H = res.shape
    assert hc == HC
    pre = _c(pre, np.float64).reshape(T, HC)
    y = np.empty((T, H))
    _load().orc_collapse_f32s(_p(res), _p(pre), T, H, _p(y))
    return y


def pre_f32s(res, hc_fn, hc_scale, hc_base, rms_eps=1e-6, pre_eps=1e-6, sinkhorn_eps=1e-6, post_mult=1.0,
             num_iters=20):
    """The pre-map on fp32 streams res [T,4,H].  Returns dict of fp64 arrays: y, post, comb, pre."""
    res = _c(res, np.float32)
    T, hc, H = res.shape
    assert hc == HC
    hc_fn = _c(hc_fn, np.float32)
    assert hc_fn.shape == (MIX, HC * H)
    y = np.empty((T, H))
    post_ = np.empty((T, HC))
    comb = np.empty((T, HC, HC))
    pre_ = np.empty((T, HC))
    _load().orc_pre_f32s(_p(res), _p(hc_fn), _p(_c(hc_scale, np.float32)), _p(_c(hc_base, np.float32)), T, H,
                         rms_eps, pre_eps, sinkhorn_eps, post_mult, int(num_iters), _p(y), _p(post_), _p(comb),
                         _p(pre_))
    return dict(y=y, post=post_, comb=comb, pre=pre_)


def post_f32s(x: np.ndarray, res: np.ndarray, post: np.ndarray, comb: np.ndarray) -> np.ndarray:
    """Step A6 on fp32 streams: x [T,H] bf16 bits, res [T,4,H] fp32, post [T,4], comb [T,4,4]
    (real values) -> out [T,4,H] fp64 (unrounded)."""
    res = _c(res, np.float32)
    T, hc, H = res.shape
    assert hc == HC
    x = _c(x, np.uint16)
    assert x.shape == (T, H)
    post = _c(post, np.float64).reshape(T, HC)
    comb = _c(comb, np.float64).reshape(T, HC, HC)
    out = np.empty((T, HC, H))
    _load().orc_post_f32s(_p(x), _p(res), _p(post), _p(comb), T, H, _p(out))
    return out


def expand_f32s(hidden):
    """Model entry on fp32 streams: [T,H] bf16 bits -> [T,4,H] float32 (exact widening)."""
    hidden = _c(hidden, np.uint16)
    T, H = hidden.shape
    out = np.empty((T, HC, H), np.float32)
    _load().orc_expand_f32s(_p(hidden), T, H, _p(out))
    return out


def head_mean_f32s(res):
    """Model exit, unweighted, on fp32 streams: [T,H] fp64 (unrounded)."""
    res = _c(res, np.float32)
    T, hc, H = res.shape
    assert hc == HC
    y = np.empty((T, H))
    _load().orc_head_mean_f32s(_p(res), T, H, _p(y))
    return y
