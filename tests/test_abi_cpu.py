"""Host-side checks of libmhc's C ABI (no GPU needed, no kernel is launched).

Every call here fails validation, or is a T == 0 no-op, before any HIP call,
so fake non-null pointers are never dereferenced.
"""
import ctypes
import re
from pathlib import Path

import pytest

import mhc_hyper_connection_amd as mhc

HEADER = Path(__file__).resolve().parents[1] / "include" / "mhc.h"
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation rejects before use
FAKE2 = ctypes.c_void_p(0x20000000)
NULL = None


def _declared():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(mhc_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = mhc.lib()
    names = _declared()
    assert {"mhc_sinkhorn", "mhc_pre_fused", "mhc_pre_fused_workspace_bytes", "mhc_pre_from_dots", "mhc_post",
            "mhc_sinkhorn_backward", "mhc_post_backward", "mhc_pre_from_dots_backward",
            "mhc_pre_backward_workspace_bytes", "mhc_pre_fused_bf16", "mhc_expand", "mhc_head_mean", "mhc_head",
            "mhc_abi_version", "mhc_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    ver = int(re.search(r"#define MHC_ABI_VERSION (\d+)", HEADER.read_text()).group(1))
    assert mhc.abi_version() == ver
    assert mhc.status_string(0) == "success"
    for s in (1, 2, 3):
        assert mhc.status_string(s) not in ("success", "unknown status")
    assert mhc.status_string(99) == "unknown status"


def test_workspace_bytes():
    assert mhc.mhc_pre_fused_workspace_bytes(0, 7168) == 0
    assert mhc.mhc_pre_fused_workspace_bytes(16, 0) == 0
    assert mhc.mhc_pre_fused_workspace_bytes(16, (1 << 21) + 8) == 0
    a = mhc.mhc_pre_fused_workspace_bytes(16, 256)
    b = mhc.mhc_pre_fused_workspace_bytes(8192, 7168)
    assert a > 0 and b > a and b % 256 == 0
    # the per-token partial records stay a small fraction of the streams
    assert b < 0.125 * 8192 * 4 * 7168 * 2


def test_sinkhorn_validation():
    lib = mhc.lib()
    assert lib.mhc_sinkhorn(FAKE, FAKE2, -1, 20, 1e-6, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_sinkhorn(FAKE, FAKE2, 10, 0, 1e-6, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_sinkhorn(FAKE, FAKE2, 10, 20, 0.0, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_sinkhorn(FAKE, FAKE2, 10, 20, float("nan"), NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_sinkhorn(NULL, FAKE2, 10, 20, 1e-6, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    # partial overlap of out and logits
    assert lib.mhc_sinkhorn(FAKE, ctypes.c_void_p(0x10000 + 64), 10, 20, 1e-6, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_sinkhorn(NULL, NULL, 0, 20, 1e-6, NULL) == mhc.MHC_SUCCESS  # empty: no-op


def _pre(lib, **kw):
    a = dict(res=FAKE, fn=ctypes.c_void_p(0x4000000), sc=ctypes.c_void_p(0x8000000), base=ctypes.c_void_p(0x8001000),
             T=16, H=256, rms=1e-6, pe=1e-6, se=1e-6, pm=1.0, it=20, y=ctypes.c_void_p(0x9000000),
             post=ctypes.c_void_p(0xA000000), comb=ctypes.c_void_p(0xB000000), pre=None,
             ws=ctypes.c_void_p(0xC000000), wsb=1 << 30)
    a.update(kw)
    return lib.mhc_pre_fused(a["res"], a["fn"], a["sc"], a["base"], a["T"], a["H"], a["rms"], a["pe"], a["se"],
                             a["pm"], a["it"], a["y"], a["post"], a["comb"], a["pre"], a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(H=(1 << 21) + 8), dict(it=0), dict(rms=0.0), dict(se=-1e-6), dict(pe=-1.0),
    dict(rms=float("inf")), dict(pm=float("nan")), dict(res=None), dict(fn=None), dict(sc=None),
    dict(base=None), dict(y=None), dict(post=None), dict(comb=None),
    dict(y=ctypes.c_void_p(0x10000 + 100)),           # y overlaps res
    dict(comb=ctypes.c_void_p(0xA000000 + 32)),        # comb overlaps post
    dict(pre=ctypes.c_void_p(0xB000000)),              # pre overlaps comb
])
def test_pre_validation_invalid(kw):
    assert _pre(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_pre_validation_workspace():
    lib = mhc.lib()
    # every form needs more than the weight split's place: the two-pass form keeps partial
    # sums behind it, the small-batch form its exchange records (which of the two a call
    # takes depends on the device, so the bound tested is below both)
    assert _pre(lib, wsb=mhc.mhc_pre_split_bytes(256)) == mhc.MHC_ERROR_WORKSPACE
    assert mhc.mhc_pre_fused_workspace_bytes(16, 256) > mhc.mhc_pre_split_bytes(256)
    assert _pre(lib, ws=None) == mhc.MHC_ERROR_WORKSPACE
    assert _pre(lib, ws=ctypes.c_void_p(0xC000000 + 8)) == mhc.MHC_ERROR_WORKSPACE  # not 256-byte aligned
    assert _pre(lib, T=0, res=None, y=None, ws=None) == mhc.MHC_SUCCESS  # empty: no-op


def _pre_noalloc(lib, **kw):
    G = 1 << 40  # fake addresses 1 TiB apart: no overlap at any size used here
    a = dict(res=ctypes.c_void_p(G), fn=ctypes.c_void_p(2 * G), sc=ctypes.c_void_p(3 * G), base=ctypes.c_void_p(4 * G),
             T=16, H=256, rms=1e-6, pe=1e-6, se=1e-6, pm=1.0, it=20, y=ctypes.c_void_p(5 * G),
             post=ctypes.c_void_p(6 * G), comb=ctypes.c_void_p(7 * G), pre=None)
    a.update(kw)
    return lib.mhc_pre_fused_noalloc(a["res"], a["fn"], a["sc"], a["base"], a["T"], a["H"], a["rms"], a["pe"],
                                     a["se"], a["pm"], a["it"], a["y"], a["post"], a["comb"], a["pre"], NULL)


def test_pre_noalloc_limit_matches_header():
    m = re.search(r"#define\s+MHC_PRE_FUSED_NOALLOC_MAX_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", HEADER.read_text())
    assert m and int(m.group(1)) << int(m.group(2)) == mhc.MHC_PRE_FUSED_NOALLOC_MAX_BYTES


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(it=0), dict(rms=0.0), dict(se=0.0), dict(pe=-1.0), dict(pm=float("nan")),
    dict(res=None), dict(fn=None), dict(y=None), dict(post=None), dict(comb=None),
    dict(y=ctypes.c_void_p((1 << 40) + 64)),           # y overlaps res
])
def test_pre_noalloc_validation_invalid(kw):
    assert _pre_noalloc(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_pre_noalloc_rejects_shapes_beyond_the_scratch():
    """Checked before any HIP call: these shapes always take the two-pass form (H above the
    one-read form's range, or a single-wave slice), whose workspace exceeds the scratch."""
    lib = mhc.lib()
    for T, H in [(2000, 16384), (20000, 1024)]:
        assert mhc.mhc_pre_fused_workspace_bytes(T, H) > mhc.MHC_PRE_FUSED_NOALLOC_MAX_BYTES
        assert _pre_noalloc(lib, T=T, H=H) == mhc.MHC_ERROR_WORKSPACE
    assert _pre_noalloc(lib, T=0, res=None, y=None) == mhc.MHC_SUCCESS  # empty: no-op


def _dots(lib, **kw):
    a = dict(dm=ctypes.c_void_p(0x1000000), sq=None, S=1, res=FAKE, sc=ctypes.c_void_p(0x8000000),
             base=ctypes.c_void_p(0x8001000), T=16, H=256, k=1024.0, rms=1e-6, pe=1e-6, se=1e-6, pm=1.0, it=20,
             y=ctypes.c_void_p(0x9000000), post=ctypes.c_void_p(0xA000000), comb=ctypes.c_void_p(0xB000000),
             pre=None)
    a.update(kw)
    return lib.mhc_pre_from_dots(a["dm"], a["sq"], a["S"], a["res"], a["sc"], a["base"], a["T"], a["H"], a["k"],
                                 a["rms"], a["pe"], a["se"], a["pm"], a["it"], a["y"], a["post"], a["comb"],
                                 a["pre"], NULL)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(S=0), dict(S=65537), dict(k=0.0), dict(k=float("inf")), dict(it=0),
    dict(rms=0.0), dict(se=0.0), dict(pe=-1.0), dict(pm=float("nan")), dict(dm=None), dict(res=None),
    dict(sc=None), dict(base=None), dict(y=None), dict(post=None), dict(comb=None),
    dict(y=ctypes.c_void_p(0x10000 + 64)),                     # y overlaps res
    dict(post=ctypes.c_void_p(0x1000000 + 32)),                # post overlaps dot_mix
    dict(sq=ctypes.c_void_p(0xA000000 - 8), S=1),             # sqrsum overlaps post
    dict(pre=ctypes.c_void_p(0xB000000 + 16)),                 # pre overlaps comb
])
def test_pre_from_dots_validation_invalid(kw):
    assert _dots(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_pre_from_dots_empty_is_a_no_op():
    assert _dots(mhc.lib(), T=0, dm=None, res=None, y=None, post=None, comb=None) == mhc.MHC_SUCCESS


def test_post_validation():
    lib = mhc.lib()
    x, res, post, comb, out = (ctypes.c_void_p(v) for v in (0x100000, 0x200000, 0x300000, 0x310000, 0x400000))
    call = lambda **k: lib.mhc_post(k.get("x", x), k.get("res", res), k.get("post", post), k.get("comb", comb),
                                    k.get("T", 8), k.get("H", 64), k.get("out", out), NULL)
    E = mhc.MHC_ERROR_INVALID_VALUE
    assert call(T=-1) == E
    assert call(H=0) == E
    for name in ("x", "res", "post", "comb", "out"):
        assert call(**{name: None}) == E
    assert call(out=ctypes.c_void_p(0x200000 + 2)) == E  # partial overlap with res
    assert call(out=ctypes.c_void_p(0x100000 - 64)) == E  # overlaps x
    assert call(T=0, x=None, res=None, post=None, comb=None, out=None) == mhc.MHC_SUCCESS


def test_sinkhorn_backward_validation():
    lib = mhc.lib()
    g, lg, d = FAKE, FAKE2, ctypes.c_void_p(0x30000000)
    E = mhc.MHC_ERROR_INVALID_VALUE
    call = lambda **k: lib.mhc_sinkhorn_backward(k.get("g", g), k.get("lg", lg), k.get("n", 10), k.get("it", 20),
                                                 k.get("eps", 1e-6), k.get("d", d), NULL)
    assert call(n=-1) == E
    assert call(n=(1 << 32) + 1) == E
    assert call(it=0) == E
    header_max = int(re.search(r"#define MHC_SINKHORN_BWD_MAX_ITERS (\d+)", HEADER.read_text()).group(1))
    assert header_max == mhc.SINKHORN_BWD_MAX_ITERS
    assert call(it=header_max + 1) == E
    assert call(eps=0.0) == E
    assert call(eps=float("inf")) == E
    for name in ("g", "lg", "d"):
        assert call(**{name: None}) == E
    assert call(d=ctypes.c_void_p(0x10000 + 4)) == E          # partial overlap with grad
    assert call(d=ctypes.c_void_p(0x20000000 - 64)) == E      # partial overlap with logits
    assert call(n=0, g=None, lg=None, d=None) == mhc.MHC_SUCCESS


def test_post_backward_validation():
    lib = mhc.lib()
    base = dict(go=0x100000, x=0x200000, res=0x300000, post=0x400000, comb=0x410000, dx=0x500000, dr=0x600000,
                dp=0x700000, dc=0x710000)
    E = mhc.MHC_ERROR_INVALID_VALUE

    def call(T=8, H=64, **k):
        a = {n: ctypes.c_void_p(v) if v is not None else None for n, v in {**base, **k}.items()}
        return lib.mhc_post_backward(a["go"], a["x"], a["res"], a["post"], a["comb"], T, H, a["dx"], a["dr"],
                                     a["dp"], a["dc"], NULL)

    assert call(T=-1) == E
    assert call(H=0) == E
    for name in base:
        assert call(**{name: None}) == E
    assert call(dr=0x100000 + 2) == E      # d_res overlaps d_out without being it
    assert call(dr=0x300000) == E          # d_res is res (only d_out may be updated in place)
    assert call(dx=0x200000) == E          # d_x is x
    assert call(dx=0x600000 + 128) == E    # d_x overlaps d_res
    assert call(dp=0x710000 - 64) == E     # d_post overlaps d_comb
    assert call(dc=0x410000) == E          # d_comb is comb
    assert call(T=0, **{n: None for n in base}) == mhc.MHC_SUCCESS


def _dbwd(lib, **kw):
    a = dict(dy=0x100000, dpost=0x200000, dcomb=0x210000, dm=0x300000, sq=None, S=1, res=0x400000,
             sc=0x500000, base=0x500100, T=8, H=64, k=256.0, rms=1e-6, pe=1e-6, se=1e-6, pm=1.0, it=20,
             dres=0x600000, ddot=0x700000, dsq=None, dsc=0x800000, dbase=0x800100, ws=0x900000, wsb=1 << 20)
    a.update(kw)
    v = lambda n: ctypes.c_void_p(a[n]) if a[n] is not None else None
    return lib.mhc_pre_from_dots_backward(v("dy"), v("dpost"), v("dcomb"), v("dm"), v("sq"), a["S"], v("res"),
                                          v("sc"), v("base"), a["T"], a["H"], a["k"], a["rms"], a["pe"], a["se"],
                                          a["pm"], a["it"], v("dres"), v("ddot"), v("dsq"), v("dsc"), v("dbase"),
                                          v("ws"), a["wsb"], NULL)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(S=0), dict(S=65537), dict(it=0), dict(it=256), dict(k=0.0), dict(rms=0.0),
    dict(se=0.0), dict(pe=-1.0), dict(pm=float("inf")), dict(dy=None), dict(dpost=None), dict(dcomb=None),
    dict(dm=None), dict(res=None), dict(sc=None), dict(base=None), dict(dres=None), dict(ddot=None),
    dict(dsc=None), dict(dbase=None), dict(T=0, dsc=None),
    dict(sq=0x380000),                              # sqrsum given without d_sqrsum
    dict(dres=0x400000 + 64),                       # d_res overlaps res without being it
    dict(ddot=0x300000 + 32),                       # d_dot overlaps dot_mix
    dict(dbase=0x800000 + 8),                       # d_hc_base overlaps d_hc_scale
    dict(ws=0x600000 + 256),                        # workspace overlaps d_res
])
def test_pre_from_dots_backward_validation_invalid(kw):
    assert _dbwd(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_pre_from_dots_backward_workspace():
    lib = mhc.lib()
    need = mhc.mhc_pre_backward_workspace_bytes(8)
    assert need >= 8 * 28 * 4 and need % 256 == 0
    assert mhc.mhc_pre_backward_workspace_bytes(0) == 0
    assert _dbwd(lib, wsb=need - 1) == mhc.MHC_ERROR_WORKSPACE
    assert _dbwd(lib, ws=None) == mhc.MHC_ERROR_WORKSPACE
    assert _dbwd(lib, ws=0x900000 + 16) == mhc.MHC_ERROR_WORKSPACE


def test_expand_and_head_mean_validation():
    lib = mhc.lib()
    E = mhc.MHC_ERROR_INVALID_VALUE
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    for fn in (lib.mhc_expand, lib.mhc_head_mean):
        assert fn(a, -1, 64, b, NULL) == E
        assert fn(a, 8, 0, b, NULL) == E
        assert fn(None, 8, 64, b, NULL) == E
        assert fn(a, 8, 64, None, NULL) == E
        assert fn(None, 0, 64, None, NULL) == mhc.MHC_SUCCESS
    assert lib.mhc_expand(a, 8, 64, ctypes.c_void_p(0x100000 + 512), NULL) == E     # streams overlap hidden
    assert lib.mhc_head_mean(a, 8, 64, ctypes.c_void_p(0x100000 + 512), NULL) == E  # y overlaps res


def _head(lib, **kw):
    a = dict(res=0x100000, fn=0x4000000, sc=0x8000000, base=0x8001000, T=16, H=256, ne=1e-6, he=1e-6,
             y=0x9000000, pre=None, ws=0xC000000, wsb=1 << 30)
    a.update(kw)
    v = lambda n: ctypes.c_void_p(a[n]) if a[n] is not None else None
    return lib.mhc_head(v("res"), v("fn"), v("sc"), v("base"), a["T"], a["H"], a["ne"], a["he"], v("y"), v("pre"),
                        v("ws"), a["wsb"], NULL)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(H=(1 << 21) + 8), dict(ne=0.0), dict(he=-1.0), dict(ne=float("nan")),
    dict(res=None), dict(fn=None), dict(sc=None), dict(base=None), dict(y=None),
    dict(y=0x100000 + 64),                  # y overlaps res
    dict(pre=0x8001000 + 4),                # pre overlaps hc_base (4 floats)
    dict(y=0x4000000 + 1024),               # y overlaps hc_fn ([4, 4H] fp32 = 16 KB)
])
def test_head_validation_invalid(kw):
    assert _head(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_head_workspace_and_bf16_pre_validation():
    lib = mhc.lib()
    small = mhc.mhc_pre_split_bytes(256)  # below what either small-batch form needs
    assert _head(lib, wsb=small) == mhc.MHC_ERROR_WORKSPACE
    assert _head(lib, ws=None) == mhc.MHC_ERROR_WORKSPACE
    assert _head(lib, T=0, res=None, y=None, ws=None) == mhc.MHC_SUCCESS
    # mhc_pre_fused_bf16 shares mhc_pre_fused's checks; bf16 weights are [24, 4H] x 2 bytes
    f = lambda **k: lib.mhc_pre_fused_bf16(ctypes.c_void_p(0x10000), ctypes.c_void_p(k.get("fn", 0x4000000)),
                                           ctypes.c_void_p(0x8000000), ctypes.c_void_p(0x8001000), 16, 256, 1e-6,
                                           1e-6, 1e-6, 1.0, k.get("it", 20), ctypes.c_void_p(k.get("y", 0x9000000)),
                                           ctypes.c_void_p(0xA000000), ctypes.c_void_p(0xB000000), None,
                                           ctypes.c_void_p(0xC000000), k.get("wsb", 1 << 30), NULL)
    assert f(it=0) == mhc.MHC_ERROR_INVALID_VALUE
    assert f(y=0x4000000 + 24 * 1024 * 2 - 64) == mhc.MHC_ERROR_INVALID_VALUE   # y overlaps the bf16 weights
    assert f(wsb=small) == mhc.MHC_ERROR_WORKSPACE


def _fbwd(lib, **kw):
    a = dict(dy=0x100000, dpost=0x200000, dcomb=0x210000, res=0x400000, fn=0x1000000, sc=0x500000,
             base=0x500100, T=8, H=64, rms=1e-6, pe=1e-6, se=1e-6, pm=1.0, it=20, dres=0x600000,
             dfn=0x2000000, dsc=0x800000, dbase=0x800100, ws=0x9000000, wsb=1 << 30)
    a.update(kw)
    v = lambda n: ctypes.c_void_p(a[n]) if a[n] is not None else None
    return lib.mhc_pre_fused_backward(v("dy"), v("dpost"), v("dcomb"), v("res"), v("fn"), v("sc"), v("base"),
                                      a["T"], a["H"], a["rms"], a["pe"], a["se"], a["pm"], a["it"], v("dres"),
                                      v("dfn"), v("dsc"), v("dbase"), v("ws"), a["wsb"], NULL)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(H=60), dict(H=(1 << 21) + 8), dict(it=0), dict(it=256), dict(rms=0.0),
    dict(se=0.0), dict(pe=-1.0), dict(pm=float("nan")), dict(dy=None), dict(dpost=None), dict(dcomb=None),
    dict(res=None), dict(fn=None), dict(sc=None), dict(base=None), dict(dres=None), dict(dfn=None),
    dict(dsc=None), dict(dbase=None), dict(T=0, dfn=None),
    dict(dy=0x100000 + 8),                  # dy not 16-byte aligned
    dict(dres=0x400000 + 64),               # d_res overlaps res without being it
    dict(dfn=0x1000000 + 1024),             # d_hc_fn overlaps hc_fn
    dict(dbase=0x800000 + 4),               # d_hc_base overlaps d_hc_scale
    dict(ws=0x600000 + 256),                # workspace overlaps d_res
])
def test_pre_fused_backward_validation_invalid(kw):
    assert _fbwd(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_pre_fused_backward_workspace():
    lib = mhc.lib()
    need = mhc.mhc_pre_fused_backward_workspace_bytes(8, 64)
    # the weight split, the recompute's partial sums and the reverse's own sums
    assert need > mhc.mhc_pre_split_bytes(64) and need % 256 == 0
    assert mhc.mhc_pre_fused_backward_workspace_bytes(8, 60) == 0
    assert mhc.mhc_pre_fused_backward_workspace_bytes(0, 64) == 0
    assert _fbwd(lib, wsb=need - 1) == mhc.MHC_ERROR_WORKSPACE
    assert _fbwd(lib, ws=None) == mhc.MHC_ERROR_WORKSPACE
    assert _fbwd(lib, ws=0x9000000 + 16) == mhc.MHC_ERROR_WORKSPACE


def _pproj(lib, **kw):
    # every case below turns one argument invalid: validation fails before any launch
    a = dict(x=0x100000, res=0x400000, post=0x200000, comb=0x210000, fn=0x1000000, T=8, H=64, out=0x600000,
             dm=0x2000000, sq=0x800000, ws=0x9000000, wsb=1 << 30)
    a.update(kw)
    v = lambda n: ctypes.c_void_p(a[n]) if a[n] is not None else None
    return lib.mhc_post_project(v("x"), v("res"), v("post"), v("comb"), v("fn"), a["T"], a["H"], v("out"), v("dm"),
                                v("sq"), v("ws"), a["wsb"], NULL)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(H=60), dict(H=(1 << 21) + 8), dict(x=None), dict(res=None), dict(post=None),
    dict(comb=None), dict(fn=None), dict(out=None), dict(dm=None), dict(sq=None), dict(x=0x100000 + 8),
    dict(res=0x400000 + 8), dict(out=0x600000 + 8), dict(out=0x400000 + 16), dict(out=0x100000),
    dict(dm=0x400000), dict(sq=0x2000000 + 16), dict(dm=0x1000000), dict(ws=0x600000),
])
def test_post_project_validation_invalid(kw):
    assert _pproj(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_post_project_workspace():
    lib = mhc.lib()
    need = mhc.mhc_post_project_workspace_bytes(8, 64)
    assert need > 0 and need % 256 == 0
    assert mhc.mhc_post_project_workspace_bytes(8, 60) == 0 and mhc.mhc_post_project_workspace_bytes(0, 64) == 0
    # laid out as the two-pass pre-map's: the split weights and one token chunk's partial
    # records (the pre-map's own size also covers its other forms, so it is never smaller)
    for T, H in ((8, 64), (3000, 1000), (8192, 7168)):
        assert mhc.mhc_post_project_workspace_bytes(T, H) <= mhc.mhc_pre_fused_workspace_bytes(T, H)
    assert mhc.mhc_post_project_workspace_bytes(3000, 1000) == mhc.mhc_pre_fused_workspace_bytes(3000, 1000)
    assert _pproj(lib, wsb=need - 1) == mhc.MHC_ERROR_WORKSPACE
    assert _pproj(lib, ws=None) == mhc.MHC_ERROR_WORKSPACE
    assert _pproj(lib, ws=0x9000000 + 16) == mhc.MHC_ERROR_WORKSPACE
    # T == 0: nothing to do, no pointer is looked at
    assert _pproj(lib, T=0, x=None, res=None, post=None, comb=None, fn=None, out=None, dm=None, sq=None,
                  ws=None, wsb=0) == mhc.MHC_SUCCESS


def _postpre(lib, **kw):
    # every case below turns one argument invalid: validation fails before any launch
    a = dict(x=0x100000, res=0x400000, post=0x200000, comb=0x210000, fn=0x1000000, sc=0x300000, base=0x310000, T=8,
             H=64, rms=1e-6, pre_eps=1e-6, sk=1e-6, pm=1.0, iters=20, out=0x600000, y=0x700000, pn=0x800000,
             cn=0x810000, pre=0x820000, ws=0x9000000, wsb=1 << 30)
    a.update(kw)
    v = lambda n: ctypes.c_void_p(a[n]) if a[n] is not None else None
    return lib.mhc_post_pre_fused(v("x"), v("res"), v("post"), v("comb"), v("fn"), v("sc"), v("base"), a["T"], a["H"],
                                  a["rms"], a["pre_eps"], a["sk"], a["pm"], a["iters"], v("out"), v("y"), v("pn"),
                                  v("cn"), v("pre"), v("ws"), a["wsb"], NULL)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(iters=0), dict(rms=0.0), dict(sk=0.0), dict(pre_eps=-1.0), dict(pm=float("inf")),
    dict(x=None), dict(res=None), dict(post=None), dict(comb=None), dict(fn=None), dict(sc=None), dict(base=None),
    dict(out=None), dict(y=None), dict(pn=None), dict(cn=None),
    dict(out=0x400000 + 16), dict(out=0x100000), dict(out=0x200000), dict(out=0x1000000), dict(out=0x300000),
    dict(y=0x400000), dict(y=0x600000 + 64), dict(y=0x100000), dict(pn=0x200000), dict(cn=0x210000 + 64),
    dict(pre=0x200000), dict(pn=0x810000), dict(ws=0x100000), dict(ws=0x400000), dict(ws=0x1000000),
])
def test_post_pre_fused_validation_invalid(kw):
    assert _postpre(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_post_pre_fused_workspace():
    lib = mhc.lib()
    assert _postpre(lib, wsb=mhc.mhc_pre_split_bytes(64)) == mhc.MHC_ERROR_WORKSPACE  # below every form's need
    assert _postpre(lib, ws=None) == mhc.MHC_ERROR_WORKSPACE
    assert _postpre(lib, ws=0x9000000 + 16) == mhc.MHC_ERROR_WORKSPACE
    # T == 0: nothing to do, no pointer is looked at
    assert _postpre(lib, T=0, x=None, res=None, post=None, comb=None, fn=None, sc=None, base=None, out=None, y=None,
                    pn=None, cn=None, pre=None, ws=None, wsb=0) == mhc.MHC_SUCCESS


def test_binding_rejects_cpu_tensors_before_the_library():
    import torch
    with pytest.raises(ValueError):
        mhc.mhc_post(torch.zeros(2, 8, dtype=torch.bfloat16), torch.zeros(2, 4, 8, dtype=torch.bfloat16),
                     torch.zeros(2, 4), torch.zeros(2, 4, 4))
    with pytest.raises(ValueError):
        mhc.mhc_post_project(torch.zeros(2, 8, dtype=torch.bfloat16), torch.zeros(2, 4, 8, dtype=torch.bfloat16),
                             torch.zeros(2, 4), torch.zeros(2, 4, 4), torch.zeros(24, 32))
    with pytest.raises(ValueError):
        mhc.mhc_post_pre_fused(torch.zeros(2, 8, dtype=torch.bfloat16), torch.zeros(2, 4, 8, dtype=torch.bfloat16),
                               torch.zeros(2, 4), torch.zeros(2, 4, 4), torch.zeros(24, 32), torch.ones(3),
                               torch.zeros(24))
    with pytest.raises(ValueError):
        mhc.mhc_sinkhorn(torch.zeros(3, 4, 4))
    with pytest.raises(ValueError):
        mhc.mhc_sinkhorn_backward(torch.zeros(3, 4, 4), torch.zeros(3, 4, 4))
    with pytest.raises(ValueError):
        mhc.mhc_post_backward(torch.zeros(2, 4, 8, dtype=torch.bfloat16), torch.zeros(2, 8, dtype=torch.bfloat16),
                              torch.zeros(2, 4, 8, dtype=torch.bfloat16), torch.zeros(2, 4), torch.zeros(2, 4, 4))


PLAN_ENTRIES = ["post", "expand", "head_mean", "pre_fused", "collapse", "pre_from_dots", "pre_from_dots_backward",
                "post_backward", "sinkhorn", "sinkhorn_backward", "post_f32", "expand_f32", "head_mean_f32"]


@pytest.mark.parametrize("entry", PLAN_ENTRIES)
@pytest.mark.parametrize("vec8", [True, False])
def test_launch_plan_keeps_every_launch_below_the_grid_limit(entry, vec8):
    """Host grid arithmetic only (no GPU): at the largest sizes validation accepts, every
    launch covers fewer than 2^31 work-items (a grid dimension must stay below 2^32) and
    at most 2^24 tokens, and the launches cover all T tokens."""
    sizes = [(1 << 27, 8), ((1 << 29) - 1, 64), (1 << 22, 1000), (825_000, 6400), (8192, 7168), (300, 1 << 21),
             (1, 1 << 21), (1, 1), (0, 64)]
    if entry.startswith("sinkhorn"):
        sizes = [(1 << 32, 1), ((1 << 40), 1), (1 << 20, 1), (1, 1), (0, 1)]
    for T, H in sizes:
        p = mhc.launch_plan(entry, T, H, vec8)
        assert p["max_items"] < 1 << 31, (entry, T, H, p)
        assert 1 <= p["tokens_per_launch"] <= 1 << 24, (entry, T, H, p)
        assert p["launches"] * p["tokens_per_launch"] >= T > (p["launches"] - 1) * p["tokens_per_launch"] or T == 0, \
            (entry, T, H, p)
        # per-token offsets of 24 fp32 (t * 24) inside one launch stay int-exact
        assert p["tokens_per_launch"] * 24 < 1 << 31


def test_launch_plan_cases_from_the_review():
    """T = 2^27 at H = 8 splits the post-map into launches of 2^24 tokens (its coefficient
    offsets t * 16 stay below 2^28), and 2^32 Sinkhorn matrices into 256 launches."""
    p = mhc.launch_plan("post", 1 << 27, 8, True)
    assert p == {"launches": 8, "tokens_per_launch": 1 << 24, "max_items": (1 << 24) * 64}
    p = mhc.launch_plan("post", 1 << 27, 8, False)
    assert p["launches"] == 8 and p["max_items"] == (1 << 24) * 64
    p = mhc.launch_plan("sinkhorn", 1 << 32, 1, True)
    assert p == {"launches": 256, "tokens_per_launch": 1 << 24, "max_items": 1 << 24}
    p = mhc.launch_plan("sinkhorn_backward", 1 << 32, 1, True)
    assert p["launches"] == 256 and p["max_items"] == (1 << 24) * 16
    # a scalar collapse at T = 825 000, H = 6400 (42 GB of streams) would need 5.3e9
    # work-items in one launch; the pre-map's chunks keep it below 2^31
    p = mhc.launch_plan("pre_fused", 825_000, 6400, False)
    assert p["launches"] >= 3 and p["max_items"] < 1 << 31


def test_launch_plan_rejects_bad_arguments():
    lib = mhc.lib()
    n = ctypes.c_int64()
    assert lib.mhc_launch_plan(b"nope", 1, 1, 1, ctypes.byref(n), ctypes.byref(n), ctypes.byref(n)) == \
        mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_launch_plan(b"post", -1, 1, 1, ctypes.byref(n), ctypes.byref(n), ctypes.byref(n)) == \
        mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_launch_plan(b"post", 1, 0, 1, ctypes.byref(n), ctypes.byref(n), ctypes.byref(n)) == \
        mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_launch_plan(b"post", 1, 1, 1, None, ctypes.byref(n), ctypes.byref(n)) == \
        mhc.MHC_ERROR_INVALID_VALUE


def _pre_f32(lib, **kw):
    G = 1 << 40
    a = dict(res=ctypes.c_void_p(G), fn=ctypes.c_void_p(2 * G), sc=ctypes.c_void_p(3 * G), base=ctypes.c_void_p(4 * G),
             T=16, H=256, rms=1e-6, pe=1e-6, se=1e-6, pm=1.0, it=20, y=ctypes.c_void_p(5 * G),
             post=ctypes.c_void_p(6 * G), comb=ctypes.c_void_p(7 * G), pre=None, ws=ctypes.c_void_p(8 * G),
             wsb=1 << 30)
    a.update(kw)
    return lib.mhc_pre_fused_f32(a["res"], a["fn"], a["sc"], a["base"], a["T"], a["H"], a["rms"], a["pe"], a["se"],
                                 a["pm"], a["it"], a["y"], a["post"], a["comb"], a["pre"], a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(H=(1 << 20) + 4), dict(it=0), dict(rms=0.0), dict(se=-1e-6), dict(pe=-1.0),
    dict(pm=float("nan")), dict(res=None), dict(fn=None), dict(sc=None), dict(base=None), dict(y=None),
    dict(post=None), dict(comb=None),
    dict(y=ctypes.c_void_p((1 << 40) + 16 * 4 * 256 * 4 - 8)),   # y overlaps the fp32 streams' last bytes
    dict(pre=ctypes.c_void_p(7 << 40)),                          # pre overlaps comb
])
def test_pre_f32_validation_invalid(kw):
    assert _pre_f32(mhc.lib(), **kw) == mhc.MHC_ERROR_INVALID_VALUE


def test_pre_f32_validation_workspace_and_empty():
    lib = mhc.lib()
    need = mhc.mhc_pre_fused_workspace_bytes(16, 256)
    assert _pre_f32(lib, wsb=need // 8) == mhc.MHC_ERROR_WORKSPACE
    assert _pre_f32(lib, ws=None) == mhc.MHC_ERROR_WORKSPACE
    assert _pre_f32(lib, ws=ctypes.c_void_p((8 << 40) + 64)) == mhc.MHC_ERROR_WORKSPACE  # not 256-byte aligned
    assert _pre_f32(lib, T=0, res=None, y=None, ws=None) == mhc.MHC_SUCCESS


def test_f32_stream_post_expand_head_validation():
    lib = mhc.lib()
    G = 1 << 40
    x, res, post, comb, out = (ctypes.c_void_p(k * G) for k in range(1, 6))
    assert lib.mhc_post_f32(x, res, post, comb, -1, 64, out, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_post_f32(x, res, post, comb, 8, (1 << 20) + 1, out, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_post_f32(None, res, post, comb, 8, 64, out, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    # out overlapping res partly (not exactly) is rejected; x overlapping out too
    assert lib.mhc_post_f32(x, res, post, comb, 8, 64, ctypes.c_void_p(G * 2 + 4), NULL) == \
        mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_post_f32(ctypes.c_void_p(5 * G + 8), res, post, comb, 8, 64, out, NULL) == \
        mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_post_f32(None, None, None, None, 0, 64, None, NULL) == mhc.MHC_SUCCESS
    assert lib.mhc_expand_f32(x, 8, 0, out, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_expand_f32(None, 8, 64, out, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_expand_f32(ctypes.c_void_p(5 * G + 16), 8, 64, out, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_head_mean_f32(res, 8, 64, None, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_head_mean_f32(res, 8, 64, ctypes.c_void_p(2 * G + 8), NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_head_mean_f32(None, 0, 64, None, NULL) == mhc.MHC_SUCCESS


def test_pre_split_weights_validation():
    lib = mhc.lib()
    G = 1 << 40
    fn, ws = ctypes.c_void_p(G), ctypes.c_void_p(2 * G)
    need = mhc.mhc_pre_split_bytes(7168)
    assert 0 < need <= mhc.mhc_pre_fused_workspace_bytes(32, 7168)
    assert mhc.mhc_pre_split_bytes(0) == 0 and mhc.mhc_pre_split_bytes((1 << 21) + 1) == 0
    assert lib.mhc_pre_split_weights(fn, 0, ws, need, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_pre_split_weights(None, 7168, ws, need, NULL) == mhc.MHC_ERROR_INVALID_VALUE
    assert lib.mhc_pre_split_weights(fn, 7168, ws, need - 1, NULL) == mhc.MHC_ERROR_WORKSPACE
    assert lib.mhc_pre_split_weights(fn, 7168, None, need, NULL) == mhc.MHC_ERROR_WORKSPACE
    assert lib.mhc_pre_split_weights(fn, 7168, ctypes.c_void_p(2 * G + 64), need, NULL) == mhc.MHC_ERROR_WORKSPACE
    assert lib.mhc_pre_split_weights(fn, 7168, ctypes.c_void_p(G + 256), need, NULL) == mhc.MHC_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(T=-1), dict(H=0), dict(it=0), dict(rms=0.0), dict(res=None), dict(y=None)])
def test_pre_fused_presplit_validation(kw):
    a = dict(res=FAKE, fn=ctypes.c_void_p(0x4000000), sc=ctypes.c_void_p(0x8000000), base=ctypes.c_void_p(0x8001000),
             T=16, H=256, rms=1e-6, pe=1e-6, se=1e-6, pm=1.0, it=20, y=ctypes.c_void_p(0x9000000),
             post=ctypes.c_void_p(0xA000000), comb=ctypes.c_void_p(0xB000000), pre=None,
             ws=ctypes.c_void_p(0xC000000), wsb=1 << 30)
    a.update(kw)
    assert mhc.lib().mhc_pre_fused_presplit(a["res"], a["fn"], a["sc"], a["base"], a["T"], a["H"], a["rms"], a["pe"],
                                            a["se"], a["pm"], a["it"], a["y"], a["post"], a["comb"], a["pre"],
                                            a["ws"], a["wsb"], NULL) == mhc.MHC_ERROR_INVALID_VALUE
