"""CPU oracle for the tree-flattened attention and forked Gated DeltaNet.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product path (the HIP library and
its binding) never imports this package.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over segment x head),
compiled by ``build()`` with gcc into two libraries from the same source:
``liboracle_f64.so`` (double, the parity reference) and ``liboracle_f32.so``
(float, the float32 reference for total-variation distance). See the header
of ``oracle.c`` for what is computed and where the pages define it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIBS = {"f64": os.path.join(_HERE, "liboracle_f64.so"),
         "f32": os.path.join(_HERE, "liboracle_f32.so")}
_REAL = {"f64": ("double", np.float64), "f32": ("float", np.float32)}
_loaded = {}


def build() -> None:
    """Compile both precisions of the oracle (no fast-math, no FMA contraction,
    so every sum runs in the order written)."""
    for prec, path in _LIBS.items():
        tmp = path + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", f"-DREAL={_REAL[prec][0]}", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
    _loaded.clear()


def _lib(prec: str):
    if prec not in _loaded:
        path = _LIBS[prec]
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(path)
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        rp = np.ctypeslib.ndpointer(_REAL[prec][1], flags="C_CONTIGUOUS")
        vp = ctypes.c_void_p
        c_int = ctypes.c_int
        lib.oracle_meta.argtypes = [c_int, i32p, i32p] + [i32p] * 7
        lib.oracle_meta_ctx.argtypes = [c_int, i32p, i32p, vp] + [i32p] * 7
        lib.oracle_attention_ctx.argtypes = [c_int, i32p, i32p, vp, vp, c_int, c_int, c_int,
                                             ctypes.c_double, f32p, f32p, f32p, vp, vp, vp, rp, vp]
        lib.oracle_mask.argtypes = [c_int, i32p, i32p, np.ctypeslib.ndpointer(np.uint8)]
        lib.oracle_attention.argtypes = [c_int, i32p, i32p, c_int, c_int, c_int, ctypes.c_double,
                                         f32p, f32p, f32p, vp, rp, vp]
        lib.oracle_gdn.argtypes = [c_int, i32p, i32p, c_int, c_int, c_int, ctypes.c_double,
                                   f32p, f32p, f32p, f32p, f32p, vp, vp, rp, vp, vp]
        lib.oracle_num_tokens.argtypes = [c_int, i32p, i32p, ctypes.POINTER(ctypes.c_longlong)]
        lib.oracle_rope.argtypes = [c_int, i32p, i32p, vp, c_int, c_int, ctypes.c_double, f32p, rp]
        lib.oracle_conv.argtypes = [c_int, i32p, i32p, c_int, c_int, c_int, f32p, f32p, vp, vp, rp]
        lib.oracle_set_threads.argtypes = [c_int]
        lib.oracle_max_threads.restype = c_int
        lib.oracle_real_bytes.restype = c_int
        assert lib.oracle_real_bytes() == np.dtype(_REAL[prec][1]).itemsize
        _loaded[prec] = lib
    return _loaded[prec]


class OracleError(RuntimeError):
    pass


def _tree(parent, seg_len):
    return (np.ascontiguousarray(parent, np.int32), np.ascontiguousarray(seg_len, np.int32))


def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle rejected the input (code {rc})")


def set_threads(n: int, prec: str = "f64") -> None:
    _lib(prec).oracle_set_threads(int(n))


def max_threads(prec: str = "f64") -> int:
    return int(_lib(prec).oracle_max_threads())


def num_tokens(parent, seg_len) -> int:
    parent, seg_len = _tree(parent, seg_len)
    T = ctypes.c_longlong(0)
    _check(_lib("f64").oracle_num_tokens(len(parent), parent, seg_len, ctypes.byref(T)))
    return int(T.value)


def meta(parent, seg_len, ctx_len=None) -> dict:
    """Segment and token index arrays (int32), see ``oracle_meta``; with
    ``ctx_len`` ([S], roots only) the positions count resumed contexts
    (``oracle_meta_ctx``)."""
    parent, seg_len = _tree(parent, seg_len)
    S = len(parent)
    T = num_tokens(parent, seg_len)
    out = {n: np.zeros(S, np.int32) for n in ("seg_start", "depth", "root", "anc_len")}
    out.update({n: np.zeros(T, np.int32) for n in ("tok_seg", "tok_pos", "tok_iso_pos")})
    cl = None if ctx_len is None else np.ascontiguousarray(ctx_len, np.int32)
    _check(_lib("f64").oracle_meta_ctx(S, parent, seg_len, None if cl is None else cl.ctypes.data,
                                       out["seg_start"], out["depth"], out["root"],
                                       out["anc_len"], out["tok_seg"], out["tok_pos"],
                                       out["tok_iso_pos"]))
    return out


def mask(parent, seg_len) -> np.ndarray:
    """Dense [T, T] uint8 visibility mask of the flattened stream."""
    parent, seg_len = _tree(parent, seg_len)
    T = num_tokens(parent, seg_len)
    m = np.zeros((T, T), np.uint8)
    _check(_lib("f64").oracle_mask(len(parent), parent, seg_len, m))
    return m


def attention(parent, seg_len, q, k, v, scale: Optional[float] = None, prec: str = "f64",
              tok_select: Optional[np.ndarray] = None, ctx_start=None, ctx_len=None, kc=None,
              vc=None):
    """Tree attention by isolated per-segment sequences.
    q [T,H,D], k/v [T,Hkv,D] float32. Returns (o [T,H,D], lse [T,H]) in the
    oracle's precision; rows outside ``tok_select`` are NaN. Resumed contexts:
    ctx_start/ctx_len [S] (roots only) index rows of kc/vc [C,Hkv,D] that
    precede the root's tokens (``oracle_attention_ctx``)."""
    parent, seg_len = _tree(parent, seg_len)
    q = np.ascontiguousarray(q, np.float32)
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    T, H, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rt = _REAL[prec][1]
    o = np.full((T, H, D), np.nan, rt)
    lse = np.full((T, H), np.nan, rt)
    sel = None
    if tok_select is not None:
        sel = np.ascontiguousarray(tok_select, np.uint8)
        assert sel.shape == (T,)
    cs = cl = kcc = vcc = None
    if ctx_len is not None:
        cs = np.ascontiguousarray(ctx_start, np.int32)
        cl = np.ascontiguousarray(ctx_len, np.int32)
        kcc = np.ascontiguousarray(kc, np.float32)
        vcc = np.ascontiguousarray(vc, np.float32)
        assert cs.shape == cl.shape == (len(parent),) and kcc.shape == vcc.shape
        assert kcc.shape[1:] == (Hkv, D) and int((cs + cl).max(initial=0)) <= kcc.shape[0]
    ptr = lambda x: None if x is None else x.ctypes.data
    _check(_lib(prec).oracle_attention_ctx(len(parent), parent, seg_len, ptr(cs), ptr(cl), H, Hkv,
                                           D, float(scale), q, k, v, ptr(kcc), ptr(vcc),
                                           None if sel is None else sel.ctypes.data, o,
                                           lse.ctypes.data))
    return o, lse


def gdn(parent, seg_len, q, k, v, a, b, root_state=None, scale: float = 1.0, prec: str = "f64",
        seg_select: Optional[np.ndarray] = None):
    """Forked Gated DeltaNet by isolated per-segment recurrences.
    Returns (o [T,H,dv], seg_start_state [S,H,dv,dk], seg_final_state [S,H,dv,dk]);
    entries of unselected segments are NaN."""
    parent, seg_len = _tree(parent, seg_len)
    q = np.ascontiguousarray(q, np.float32)
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    T, H, dk = q.shape
    dv = v.shape[2]
    S = len(parent)
    rt = _REAL[prec][1]
    o = np.full((T, H, dv), np.nan, rt)
    st0 = np.full((S, H, dv, dk), np.nan, rt)
    st1 = np.full((S, H, dv, dk), np.nan, rt)
    rs = None
    if root_state is not None:
        rs = np.ascontiguousarray(root_state, np.float32)
        assert rs.shape == (int((parent < 0).sum()), H, dv, dk)
    sel = None
    if seg_select is not None:
        sel = np.ascontiguousarray(seg_select, np.uint8)
        assert sel.shape == (S,)
    _check(_lib(prec).oracle_gdn(S, parent, seg_len, H, dk, dv, float(scale), q, k, v, a, b,
                                 None if rs is None else rs.ctypes.data,
                                 None if sel is None else sel.ctypes.data, o,
                                 st0.ctypes.data, st1.ctypes.data))
    return o, st0, st1


def rope(parent, seg_len, x, theta: float = 10000.0, ctx_len=None, prec: str = "f64"):
    """Rotary position embedding at the isolated positions (``oracle_rope``).
    x [T,nh,D] float32 -> [T,nh,D] in the oracle's precision."""
    parent, seg_len = _tree(parent, seg_len)
    x = np.ascontiguousarray(x, np.float32)
    T, nh, D = x.shape
    y = np.full((T, nh, D), np.nan, _REAL[prec][1])
    cl = None if ctx_len is None else np.ascontiguousarray(ctx_len, np.int32)
    _check(_lib(prec).oracle_rope(len(parent), parent, seg_len, None if cl is None else cl.ctypes.data,
                                  nh, D, float(theta), x, y))
    return y


def conv(parent, seg_len, x, w, bias=None, conv_state=None, act: int = 1, prec: str = "f64"):
    """Causal depthwise convolution along the isolated sequences
    (``oracle_conv``). x [T,C], w [C,K], bias [C], conv_state [R,C,K-1]."""
    parent, seg_len = _tree(parent, seg_len)
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    T, C = x.shape
    K = w.shape[1]
    assert w.shape == (C, K)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    cs = None if conv_state is None else np.ascontiguousarray(conv_state, np.float32)
    if cs is not None:
        assert cs.shape == (int((parent < 0).sum()), C, K - 1)
    y = np.full((T, C), np.nan, _REAL[prec][1])
    _check(_lib(prec).oracle_conv(len(parent), parent, seg_len, C, K, int(act), x, w,
                                  None if b is None else b.ctypes.data,
                                  None if cs is None else cs.ctypes.data, y))
    return y
