"""ctypes binding of libforkattn.so (include/fork.h), argument marshalling only.

Every function keeps the C name and argument order; tensors are passed as
torch tensors (device or pinned host memory, contiguous) or raw integer
addresses, streams as torch streams, raw handles or None (torch's current
stream). A negative status raises ForkError carrying fork_last_error(). There
is no fallback: if the library is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libforkattn.so")

FORK_F32, FORK_BF16 = 0, 1
STATUS = {0: "FORK_OK", -1: "FORK_E_ARG", -2: "FORK_E_TREE", -3: "FORK_E_UNSUPPORTED",
          -4: "FORK_E_WORKSPACE", -5: "FORK_E_CAPACITY", -6: "FORK_E_HIP", -7: "FORK_E_DEVICE"}
FORK_DEVERR_MAGIC, FORK_DEVERR_CAPACITY = 1, 2
(ARR_TOK_SEG, ARR_TOK_POS, ARR_TOK_ISO_POS, ARR_SEG_START, ARR_DEPTH, ARR_ANC_LEN, ARR_ROOT,
 ARR_CTX_START, ARR_CTX_LEN) = range(9)

# every symbol include/fork.h declares
EXPORTS = ("fork_meta_size", "fork_meta_build", "fork_meta_plan", "fork_meta_build_ctx",
           "fork_meta_plan_ctx", "fork_meta_export", "fork_meta_check",
           "fork_meta_dense_mask", "fork_attn_workspace", "fork_attn_forward", "fork_attn_forward_ctx", "fork_attn_forward_noalloc", "fork_attn_forward_qk8",
           "gdn_fork_workspace", "gdn_fork_forward", "gdn_fork_forward_fp8", "fork_rope_forward", "fork_rope_copy_forward", "fork_conv_forward",
           "fork_gate_forward", "gdn_inputs_forward", "gdn_conv_inputs_forward", "fork_linear_forward",
           "fork_quantize_fp8", "fork_linear_fp8_forward", "fork_option_readout",
           "fork_graph_create", "fork_graph_launch",
           "fork_graph_destroy", "fork_last_error", "fork_version")


class ForkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class fork_caps(ctypes.Structure):
    _fields_ = [("t_cap", ctypes.c_int32), ("s_cap", ctypes.c_int32),
                ("depth_cap", ctypes.c_int32), ("gqa_group", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("ctx_cap", ctypes.c_int32)]


class fork_meta(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_segments", ctypes.c_int32),
                ("num_roots", ctypes.c_int32), ("max_depth", ctypes.c_int32),
                ("num_attn_tiles", ctypes.c_int32), ("num_chunks", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("num_attn_merges", ctypes.c_int32),
                ("caps", fork_caps), ("dev", ctypes.c_void_p), ("dev_bytes", ctypes.c_size_t),
                ("level_segs", ctypes.c_int32 * 32), ("level_long", ctypes.c_int32 * 32),
                ("num_attn_parts", ctypes.c_int32)]


class fork_graph_args(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("scale", ctypes.c_float), ("attn_ws", ctypes.c_void_p),
                ("attn_ws_bytes", ctypes.c_size_t),
                ("gq", ctypes.c_void_p), ("gk", ctypes.c_void_p), ("gv", ctypes.c_void_p),
                ("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("root_state", ctypes.c_void_p),
                ("go", ctypes.c_void_p), ("seg_start_state", ctypes.c_void_p),
                ("seg_final_state", ctypes.c_void_p),
                ("gH", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("gscale", ctypes.c_float), ("gdn_ws", ctypes.c_void_p),
                ("gdn_ws_bytes", ctypes.c_size_t), ("dt", ctypes.c_int32),
                ("kc", ctypes.c_void_p), ("vc", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libforkattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tree_structured_decision_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        P = ctypes.POINTER
        sig = {
            "fork_meta_size": [P(fork_caps), P(sz), P(sz)],
            "fork_meta_build": [vp, vp, i32, P(fork_caps), vp, sz, vp, sz, P(fork_meta), vp],
            "fork_meta_plan": [vp, vp, i32, P(fork_caps), vp, sz, P(sz), P(fork_meta)],
            "fork_meta_build_ctx": [vp, vp, vp, vp, i32, P(fork_caps), vp, sz, vp, sz,
                                    P(fork_meta), vp],
            "fork_meta_plan_ctx": [vp, vp, vp, vp, i32, P(fork_caps), vp, sz, P(sz), P(fork_meta)],
            "fork_meta_export": [P(fork_meta), i32, vp, vp],
            "fork_meta_dense_mask": [P(fork_meta), vp, vp],
            "fork_meta_check": [P(fork_meta), P(i32), vp],
            "fork_attn_workspace": [P(fork_meta), i32, i32, i32, i32, P(sz)],
            "fork_attn_forward": [P(fork_meta), vp, vp, vp, vp, vp, i32, i32, i32, f32, i32,
                                  vp, sz, vp],
            "fork_attn_forward_ctx": [P(fork_meta), vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                      f32, i32, vp, sz, vp],
            "fork_attn_forward_noalloc": [P(fork_meta), vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, i32, vp],
            "fork_attn_forward_qk8": [P(fork_meta), vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, vp, sz, vp],
            "gdn_fork_workspace": [P(fork_meta), i32, i32, i32, i32, P(sz)],
            "gdn_fork_forward": [P(fork_meta), vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                 f32, i32, vp, sz, vp],
            "gdn_fork_forward_fp8": [P(fork_meta), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                     f32, vp],
            "fork_rope_forward": [P(fork_meta), vp, i32, i32, f32, i32, vp],
            "fork_rope_copy_forward": [P(fork_meta), vp, ctypes.c_int64, vp, i32, i32, f32, i32, vp],
            "fork_conv_forward": [P(fork_meta), vp, vp, vp, vp, vp, i32, i32, i32, i32, vp],
            "fork_gate_forward": [P(fork_meta), vp, vp, ctypes.c_int64, vp, vp, i32, i32, i32, f32, i32, vp],
            "gdn_inputs_forward": [P(fork_meta), vp, vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                   f32, i32, vp],
            "gdn_conv_inputs_forward": [P(fork_meta), vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                        i32, vp],
            "fork_linear_forward": [vp, vp, vp, i32, i32, i32, i32, i32, vp],
            "fork_quantize_fp8": [vp, vp, vp, ctypes.c_int64, i32, i32, vp],
            "fork_linear_fp8_forward": [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp],
            "fork_option_readout": [P(fork_meta), vp, vp, i32, vp, vp, i32, vp],
            "fork_graph_create": [P(fork_meta), P(fork_graph_args), vp, P(vp)],
            "fork_graph_launch": [vp, vp],
            "fork_graph_destroy": [vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.fork_last_error.restype = ctypes.c_char_p
        L.fork_last_error.argtypes = []
        L.fork_version.restype = ctypes.c_char_p
        L.fork_version.argtypes = []
        _lib = L
    return _lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        assert x.is_contiguous(), "tensors must be contiguous"
        return x.data_ptr()
    if hasattr(x, "ctypes"):  # numpy array
        return x.ctypes.data
    raise TypeError(f"cannot take a pointer of {type(x)}")


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _nbytes(x) -> int:
    if x is None or isinstance(x, int):
        return 0
    if hasattr(x, "numel"):
        return x.numel() * x.element_size()
    return int(x.nbytes)


def _check(status: int) -> None:
    if status != 0:
        raise ForkError(status, lib().fork_last_error().decode())


def fork_last_error() -> str:
    return lib().fork_last_error().decode()


def fork_version() -> str:
    return lib().fork_version().decode()


def make_caps(t_cap: int, s_cap: int, depth_cap: int, gqa_group: int, kv_heads: int = 0,
              ctx_cap: int = 0) -> fork_caps:
    return fork_caps(int(t_cap), int(s_cap), int(depth_cap), int(gqa_group), int(kv_heads),
                     int(ctx_cap))


def fork_meta_size(caps: fork_caps):
    dev, stg = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().fork_meta_size(ctypes.byref(caps), ctypes.byref(dev), ctypes.byref(stg)))
    return dev.value, stg.value


def fork_meta_plan(parent, seg_len, caps: fork_caps, staging):
    """parent/seg_len: int32 numpy arrays; staging: host buffer (numpy/torch)."""
    out = fork_meta()
    up = ctypes.c_size_t(0)
    _check(lib().fork_meta_plan(_ptr(parent), _ptr(seg_len), len(parent), ctypes.byref(caps),
                                _ptr(staging), _nbytes(staging), ctypes.byref(up),
                                ctypes.byref(out)))
    return out, up.value


def fork_meta_build(parent, seg_len, caps: fork_caps, dev, staging, stream=None) -> fork_meta:
    out = fork_meta()
    _check(lib().fork_meta_build(_ptr(parent), _ptr(seg_len), len(parent), ctypes.byref(caps),
                                 _ptr(dev), _nbytes(dev), _ptr(staging), _nbytes(staging),
                                 ctypes.byref(out), _stream(stream)))
    return out


def fork_meta_plan_ctx(parent, seg_len, ctx_start, ctx_len, caps: fork_caps, staging):
    """As fork_meta_plan, with resumed contexts (int32 arrays or None)."""
    out = fork_meta()
    up = ctypes.c_size_t(0)
    _check(lib().fork_meta_plan_ctx(_ptr(parent), _ptr(seg_len), _ptr(ctx_start), _ptr(ctx_len),
                                    len(parent), ctypes.byref(caps), _ptr(staging),
                                    _nbytes(staging), ctypes.byref(up), ctypes.byref(out)))
    return out, up.value


def fork_meta_build_ctx(parent, seg_len, ctx_start, ctx_len, caps: fork_caps, dev, staging,
                        stream=None) -> fork_meta:
    out = fork_meta()
    _check(lib().fork_meta_build_ctx(_ptr(parent), _ptr(seg_len), _ptr(ctx_start), _ptr(ctx_len),
                                     len(parent), ctypes.byref(caps), _ptr(dev), _nbytes(dev),
                                     _ptr(staging), _nbytes(staging), ctypes.byref(out),
                                     _stream(stream)))
    return out


def fork_meta_export(meta: fork_meta, array_id: int, dst, stream=None) -> None:
    _check(lib().fork_meta_export(ctypes.byref(meta), int(array_id), _ptr(dst), _stream(stream)))


def fork_meta_check(meta: fork_meta, stream=None, raise_on_error: bool = True) -> int:
    """The blob's device error word (FORK_DEVERR_* bits); raises ForkError
    (FORK_E_DEVICE) when it is nonzero, unless raise_on_error is False."""
    word = ctypes.c_int32(0)
    st = lib().fork_meta_check(ctypes.byref(meta), ctypes.byref(word), _stream(stream))
    if st != 0 and (raise_on_error or st != -7):
        _check(st)
    return int(word.value)


def fork_meta_dense_mask(meta: fork_meta, mask, stream=None) -> None:
    _check(lib().fork_meta_dense_mask(ctypes.byref(meta), _ptr(mask), _stream(stream)))


def fork_attn_workspace(meta: fork_meta, H: int, Hkv: int, D: int, dt: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().fork_attn_workspace(ctypes.byref(meta), H, Hkv, D, dt, ctypes.byref(n)))
    return n.value


def fork_attn_forward(meta: fork_meta, q, k, v, o, lse, H: int, Hkv: int, D: int, scale: float,
                      dt: int, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(lib().fork_attn_forward(ctypes.byref(meta), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(lse), H, Hkv, D, float(scale), dt, _ptr(ws),
                                   int(ws_bytes), _stream(stream)))


def fork_attn_forward_ctx(meta: fork_meta, q, k, v, kc, vc, o, lse, H: int, Hkv: int, D: int,
                          scale: float, dt: int, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(lib().fork_attn_forward_ctx(ctypes.byref(meta), _ptr(q), _ptr(k), _ptr(v), _ptr(kc),
                                       _ptr(vc), _ptr(o), _ptr(lse), H, Hkv, D, float(scale), dt,
                                       _ptr(ws), int(ws_bytes), _stream(stream)))


def fork_attn_forward_noalloc(meta: fork_meta, q, k, v, kc, vc, o, lse, H: int, Hkv: int, D: int,
                              scale: float, dt: int, stream=None) -> None:
    _check(lib().fork_attn_forward_noalloc(ctypes.byref(meta), _ptr(q), _ptr(k), _ptr(v), _ptr(kc),
                                           _ptr(vc), _ptr(o), _ptr(lse), H, Hkv, D, float(scale), dt,
                                           _stream(stream)))


def fork_attn_forward_qk8(meta: fork_meta, q8, q_scale, k8, k_scale, v, o, lse, H: int, Hkv: int, D: int,
                          scale: float, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(lib().fork_attn_forward_qk8(ctypes.byref(meta), _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v),
                                       _ptr(o), _ptr(lse), H, Hkv, D, float(scale), _ptr(ws), int(ws_bytes),
                                       _stream(stream)))


def gdn_fork_workspace(meta: fork_meta, H: int, dk: int, dv: int, dt: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_fork_workspace(ctypes.byref(meta), H, dk, dv, dt, ctypes.byref(n)))
    return n.value


def gdn_fork_forward(meta: fork_meta, q, k, v, a, b, root_state, o, seg_start_state,
                     seg_final_state, H: int, dk: int, dv: int, scale: float, dt: int, ws,
                     ws_bytes: int, stream=None) -> None:
    _check(lib().gdn_fork_forward(ctypes.byref(meta), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                  _ptr(root_state), _ptr(o), _ptr(seg_start_state),
                                  _ptr(seg_final_state), H, dk, dv, float(scale), dt, _ptr(ws),
                                  int(ws_bytes), _stream(stream)))


def gdn_fork_forward_fp8(meta: fork_meta, q8, q_scale, k8, k_scale, v8, v_scale, a, b, root_state, o,
                         seg_start_state, seg_final_state, H: int, dk: int, dv: int, scale: float,
                         stream=None) -> None:
    _check(lib().gdn_fork_forward_fp8(ctypes.byref(meta), _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale),
                                      _ptr(v8), _ptr(v_scale), _ptr(a), _ptr(b), _ptr(root_state), _ptr(o),
                                      _ptr(seg_start_state), _ptr(seg_final_state), H, dk, dv, float(scale),
                                      _stream(stream)))


def fork_rope_forward(meta: fork_meta, x, nheads: int, D: int, theta: float, dt: int,
                      stream=None) -> None:
    _check(lib().fork_rope_forward(ctypes.byref(meta), _ptr(x), nheads, D, float(theta), dt,
                                   _stream(stream)))


def fork_rope_copy_forward(meta: fork_meta, src, ld_src: int, dst, nheads: int, D: int, theta: float, dt: int,
                           stream=None) -> None:
    _check(lib().fork_rope_copy_forward(ctypes.byref(meta), _ptr(src), ld_src, _ptr(dst), nheads, D,
                                        float(theta), dt, _stream(stream)))


def fork_conv_forward(meta: fork_meta, x, w, bias, conv_state, y, C: int, K: int, act: int, dt: int,
                      stream=None) -> None:
    _check(lib().fork_conv_forward(ctypes.byref(meta), _ptr(x), _ptr(w), _ptr(bias),
                                   _ptr(conv_state), _ptr(y), C, K, act, dt, _stream(stream)))


def fork_gate_forward(meta: fork_meta, x, g, w, y, nheads: int, D: int, mode: int, eps: float,
                      dt: int, stream=None, ld_g: int = 0) -> None:
    _check(lib().fork_gate_forward(ctypes.byref(meta), _ptr(x), _ptr(g), ld_g, _ptr(w), _ptr(y), nheads, D,
                                   mode, float(eps), dt, _stream(stream)))


def fork_option_readout(meta: fork_meta, x, w, C: int, score, prob, dt: int, stream=None) -> None:
    _check(lib().fork_option_readout(ctypes.byref(meta), _ptr(x), _ptr(w), C, _ptr(score), _ptr(prob), dt,
                                     _stream(stream)))


def gdn_inputs_forward(meta: fork_meta, c, ab, a_log, dt_bias, q, k, v, a, b, H: int, dk: int,
                       dv: int, eps: float, dt: int, stream=None, ld_ab: int = 0) -> None:
    _check(lib().gdn_inputs_forward(ctypes.byref(meta), _ptr(c), _ptr(ab), ld_ab, _ptr(a_log),
                                    _ptr(dt_bias), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), H,
                                    dk, dv, float(eps), dt, _stream(stream)))


def gdn_conv_inputs_forward(meta: fork_meta, x, w, bias, conv_state, q, k, v, H: int, dk: int, dv: int,
                            K: int, eps: float, dt: int, stream=None) -> None:
    _check(lib().gdn_conv_inputs_forward(ctypes.byref(meta), _ptr(x), _ptr(w), _ptr(bias), _ptr(conv_state),
                                         _ptr(q), _ptr(k), _ptr(v), H, dk, dv, K, float(eps), dt,
                                         _stream(stream)))


def fork_linear_forward(x, w, y, M: int, N: int, K: int, accumulate: int, dt: int, stream=None) -> None:
    _check(lib().fork_linear_forward(_ptr(x), _ptr(w), _ptr(y), M, N, K, accumulate, dt, _stream(stream)))


def fork_quantize_fp8(x, q, scales, rows: int, K: int, dt: int, stream=None) -> None:
    _check(lib().fork_quantize_fp8(_ptr(x), _ptr(q), _ptr(scales), rows, K, dt, _stream(stream)))


def fork_linear_fp8_forward(xq, x_scale, wq, w_scale, y, M: int, N: int, K: int, accumulate: int,
                            stream=None) -> None:
    _check(lib().fork_linear_fp8_forward(_ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), _ptr(y), M, N, K,
                                         accumulate, _stream(stream)))


def fork_graph_create(meta: fork_meta, args: fork_graph_args, stream=None) -> int:
    g = ctypes.c_void_p(0)
    _check(lib().fork_graph_create(ctypes.byref(meta), ctypes.byref(args), _stream(stream),
                                   ctypes.byref(g)))
    return g.value


def fork_graph_launch(graph: int, stream=None) -> None:
    _check(lib().fork_graph_launch(graph, _stream(stream)))


def fork_graph_destroy(graph: int) -> None:
    _check(lib().fork_graph_destroy(graph))
