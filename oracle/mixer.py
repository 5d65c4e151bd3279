"""Oracle of the two token mixers of a hybrid block on the flattened stream.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite, the
smoke check and the benchmark's CPU-baseline leg are its only callers.

The pages describe the attention and Gated DeltaNet layers and the exactness
of forking (kongchang.com page, section "ForkAttention: exact forking in GPU
indices"; techfi24.com page, "Exact State Forking"), not the block around
them. The forms here follow the published Gated DeltaNet layer (Yang, Kautz,
Hatamizadeh, "Gated Delta Networks", 2024: short causal convolution with
SiLU, L2-normalised query and key, decay exp(-exp(a_log) softplus(.)),
sigmoid write strength, gated RMS norm at the output) and sigmoid output
gating of attention:

  attention mixer:  q, k, v, g = x Wq^T, x Wk^T, x Wv^T, x Wg^T
                    q, k <- rotary(q), rotary(k) at the isolated positions
                    y = (attention(q, k, v) * sigmoid(g)) Wo^T
  GDN mixer:        c = silu(conv(x Wqkv^T)) along the isolated sequences
                    q, k = l2norm(c_q), l2norm(c_k);  v = c_v
                    alpha, beta = x Wab^T
                    a = exp(-exp(a_log) softplus(alpha + dt_bias)),  b = sigmoid(beta)
                    o = gated_deltanet(q, k, v, a, b), scale 1/sqrt(dk)
                    y = (rmsnorm(o) * w * silu(x Wz^T)) Wo^T

With ``fp8=True`` every projection takes E4M3 operands: its input (per token)
and its weight (per output channel) are quantised as ``quantize_fp8`` (row
scale = max|.| / 448, nearest-even codes, decided in fp32 as on the GPU) and
the product is taken on the decoded values.

A stack applies pre-norm residual layers, x <- x + mixer(rmsnorm(x) w_l),
then a final RMS norm; the residual add happens before the one rounding of
the sum, as in a product that accumulates into its output.

Per-token steps are numpy float64; the tree-dependent steps call the oracle's
rotary, convolution, attention and Gated DeltaNet (oracle.c). With
``bf16=True`` every stored intermediate is rounded to bf16 (nearest, ties to
even, from float64) at the points where the GPU path stores bf16 tensors.
"""
from __future__ import annotations

import numpy as np


def to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (8 significant bits, ties to
    even) directly, without passing through float32; float64 out."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                    # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)  # numpy rounds halves to even


def linear(x, w) -> np.ndarray:
    """y = x w^T (w stored [out, in])."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def sigmoid(x) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def softplus(x) -> np.ndarray:
    """log(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, np.asarray(x, np.float64))


def gate(x, g, w, mode: int, eps: float = 1e-6) -> np.ndarray:
    """Over the last axis (D): mode 0 x sigmoid(g); mode 1
    x / sqrt(mean(x^2) + eps) w silu(g); mode 2 x / sqrt(mean(x^2) + eps) w."""
    x = np.asarray(x, np.float64)
    if mode == 0:
        return x * sigmoid(g)
    r = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)
    if mode == 1:
        g = np.asarray(g, np.float64)
        r = r * g * sigmoid(g)
    return r


def gdn_inputs(c, ab, a_log, dt_bias, H: int, dk: int, dv: int, eps: float = 1e-6):
    """Split c [T, 2 H dk + H dv] into L2-normalised query and key heads and the
    value heads; decay and write strength from ab [T, 2 H]."""
    c = np.asarray(c, np.float64)
    ab = np.asarray(ab, np.float64)
    T = c.shape[0]
    cq = c[:, :H * dk].reshape(T, H, dk)
    ck = c[:, H * dk:2 * H * dk].reshape(T, H, dk)
    v = c[:, 2 * H * dk:].reshape(T, H, dv)
    q = cq / np.sqrt(np.sum(cq * cq, axis=-1, keepdims=True) + eps)
    k = ck / np.sqrt(np.sum(ck * ck, axis=-1, keepdims=True) + eps)
    a = np.exp(-np.exp(np.asarray(a_log, np.float64)) * softplus(ab[:, :H] + np.asarray(dt_bias, np.float64)))
    b = sigmoid(ab[:, H:])
    return q, k, v, a, b


def _f32(x):
    return np.ascontiguousarray(x, np.float32)


def _lin(x, w, fp8):
    """A projection; with fp8 both operands are quantised row-wise first."""
    if not fp8:
        return linear(x, w)
    qx, sx = quantize_fp8(x)
    qw, sw = quantize_fp8(w)
    return linear_fp8(qx, sx, qw, sw)


def _out(r, u, wo, residual, fp8=False):
    """Output projection, with the residual added before the one rounding of the sum."""
    y = _lin(u, wo, fp8)
    return r(y if residual is None else np.asarray(residual, np.float64) + y)


def attention_mixer(parent, seg_len, x, W: dict, theta: float = 10000.0, bf16: bool = False,
                    residual=None, prec: str = "f64", fp8: bool = False, return_u: bool = False):
    """y [T, dm] of the attention mixer (weights as workloads.mixer_weights()['attn']);
    with residual, residual + y. prec: precision of the attention oracle. fp8:
    every projection takes E4M3 operands (input per token and weight per
    output channel, quantised as quantize_fp8). return_u: also the output
    projection's input u [T, H D]."""
    from . import attention, rope
    r = to_bf16 if bf16 else (lambda t: t)
    T = x.shape[0]
    H, Hkv, D = W["H"], W["Hkv"], W["D"]
    q = r(_lin(x, W["wq"], fp8)).reshape(T, H, D)
    k = r(_lin(x, W["wk"], fp8)).reshape(T, Hkv, D)
    v = r(_lin(x, W["wv"], fp8)).reshape(T, Hkv, D)
    g = r(_lin(x, W["wg"], fp8)).reshape(T, H, D)
    q = r(rope(parent, seg_len, _f32(q), theta=theta))
    k = r(rope(parent, seg_len, _f32(k), theta=theta))
    o, _ = attention(parent, seg_len, _f32(q), _f32(k), _f32(v), prec=prec)
    u = r(gate(r(o), g, None, 0))
    y = _out(r, u.reshape(T, H * D), W["wo"], residual, fp8)
    return (y, u.reshape(T, H * D)) if return_u else y


def gdn_mixer(parent, seg_len, x, W: dict, eps: float = 1e-6, bf16: bool = False,
              return_state: bool = False, residual=None, prec: str = "f64", fp8: bool = False,
              return_u: bool = False):
    """y [T, dm] of the Gated DeltaNet mixer (weights as
    workloads.mixer_weights()['gdn']); with residual, residual + y; with
    return_state also the per-segment start and end states, with return_u
    the output projection's input u [T, H dv] instead. prec: precision of the
    Gated DeltaNet oracle. fp8: as attention_mixer."""
    from . import conv, gdn
    r = to_bf16 if bf16 else (lambda t: t)
    T = x.shape[0]
    H, dk, dv = W["H"], W["dk"], W["dv"]
    p = r(_lin(x, W["wqkv"], fp8))
    # the convolution's output is normalised and split before it is stored:
    # q, k and v are the stored (rounded) tensors
    c = conv(parent, seg_len, _f32(p), W["conv_w"], act=1)
    ab = r(_lin(x, W["wab"], fp8))
    q, k, v, a, b = gdn_inputs(c, ab, W["a_log"], W["dt_bias"], H, dk, dv, eps)
    o, st0, st1 = gdn(parent, seg_len, _f32(r(q)), _f32(r(k)), _f32(r(v)), _f32(a), _f32(b),
                      scale=1.0 / np.sqrt(dk), prec=prec)
    z = r(_lin(x, W["wz"], fp8)).reshape(T, H, dv)
    u = r(gate(r(o), z, W["norm_w"], 1, eps))
    y = _out(r, u.reshape(T, H * dv), W["wo"], residual, fp8)
    if return_u:
        return y, u.reshape(T, H * dv)
    return (y, st0, st1) if return_state else y


def stack(parent, seg_len, x, layers, final_norm, theta: float = 10000.0, eps: float = 1e-6,
          bf16: bool = False, prec: str = "f64", fp8: bool = False) -> np.ndarray:
    """A pre-norm residual stack of mixers on the flattened stream:
    x <- x + mixer(rmsnorm(x) w_l) for each layer, then h = rmsnorm(x) w_final.
    layers: list of (kind, weights, norm weight [dm]) with kind "attn" or "gdn"."""
    r = to_bf16 if bf16 else (lambda t: t)
    x = np.asarray(x, np.float64)
    for kind, W, nw in layers:
        hn = r(gate(x, None, nw, 2, eps))
        if kind == "attn":
            x = attention_mixer(parent, seg_len, hn, W, theta, bf16, residual=x, prec=prec, fp8=fp8)
        else:
            x = gdn_mixer(parent, seg_len, hn, W, eps, bf16, residual=x, prec=prec, fp8=fp8)
    return r(gate(x, None, final_norm, 2, eps))



# ---------------------------------------------------------------- FP8 E4M3
# OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
# field 0 holds subnormals m/8 * 2^-6; the largest finite value is
# 1.75 * 2^8 = 448 (code 0x7E; 0x7F is NaN, there are no infinities).

def e4m3_encode(t) -> np.ndarray:
    """Nearest-even E4M3 codes (uint8) of values with |t| <= 448."""
    t = np.asarray(t, np.float64)
    a = np.abs(t)
    assert (a <= 448.0).all()
    sign = (np.signbit(t)).astype(np.int64) << 7
    e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    normal = a >= 2.0 ** -6
    # normals: 3 fraction bits at exponent e; subnormals: steps of 2^-9
    m = np.where(normal, np.round((a / np.ldexp(1.0, e) - 1.0) * 8.0), np.round(a / 2.0 ** -9))
    m = m.astype(np.int64)
    ef = np.where(normal, e + 7, 0)
    up = normal & (m == 8)            # rounding carried into the next binade
    ef = np.where(up, ef + 1, ef)
    m = np.where(up, 0, m)
    sub_up = (~normal) & (m == 8)     # largest subnormal rounded up to 2^-6
    ef = np.where(sub_up, 1, ef)
    m = np.where(sub_up, 0, m)
    return (sign | (ef << 3) | m).astype(np.uint8)


def e4m3_decode(c) -> np.ndarray:
    """Values of E4M3 codes (NaN for 0x7F / 0xFF)."""
    c = np.asarray(c, np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    v = np.where(ef == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    v = np.where((ef == 15) & (m == 7), np.nan, v)
    return s * v


def quantize_fp8(x):
    """Row-wise quantisation (rows along the last axis), decided in fp32 as on
    the GPU: scale_r = fp32(max_k |x[r][k]|) / 448 (1 for an all-zero row),
    code = E4M3(clamp(fp32(x) / scale_r, -448, 448)) with correctly rounded
    fp32 divisions. Returns (codes uint8, scales float32 [rows])."""
    x32 = np.asarray(x, np.float32)
    amax = np.max(np.abs(x32), axis=-1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    t = np.clip(x32 / scale[..., None], np.float32(-448.0), np.float32(448.0))
    return e4m3_encode(t.astype(np.float64)), scale


def dequantize_fp8(codes, scale) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scale, np.float64)[..., None]


def linear_fp8(xq, x_scale, wq, w_scale) -> np.ndarray:
    """y[m][n] = (sum_k decode(xq[m][k]) decode(wq[n][k])) x_scale[m] w_scale[n]."""
    return (e4m3_decode(xq) @ e4m3_decode(wq).T) * np.outer(np.asarray(x_scale, np.float64),
                                                          np.asarray(w_scale, np.float64))
